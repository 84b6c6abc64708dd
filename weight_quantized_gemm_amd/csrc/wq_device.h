// Device-side helpers shared by the gfx950 kernels: vector types, storage conversions,
// exact integer-code -> fp16/bf16 images, MFMA and LDS transpose-read wrappers.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace wq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x16_t __attribute__((ext_vector_type(16)));
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
typedef int16_t i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define WQ_LDS __attribute__((address_space(3)))

// ----------------------------------------------------------------------------- storage
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
template <bool BF16>
__device__ __forceinline__ float act_to_f32(uint16_t v) {
  return BF16 ? bf16_bits_to_f32(v) : f16_bits_to_f32(v);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// fp32 -> fp16, the hardware conversion (round to nearest even).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
template <bool BF16>
__device__ __forceinline__ uint16_t f32_to_act(float f) {
  return BF16 ? f32_to_bf16_rne(f) : f32_to_f16_rne(f);
}

// ----------------------------------------------------------------------------- code images
// Weight storage formats (a kernel template parameter).
enum WFmt : int { kWInt8 = 0, kWInt4 = 1, kWFp8 = 2 };

// Every int8 and int4 weight code is exact in fp16 and in bf16.  The conversions below turn
// packed codes into 16-bit floating images, two per dword, in the byte order of the input
// (consecutive k after a tr8 transpose read).  bf16 images of int4 codes are biased by a
// constant C = 136 (the fed value is code + C); the kernels remove C exactly in fp32
// through the offset term.  All other images are the codes themselves.

// 4 int8 codes (one dword) -> two dwords of bf16 images.  The signed byte -> fp32
// conversion is one instruction (v_cvt_f32_i32 with a sign-extended byte operand), and an
// integer of magnitude <= 128 is exact in bf16, i.e. the top half of its fp32 pattern.
__device__ __forceinline__ void i8x4_to_bf16(uint32_t d, uint32_t& lo, uint32_t& hi) {
  const float f0 = (float)(int8_t)(d), f1 = (float)(int8_t)(d >> 8);
  const float f2 = (float)(int8_t)(d >> 16), f3 = (float)(int8_t)(d >> 24);
  lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

// 4 int8 codes -> fp16 images of the codes (exact).  0x64xx is 1024 + xx in fp16.
__device__ __forceinline__ void i8x4_to_f16(uint32_t d, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = d ^ 0x80808080u;                      // code + 128 in [0, 255]
  const uint32_t m = 0x64646464u;
  const uint32_t a = __builtin_amdgcn_perm(m, u, 0x04010400u);  // [u0, 0x64, u1, 0x64]
  const uint32_t b = __builtin_amdgcn_perm(m, u, 0x04030402u);  // [u2, 0x64, u3, 0x64]
  const f16x2_t k = {(_Float16)1152.0f, (_Float16)1152.0f};   // 1024 + 128
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) - k);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, b) - k);
}

// 8 int8 codes of one column, consecutive k (a tr8 read) -> an MFMA B fragment.
template <bool BF16>
__device__ __forceinline__ u32x4_t i8x8_to_act(u32x2_t d) {
  uint32_t o[4];
  if constexpr (BF16) {
    i8x4_to_bf16(d[0], o[0], o[1]);
    i8x4_to_bf16(d[1], o[2], o[3]);
  } else {
    i8x4_to_f16(d[0], o[0], o[1]);
    i8x4_to_f16(d[1], o[2], o[3]);
  }
  return u32x4_t{o[0], o[1], o[2], o[3]};
}

// 8 FLOAT8_E4M3FN codes of one column, consecutive k -> an MFMA B fragment.  E4M3FN
// values have 3 mantissa bits and magnitudes from 2^-9 to 448, so each is exact in bf16 and
// in fp16; gfx950 converts two codes (one half of a dword) per instruction, here with a unit
// scale, which leaves the values unchanged.
template <bool BF16>
__device__ __forceinline__ u32x4_t f8x8_to_act(u32x2_t d) {
  uint32_t o[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (BF16) {
      o[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[h], 1.0f, false));
      o[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[h], 1.0f, true));
    } else {
      o[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d[h], 1.0f, false));
      o[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d[h], 1.0f, true));
    }
  }
  return u32x4_t{o[0], o[1], o[2], o[3]};
}

// 8 one-byte codes (int8 or FLOAT8_E4M3FN) of one column -> an MFMA B fragment.
template <bool BF16, int WF>
__device__ __forceinline__ u32x4_t w8x8_to_act(u32x2_t d) {
  if constexpr (WF == kWFp8) return f8x8_to_act<BF16>(d);
  else return i8x8_to_act<BF16>(d);
}

// 8 bytes of packed int4 (two adjacent columns, consecutive k: a tr8 read of a packed
// tile) -> the MFMA B fragments of the even column and of the odd column.
// bf16: 0x43 0x0n is 128 + n, so the image is code + 136; fp16: 0x64 0x0n is 1024 + n,
// and subtracting 1032 leaves the code.
template <bool BF16>
__device__ __forceinline__ void i4_kpairs(u32x2_t d, u32x4_t& even, u32x4_t& odd) {
  const uint32_t mag = BF16 ? 0x43434343u : 0x64646464u;
  uint32_t ev[4], od[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t u = d[h] ^ 0x88888888u;             // nibble -> code + 8 in [0, 15]
    const uint32_t e = u & 0x0f0f0f0fu, o = (u >> 4) & 0x0f0f0f0fu;
    ev[2 * h] = __builtin_amdgcn_perm(mag, e, 0x04010400u);      // [e0, M, e1, M]
    ev[2 * h + 1] = __builtin_amdgcn_perm(mag, e, 0x04030402u);  // [e2, M, e3, M]
    od[2 * h] = __builtin_amdgcn_perm(mag, o, 0x04010400u);
    od[2 * h + 1] = __builtin_amdgcn_perm(mag, o, 0x04030402u);
  }
  if constexpr (!BF16) {
    const f16x2_t k = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ev[q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, ev[q]) - k);
      od[q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, od[q]) - k);
    }
  }
  even = u32x4_t{ev[0], ev[1], ev[2], ev[3]};
  odd = u32x4_t{od[0], od[1], od[2], od[3]};
}

// 4 bytes of int4 codes packed along k (8 consecutive k of one column, the even k in the low
// nibble: a transposed int4 weight) -> an MFMA B fragment, images in k order.  Same images
// as i4_kpairs: bf16 code + 136, fp16 the code.
template <bool BF16>
__device__ __forceinline__ u32x4_t i4x8_k_to_act(uint32_t d) {
  const uint32_t mag = BF16 ? 0x43434343u : 0x64646464u;
  const uint32_t u = d ^ 0x88888888u;                 // nibble -> code + 8 in [0, 15]
  const uint32_t e = u & 0x0f0f0f0fu, o = (u >> 4) & 0x0f0f0f0fu;   // even k, odd k
  const uint32_t t0 = __builtin_amdgcn_perm(o, e, 0x05010400u);    // [k0, k1, k2, k3]
  const uint32_t t1 = __builtin_amdgcn_perm(o, e, 0x07030602u);    // [k4, k5, k6, k7]
  uint32_t w[4] = {__builtin_amdgcn_perm(mag, t0, 0x04010400u), __builtin_amdgcn_perm(mag, t0, 0x04030402u),
                   __builtin_amdgcn_perm(mag, t1, 0x04010400u), __builtin_amdgcn_perm(mag, t1, 0x04030402u)};
  if constexpr (!BF16) {
    const f16x2_t k = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, w[q]) - k);
  }
  return u32x4_t{w[0], w[1], w[2], w[3]};
}

// row sums: a * 1 + b * 1 + c for a dword of two 16-bit activations
template <bool BF16>
__device__ __forceinline__ float dot2_ones(uint32_t v, float c) {
  if constexpr (BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v),
                                           __builtin_bit_cast(bf16x2_t, 0x3f803f80u), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, v),
                                  __builtin_bit_cast(f16x2_t, 0x3c003c00u), c, false);
}

// ----------------------------------------------------------------------------- LDS DMA
// Buffer resource (4 dwords, kept in SGPRs): base, stride 0, num_records bytes.  Accesses
// at or past num_records read zero, so it doubles as the bounds check of every tile load.
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  const uint64_t b = (uint64_t)base;
  return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu)),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)n), 0x00020000u};
}
// The same with a range the caller has already bounded (bytes <= 0x7fffffff): no clamp.
__device__ __forceinline__ u32x4_t make_rsrc32(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu)),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
}
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every resource: the load reads 0

// One 16-byte-per-lane direct-to-LDS load: lane l's 16 bytes land at lds_block + 16*l.
// Written as a self-contained asm statement: it has no register result (the data goes to
// LDS), and the caller accounts for it with an explicit vmcnt wait before the barrier that
// publishes the stage.  M0 carries the LDS base (saved and restored around the load, as
// the compiler owns M0); one wait state separates the M0 write from the load.
__device__ __forceinline__ void dma16(const u32x4_t& rsrc, const void* lds_block, uint32_t voff) {
  const uint32_t lds = (uint32_t)(uintptr_t)(WQ_LDS const void*)lds_block;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds)), "v"(voff), "s"(rsrc)
      : "memory");
}


// ----------------------------------------------------------------------------- MFMA
template <bool BF16>
__device__ __forceinline__ f32x16_t mfma32x32x16(const u32x4_t& a, const u32x4_t& b,
                                                 const f32x16_t& c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ i32x16_t mfma32x32x32_i8(const u32x4_t& a, const u32x4_t& b,
                                                    const i32x16_t& c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_t, a),
                                               __builtin_bit_cast(i32x4_t, b), c, 0, 0, 0);
}

// ----------------------------------------------------------------------------- LDS reads
// gfx950 transpose read: within each group of 16 lanes, slot j of lane L is byte (L % 8) of
// the 8 bytes addressed by lane 2*j + L/8.  With a row-major (n-contiguous) tile, lanes
// addressing (row k0 + j, 8 columns) give every lane one column and consecutive k -- the
// MFMA B-operand layout.
__device__ __forceinline__ u32x2_t lds_read_tr8(const uint8_t* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr8_b64_v2i32((WQ_LDS i32x2_t*)(p)));
}

// Accumulator layout of a 32x32 MFMA block: element r of lane l sits at
// row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

}  // namespace wq

// Device-side helpers shared by the gfx950 kernels: vector types, storage conversions,
// exact integer-code -> fp16/bf16 images, MFMA and LDS transpose-read wrappers.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace wq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
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
// Every int8 and int4 weight code is exact in fp16 and in bf16.  The conversions below turn
// packed codes into 16-bit floating images, two per dword, in column order along n.
// The bf16 images are biased by a constant C (the fed value is code + C); the kernels
// remove C exactly in fp32 through the offset term.  fp16 images are the codes themselves.

// 4 int8 codes (one dword, columns c..c+3) -> bf16 images of code + 128.
__device__ __forceinline__ void i8x4_to_bf16(uint32_t d, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = d ^ 0x80808080u;  // two's complement -> code + 128 in [0, 255]
  const float f0 = (float)(u & 0xffu), f1 = (float)((u >> 8) & 0xffu);
  const float f2 = (float)((u >> 16) & 0xffu), f3 = (float)(u >> 24);
  // an integer below 256 is exact in bf16, i.e. the top half of its fp32 pattern
  lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}
constexpr float kBf16Int8Bias = 128.0f;

// 4 int8 codes -> fp16 images of the codes (exact).  0x64xx is 1024 + xx in fp16.
__device__ __forceinline__ void i8x4_to_f16(uint32_t d, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = d ^ 0x80808080u;
  const uint32_t m = 0x64646464u;
  uint32_t a = __builtin_amdgcn_perm(m, u, 0x04010400u);  // [u0, 0x64, u1, 0x64]
  uint32_t b = __builtin_amdgcn_perm(m, u, 0x04030402u);  // [u2, 0x64, u3, 0x64]
  const f16x2_t k = {(_Float16)1152.0f, (_Float16)1152.0f};  // 1024 + 128
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) - k);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, b) - k);
}

// 8 int4 codes (one dword, columns c..c+7, even column in the low nibble) -> 4 dwords of
// 16-bit images.  bf16: 0x43xx is 128 + xx, so the image is code + 136.  fp16: the code.
template <bool BF16>
__device__ __forceinline__ void i4x8_to_act(uint32_t d, uint32_t out[4]) {
  const uint32_t u = d ^ 0x88888888u;          // nibble -> code + 8 in [0, 15]
  const uint32_t e = u & 0x0f0f0f0fu;          // columns c, c+2, c+4, c+6
  const uint32_t o = (u >> 4) & 0x0f0f0f0fu;   // columns c+1, c+3, c+5, c+7
  const uint32_t mag = BF16 ? 0x43004300u : 0x64006400u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sel = 0x0c000c00u | ((uint32_t)(4 + j) << 16) | (uint32_t)j;
    out[j] = __builtin_amdgcn_perm(o, e, sel) | mag;   // [e_j, 0, o_j, 0] | magic
  }
  if (!BF16) {
    const f16x2_t k = {(_Float16)1032.0f, (_Float16)1032.0f};  // 1024 + 8
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, out[j]) - k);
  }
}
constexpr float kBf16Int4Bias = 136.0f;

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
// gfx950 transpose reads.  Within each group of 16 lanes:
//  * tr16: slot j of lane L is 16-bit element (L % 4) of the 8 bytes addressed by lane
//    4*j + L/4;
//  * tr8:  slot j of lane L is byte (L % 8) of the 8 bytes addressed by lane 2*j + L/8.
// With a row-major (n-contiguous) tile, lanes addressing (row k0 + j, 4 or 8 columns) give
// every lane one column and consecutive k -- the MFMA B-operand layout.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((WQ_LDS i16x4_t*)(p)));
}
__device__ __forceinline__ u32x2_t lds_read_tr8(const uint8_t* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr8_b64_v2i32((WQ_LDS i32x2_t*)(p)));
}

// Accumulator layout of a 32x32 MFMA block: element r of lane l sits at
// row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

}  // namespace wq

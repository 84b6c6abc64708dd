// Small passes around the anti-quant matmul:
//  * the empty-K case, out = bias + x3 ("CANN ops-transformer ... aclnnWeightQuantMatmulAllReduce
//    完全指南", section 空 tensor 支持度 (empty tensors));
//  * per-group scale and offset stored transposed with a transposed x2 (section 参数说明):
//    copied to the row-major (groups, n) layout the GEMM kernels read, in the workspace;
//  * per-group row sums of x1, S_g[r] = sum of x1[r, k] over the k of group g, which the
//    factored product's offset term needs (read after the k loop, see aq_gemm.h);
//  * the offline weight prepack (wq_prepack_weight): x2 into the packed layout of 64 k x 32
//    column blocks in MFMA B-fragment order (the layout is described in wqgemm.h).
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

// out = bias + x3 (either may be absent); one 16-bit element per thread, grid-stride.
template <bool BF16>
__global__ __launch_bounds__(256) void bias_x3_kernel(const AqArgs a) {
  const uint16_t* __restrict__ bias = (const uint16_t*)a.bias;
  const uint16_t* __restrict__ x3 = (const uint16_t*)a.x3;
  uint16_t* __restrict__ out = (uint16_t*)a.out;
  const int n = a.n;
  const int64_t total = a.m * n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v = 0.f;
    if (bias) v += act_to_f32<BF16>(bias[i % n]);
    if (x3) v += act_to_f32<BF16>(x3[i]);
    out[i] = f32_to_act<BF16>(v);
  }
}

// dst (rows, cols) = transpose of src (cols, rows), 16-bit elements, through a 64 x 64 LDS
// tile (rows = groups, cols = n): reads and writes move along the contiguous axis.  Grid z
// picks one of two tensors (scale, then offset), so both are copied by one launch.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* __restrict__ src0,
                                                          uint16_t* __restrict__ dst0,
                                                          const uint16_t* __restrict__ src1,
                                                          uint16_t* __restrict__ dst1, int rows, int cols) {
  const uint16_t* __restrict__ src = blockIdx.z ? src1 : src0;
  uint16_t* __restrict__ dst = blockIdx.z ? dst1 : dst0;
  __shared__ uint16_t tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {  // src row c0 + i, element r0 + tx
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) tile[i][tx] = src[(int64_t)c * rows + r];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {  // dst row r0 + i, element c0 + tx
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) dst[(int64_t)r * cols + c] = tile[tx][i];
  }
}

// S[g][r] = sum of x1[r, k] over group g's k, fp32, in a fixed order.  The work items are
// (row, chunk) pairs, a chunk being gpc whole groups (about 2048 k), so that short m still
// spreads over many waves.  A wave takes one item at a time: lane l sums x1[r, kb + 512 w +
// 8 l .. + 7] (v_dot2 against ones), four lanes add up a 32-k piece, and the chunk's pieces
// land in the wave's LDS strip; then lane j adds up the pieces of the chunk's group j in k
// order (groups are multiples of 32 long, k too).  Each lane keeps four 16-byte loads in
// flight: the chunk is read 2048 k at a time.
template <bool BF16>
__global__ __launch_bounds__(256) void group_rowsums_kernel(const uint16_t* __restrict__ x1,
                                                            float* __restrict__ S, int64_t m, int k,
                                                            int g, int groups, int gpc, int nchunks) {
  // each wave's strip holds one chunk's pieces (dynamic LDS: 4 strips of np floats)
  extern __shared__ float pieces[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = g / 32, np = gpc * per;
  float* piece = pieces + wave * np;
  const int64_t items = m * nchunks;
  for (int64_t it = (int64_t)blockIdx.x * 4 + wave; it < items; it += (int64_t)gridDim.x * 4) {
    const int64_t r = it / nchunks;
    const int c = (int)(it - r * nchunks);
    const int kb = c * gpc * g, ke = min(k, kb + gpc * g);
    const uint16_t* row = x1 + r * k;
    for (int w0 = kb; w0 < ke; w0 += 2048) {
      u32x4_t d[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = w0 + 512 * u + 8 * lane;
        d[u] = kk < ke ? *(const u32x4_t*)(row + kk) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = w0 + 512 * u + 8 * lane;
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) v = dot2_ones<BF16>(d[u][q], v);
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        if ((lane & 3) == 0 && kk < ke) piece[(kk - kb) / 32] = v;
      }
    }
    __builtin_amdgcn_wave_barrier();  // the strip is written (one wave: LDS in order)
    const int nloc = (ke - kb) / 32;  // pieces in this chunk
    for (int j = lane; j < gpc; j += 64) {
      const int gi = c * gpc + j;
      if (gi >= groups) break;
      const int p1 = min(nloc, (j + 1) * per);
      float t = 0.f;
      for (int p = j * per; p < p1; ++p) t += piece[p];
      S[(int64_t)gi * m + r] = t;
    }
    __builtin_amdgcn_wave_barrier();  // read before the next item overwrites it
  }
}

// One 2048-byte unit of the packed layout per workgroup (grid x: unit along n, y: k block):
// a 64 k x 32 column block of one-byte codes, or two adjacent such blocks of int4 codes.  The
// codes are gathered into LDS as one byte each (int4: the nibble's value), then written in
// fragment order: for 16-k step s and lane l, the codes of column l % 32 at k
// 16 s + 8 (l / 32) + 0 .. 7, one byte per k (int4: the unit's first block in bits 0-3, its
// second in bits 4-7).  Codes past k are zero.
template <bool W4, bool XT>
__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t* __restrict__ x2, uint8_t* __restrict__ packed,
                                                      int K, int N) {
  constexpr int kCols = W4 ? 64 : 32;   // columns of a unit
  __shared__ uint8_t tile[64][kCols + 1];  // [k][column], padded
  const int t = threadIdx.x;
  const int nb = blockIdx.x, kb = blockIdx.y;
  const int n0 = nb * kCols, k0 = kb * 64;
  typedef uint8_t u8x16 __attribute__((ext_vector_type(16)));
  if constexpr (!W4 && !XT) {         // rows of k: 32 bytes of the block per row
    if (t < 128) {
      const int r = t >> 1, h = t & 1;
      u8x16 v = {};
      if (k0 + r < K) v = *(const u8x16*)(x2 + (int64_t)(k0 + r) * N + n0 + 16 * h);
#pragma unroll
      for (int e = 0; e < 16; ++e) tile[r][16 * h + e] = v[e];
    }
  } else if constexpr (!W4) {         // rows of columns: 64 bytes of k per column
    if (t < 128) {
      const int c = t >> 2, q = t & 3;
      u8x16 v = {};
      if (k0 + 16 * q < K) v = *(const u8x16*)(x2 + (int64_t)(n0 + c) * K + k0 + 16 * q);
#pragma unroll
      for (int e = 0; e < 16; ++e) tile[16 * q + e][c] = v[e];
    }
  } else if constexpr (!XT) {         // int4 rows of k: 32 bytes (64 columns) per row
    if (t < 128) {
      const int r = t >> 1, h = t & 1;
      u8x16 v = {};
      if (k0 + r < K) v = *(const u8x16*)(x2 + (int64_t)(k0 + r) * (N / 2) + n0 / 2 + 16 * h);
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        tile[r][32 * h + 2 * b] = v[b] & 15;
        tile[r][32 * h + 2 * b + 1] = v[b] >> 4;
      }
    }
  } else {                            // int4 rows of columns: 32 bytes (64 k) per column
    if (t < 128) {
      const int c = t >> 1, h = t & 1;
      u8x16 v = {};
      if (k0 + 32 * h < K) v = *(const u8x16*)(x2 + (int64_t)(n0 + c) * (K / 2) + k0 / 2 + 16 * h);
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        tile[32 * h + 2 * b][c] = v[b] & 15;
        tile[32 * h + 2 * b + 1][c] = v[b] >> 4;
      }
    }
  }
  __syncthreads();
  const int s = t >> 6, l = t & 63;           // 16-k step and lane of this thread's codes
  const int c = l & 31, kr = 16 * s + 8 * (l >> 5);
  const int64_t unit = (int64_t)kb * (N / kCols) + nb;
  // the byte of k kr + e: the code of column c, and with int4 that of column c + 32 on top
  auto code = [&](int e) -> uint32_t {
    if constexpr (W4) return (uint32_t)(tile[kr + e][c] & 15) | ((uint32_t)(tile[kr + e][32 + c] & 15) << 4);
    else return tile[kr + e][c];
  };
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo |= code(e) << (8 * e);
    hi |= code(4 + e) << (8 * e);
  }
  *(u32x2_t*)(packed + unit * 2048 + 8 * t) = u32x2_t{lo, hi};
}

}  // namespace

hipError_t launch_prepack(const PrepackProblem& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.n / (p.w4 ? 64 : 32)), (unsigned)((p.k + 63) / 64));
  auto kern = p.w4 ? (p.x2t ? prepack_kernel<true, true> : prepack_kernel<true, false>)
                   : (p.x2t ? prepack_kernel<false, true> : prepack_kernel<false, false>);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, (const uint8_t*)p.x2, (uint8_t*)p.packed, (int)p.k,
                     (int)p.n);
  return hipGetLastError();
}

hipError_t launch_group_rowsums(const AqArgs& a, hipStream_t stream) {
  // chunks of gpc whole groups, about 2048 k (one group when groups are longer)
  const int gpc = std::max(1, 2048 / a.group);
  const int nchunks = (a.groups + gpc - 1) / gpc;
  const int64_t items = a.m * nchunks;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((items + 3) / 4, 16384));
  // 4 strips of a chunk's pieces: <= 4 x 2047 floats (a group is shorter than k <= 65535)
  const size_t lds = (size_t)4 * (size_t)(gpc * (a.group / 32)) * sizeof(float);
  if (a.bf16)
    hipLaunchKernelGGL(group_rowsums_kernel<true>, dim3((unsigned)blocks), dim3(256), lds, stream,
                       (const uint16_t*)a.x1, a.gsum, a.m, a.k, a.group, a.groups, gpc, nchunks);
  else
    hipLaunchKernelGGL(group_rowsums_kernel<false>, dim3((unsigned)blocks), dim3(256), lds, stream,
                       (const uint16_t*)a.x1, a.gsum, a.m, a.k, a.group, a.groups, gpc, nchunks);
  return hipGetLastError();
}

hipError_t launch_transpose16(const void* src0, void* dst0, const void* src1, void* dst1, int rows,
                              int cols, hipStream_t stream) {
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64), src1 ? 2u : 1u);
  hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, stream, (const uint16_t*)src0, (uint16_t*)dst0,
                     (const uint16_t*)src1, (uint16_t*)dst1, rows, cols);
  return hipGetLastError();
}

hipError_t launch_aq_bias_x3(const AqArgs& a, hipStream_t stream) {
  const int64_t total = a.m * a.n;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 65536));
  AqArgs args = a;
  return launch_main(a.bf16 ? (const void*)bias_x3_kernel<true> : (const void*)bias_x3_kernel<false>,
                     dim3((unsigned)blocks), dim3(256), 0, stream, &args);
}

}  // namespace wq

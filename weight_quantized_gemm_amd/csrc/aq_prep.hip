// Auxiliary anti-quant kernels for gfx950:
//  * row sums of x1 per quantisation group, S_g[m] = sum_{i in group g} x1[m, i], the
//    factor of the offset term in the factored form of the anti-quant matmul;
//  * the empty-K case, out = bias + x3 ("CANN ops-transformer ... aclnnWeightQuantMatmul
//    AllReduce 完全指南", section 空 tensor 支持度 (empty tensors)).
// Both are bandwidth-bound passes; every reduction runs in a fixed order (deterministic).
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

template <bool BF16>
__device__ __forceinline__ float sum8(const uint16_t* p) {
  const u32x4_t v = *(const u32x4_t*)p;
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s += act_to_f32<BF16>((uint16_t)(v[q] & 0xffffu));
    s += act_to_f32<BF16>((uint16_t)(v[q] >> 16));
  }
  return s;
}

// Sum over lanes whose index agrees outside the low log2(seg) bits (seg a power of two).
__device__ __forceinline__ float seg_reduce(float v, int seg) {
  for (int off = seg >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// One wave per row.  rs layout: [groups][mp], rows >= m written as 0.
//  * groups whose span is a multiple of 512 elements (and the single group of the
//    per-tensor / per-channel modes): lanes accumulate 8-element chunks over the group,
//    one 64-lane reduction per group;
//  * power-of-two group sizes below 512: each 512-element pass holds 512/g whole groups
//    of g/8 lanes each, reduced by a segmented butterfly;
//  * any other group size: one lane per group sums it serially.
template <bool BF16>
__global__ __launch_bounds__(256) void rowsum_kernel(const uint16_t* __restrict__ x1,
                                                     float* __restrict__ rs, int64_t m, int64_t mp,
                                                     int k, int g, int groups) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t row = wave_id; row < mp; row += nwaves) {
    if (row >= m) {
      for (int q = lane; q < groups; q += 64) rs[(int64_t)q * mp + row] = 0.f;
      continue;
    }
    const uint16_t* xr = x1 + row * k;
    if (groups == 1 || (g % 512) == 0) {
      float acc = 0.f;
      int grp = 0;
      for (int base = 0; base < k; base += 512) {
        const int kk = base + 8 * lane;
        if (kk < k) acc += sum8<BF16>(xr + kk);
        const int next = base + 512;
        const bool group_end = (groups == 1) ? (next >= k) : (next % g == 0 || next >= k);
        if (group_end) {
          const float s = seg_reduce(acc, 64);
          if (lane == 0) rs[(int64_t)grp * mp + row] = s;
          acc = 0.f;
          ++grp;
        }
      }
    } else if ((g & (g - 1)) == 0 && g < 512) {
      const int seg = g >> 3;  // lanes per group
      for (int base = 0; base < k; base += 512) {
        const int kk = base + 8 * lane;
        float v = kk < k ? sum8<BF16>(xr + kk) : 0.f;
        v = seg_reduce(v, seg);
        if (kk < k && (lane & (seg - 1)) == 0) rs[(int64_t)(kk / g) * mp + row] = v;
      }
    } else {
      for (int q = lane; q < groups; q += 64) {
        const int lo = q * g, hi = min(k, lo + g);
        float s = 0.f;
        for (int kk = lo; kk < hi; kk += 8) s += sum8<BF16>(xr + kk);
        rs[(int64_t)q * mp + row] = s;
      }
    }
  }
}

// out = bias + x3 (either may be absent); one 16-bit element per thread, grid-stride.
template <bool BF16>
__global__ __launch_bounds__(256) void bias_x3_kernel(const uint16_t* __restrict__ bias,
                                                      const uint16_t* __restrict__ x3,
                                                      uint16_t* __restrict__ out, int64_t m, int n) {
  const int64_t total = m * n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v = 0.f;
    if (bias) v += act_to_f32<BF16>(bias[i % n]);
    if (x3) v += act_to_f32<BF16>(x3[i]);
    out[i] = f32_to_act<BF16>(v);
  }
}

}  // namespace

int64_t aq_rowsum_mp(int64_t m) { return (m + 255) / 256 * 256; }

hipError_t launch_aq_rowsum(const AqArgs& a, hipStream_t stream) {
  const int64_t mp = aq_rowsum_mp(a.m);
  const int64_t waves = mp;
  const int64_t blocks = std::min<int64_t>((waves + 3) / 4, 65536);
  if (a.bf16)
    hipLaunchKernelGGL(rowsum_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)a.x1, (float*)a.rowsum, a.m, mp, a.k, a.group, a.groups);
  else
    hipLaunchKernelGGL(rowsum_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)a.x1, (float*)a.rowsum, a.m, mp, a.k, a.group, a.groups);
  return hipGetLastError();
}

hipError_t launch_aq_bias_x3(const AqArgs& a, hipStream_t stream) {
  const int64_t total = a.m * a.n;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 65536));
  if (a.bf16)
    hipLaunchKernelGGL(bias_x3_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)a.bias, (const uint16_t*)a.x3, (uint16_t*)a.out, a.m, a.n);
  else
    hipLaunchKernelGGL(bias_x3_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)a.bias, (const uint16_t*)a.x3, (uint16_t*)a.out, a.m, a.n);
  return hipGetLastError();
}

}  // namespace wq

// The empty-K case of the anti-quant matmul, out = bias + x3 ("CANN ops-transformer ...
// aclnnWeightQuantMatmulAllReduce 完全指南", section 空 tensor 支持度 (empty tensors)).
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

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

hipError_t launch_aq_bias_x3(const AqArgs& a, hipStream_t stream) {
  const int64_t total = a.m * a.n;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 65536));
  hipError_t e = profile_begin(stream);
  if (e != hipSuccess) return e;
  if (a.bf16)
    hipLaunchKernelGGL(bias_x3_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)a.bias, (const uint16_t*)a.x3, (uint16_t*)a.out, a.m, a.n);
  else
    hipLaunchKernelGGL(bias_x3_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)a.bias, (const uint16_t*)a.x3, (uint16_t*)a.out, a.m, a.n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return profile_end(stream);
}

}  // namespace wq

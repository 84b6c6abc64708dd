// Small passes around the anti-quant matmul:
//  * the empty-K case, out = bias + x3 ("CANN ops-transformer ... aclnnWeightQuantMatmulAllReduce
//    完全指南", section 空 tensor 支持度 (empty tensors));
//  * per-group scale and offset stored transposed with a transposed x2 (section 参数说明):
//    copied to the row-major (groups, n) layout the GEMM kernels read, in the workspace.
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

// dst (rows, cols) = transpose of src (cols, rows), 16-bit elements, through a 64 x 64 LDS
// tile (rows = groups, cols = n): reads and writes move along the contiguous axis.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* __restrict__ src,
                                                          uint16_t* __restrict__ dst, int rows, int cols) {
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

}  // namespace

hipError_t launch_transpose16(const void* src, void* dst, int rows, int cols, hipStream_t stream) {
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
  hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, stream, (const uint16_t*)src, (uint16_t*)dst,
                     rows, cols);
  return hipGetLastError();
}

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

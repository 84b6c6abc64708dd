// W8A8 matmul for gfx950:
//
//   out = dequant_scale * pertoken_scale * (x1_int8 @ x2_int8 + bias_int32) + x3
//
// ("aclnnQuantMatmulAllReduceV2", section Function, formula case 2; case 1 has no pertoken).
//
// int8 x int8 products accumulate exactly in int32 on the matrix cores
// (v_mfma_i32_32x32x32_i8); bias joins the int32 accumulator before any scaling; the
// scaling and x3 run in fp32 in the epilogue and the result is rounded once to the output
// dtype.  The int32 accumulator (with bias) can be stored as well.
//
// Tiling: 256 threads = 4 waves in a 2 x 2 grid, 128 x 128 per wave (4 x 4 MFMA blocks),
// 256 x 256 per workgroup, BK = 128, double-buffered in LDS.
//   * x1 tile row-major, pitch 144 B; A fragments (16 consecutive k of one row) by 16-byte
//     reads;
//   * x2 tile row-major (n-contiguous), pitch 288 B; B fragments (16 consecutive k of one
//     column) by two tr8 transpose reads.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kApitch = kBK + 16;   // bytes
constexpr int kBpitch = kBN + 32;   // bytes
constexpr int kAbytes = kBM * kApitch;
constexpr int kBbytes = kBK * kBpitch;
constexpr int kStage = kAbytes + kBbytes;
constexpr int kWM = 4, kWN = 4;

__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int t = bid;
  if ((total & 7) == 0) t = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int kGroupM = 4;
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int r = t - g * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 1) void qm_gemm_kernel(const QmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kBM;
  const int n0 = tn * kBN;
  const int64_t M = a.m;
  const int K = a.k, N = a.n;

  // staging: x1 256 rows x 128 B = 2048 chunks; x2 128 rows x 256 B = 2048 chunks
  const int a_chunk = tid & 7, a_row0 = tid >> 3;     // rows a_row0 + 32*i
  const int b_chunk = tid & 15, b_row0 = tid >> 4;    // rows b_row0 + 16*i
  u32x4_t ra[8], rb[8];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = m0 + a_row0 + 32 * i;
      const int kk = k0 + 16 * a_chunk;
      ra[i] = (row < M && kk < K) ? *(const u32x4_t*)(a.x1 + row * K + kk) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kr = k0 + b_row0 + 16 * i;
      const int col = n0 + 16 * b_chunk;
      rb[i] = (kr < K && col < N) ? *(const u32x4_t*)(a.x2 + (int64_t)kr * N + col)
                                  : u32x4_t{0, 0, 0, 0};
    }
  };
  auto store_tiles = [&](int stage) {
    uint8_t* As = smem + stage * kStage;
    uint8_t* Bs = As + kAbytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4_t*)(As + (a_row0 + 32 * i) * kApitch + 16 * a_chunk) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4_t*)(Bs + (b_row0 + 16 * i) * kBpitch + 16 * b_chunk) = rb[i];
  };

  i32x16_t acc[kWM][kWN];
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j) acc[i][j] = i32x16_t{};

  const int nk = (K + kBK - 1) / kBK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int stage = ks & 1;
    const bool more = ks + 1 < nk;
    if (more) load_tiles((ks + 1) * kBK);
    const uint8_t* As = smem + stage * kStage;
    const uint8_t* Bs = As + kAbytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      u32x4_t af[kWM], bfr[kWN];
#pragma unroll
      for (int i = 0; i < kWM; ++i) {
        const int row = wm * 128 + 32 * i + (lane & 31);
        af[i] = *(const u32x4_t*)(As + row * kApitch + 32 * kk + 16 * (lane >> 5));
      }
#pragma unroll
      for (int j = 0; j < kWN; ++j) {
        const int kr = 32 * kk + 16 * (lane >> 5) + ((lane & 15) >> 1);
        const int nc = wn * 128 + 32 * j + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
        const u32x2_t lo = lds_read_tr8(Bs + kr * kBpitch + nc);
        const u32x2_t hi = lds_read_tr8(Bs + (kr + 8) * kBpitch + nc);
        bfr[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int i = 0; i < kWM; ++i)
#pragma unroll
        for (int j = 0; j < kWN; ++j) acc[i][j] = mfma32x32x32_i8(af[i], bfr[j], acc[i][j]);
    }
    if (more) store_tiles(stage ^ 1);
    __syncthreads();
  }

  // epilogue: int32 (acc + bias), then fp32 dq[n] * pt[m] * acc + x3[m, n], rounded once
  const int lane_col = n0 + wn * 128 + (lane & 31);
  const int64_t wave_row0 = m0 + wm * 128;
  int32_t bcol[kWN];
  float dq[kWN];
#pragma unroll
  for (int j = 0; j < kWN; ++j) {
    const int col = lane_col + 32 * j;
    const bool ok = col < N;
    bcol[j] = (ok && a.bias) ? a.bias[col] : 0;
    const int dc = a.dq_per_tensor ? 0 : col;
    dq[j] = !ok ? 0.f
                : (a.dq_bf16 ? bf16_bits_to_f32(((const uint16_t*)a.dq)[dc]) : ((const float*)a.dq)[dc]);
  }
  const uint16_t* x3 = (const uint16_t*)a.x3;
  uint16_t* out = (uint16_t*)a.out;
#pragma unroll
  for (int i = 0; i < kWM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = wave_row0 + 32 * i + acc_row(r, lane);
      if (row >= M) continue;
      const float pt = a.pt ? a.pt[row] : 1.f;
#pragma unroll
      for (int j = 0; j < kWN; ++j) {
        const int col = lane_col + 32 * j;
        if (col >= N) continue;
        const int32_t v = (int32_t)((uint32_t)acc[i][j][r] + (uint32_t)bcol[j]);  // wraps
        const int64_t idx = row * N + col;
        if (a.acc_out) a.acc_out[idx] = v;
        float y = (float)v * dq[j] * pt;
        if (x3) y += OUT_BF16 ? bf16_bits_to_f32(x3[idx]) : f16_bits_to_f32(x3[idx]);
        out[idx] = OUT_BF16 ? f32_to_bf16_rne(y) : f32_to_f16_rne(y);
      }
    }
  }
}

}  // namespace

hipError_t launch_qm_gemm(const QmArgs& a0, hipStream_t stream) {
  QmArgs a = a0;
  a.tiles_m = (int)((a.m + kBM - 1) / kBM);
  a.tiles_n = (a.n + kBN - 1) / kBN;
  const size_t lds = 2 * (size_t)kStage;
  auto kern = a.out_bf16 ? qm_gemm_kernel<true> : qm_gemm_kernel<false>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace wq

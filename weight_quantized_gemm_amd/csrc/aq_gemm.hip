// Anti-quant matmul, large-m kernel for gfx950:
//
//   out = x1 @ ((x2 + offset) * scale) + bias + x3
//
// ("CANN ops-transformer ... aclnnWeightQuantMatmulAllReduce 完全指南", section 计算公式).
//
// The product is evaluated in the factored form (the same formula by linearity):
//
//   out[m,n] = sum_g s[g,n] * ( P_g[m,n] + (off[g,n] - C) * S_g[m] ) + bias[n] + x3[m,n]
//   P_g[m,n] = sum_{i in group g} x1[m,i] * (x2[i,n] + C),   S_g[m] = sum_{i in g} x1[m,i]
//
// where C is the constant bias of the fed weight images (128 for bf16/int8, 136 for
// bf16/int4, 0 for fp16).  The matrix cores see only exact 16-bit images of the integer
// codes and x1; scale and offset are applied in fp32 on the accumulators, per group at
// each group boundary, or once in the epilogue for per-tensor / per-channel parameters.
// S_g comes from the row-sum pass (aq_prep.hip).
//
// Tiling: 256 threads = 4 waves in a 2 x 2 grid; wave tile (32*WM) x (32*WN) of 32x32x16
// MFMA blocks; workgroup tile BM = 64*WM rows x BN = 64*WN columns; BK = 64 along k,
// double-buffered in LDS.
//   * x1 tile: row-major in LDS, pitch 144 B (64 values + 16 B pad), MFMA A fragments by
//     16-byte reads;
//   * x2 tile: converted once per workgroup while staging into 16-bit images, row-major
//     (n-contiguous), pitch 2*BN + 64 B, MFMA B fragments by two tr16 transpose reads.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kApitch = 72;  // u16 per x1 row in LDS (64 + 8 pad)

template <int WM, int WN>
struct AqTile {
  static constexpr int BM = 64 * WM;
  static constexpr int BN = 64 * WN;
  static constexpr int Bpitch = BN + 32;  // u16 per weight row in LDS
  static constexpr int A_elems = BM * kApitch;
  static constexpr int B_elems = kBK * Bpitch;
  static constexpr int Stage = A_elems + B_elems;
  static constexpr int A_chunks = BM * kBK / 8 / kThreads;  // 16-byte x1 chunks per thread
};

// Map a linear workgroup id to a tile.  Workgroups are dispatched round-robin over the 8
// XCDs; consecutive tile ids are handed to one XCD so that its L2 sees a compact band of
// rows and columns, and inside the band tiles are walked in groups of 4 m-tiles.
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

template <bool BF16, bool W4, int WM, int WN, bool GROUPED>
__global__ __launch_bounds__(kThreads, 1) void aq_gemm_kernel(const AqArgs a) {
  using T = AqTile<WM, WN>;
  constexpr int BM = T::BM, BN = T::BN, Bp = T::Bpitch;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const int64_t M = a.m;
  const int K = a.k, N = a.n;

  const uint16_t* __restrict__ x1 = (const uint16_t*)a.x1;
  const uint8_t* __restrict__ x2 = (const uint8_t*)a.x2;

  // ---------------------------------------------------------------- staging registers
  // x1: thread owns 16-byte chunk (tid % 8) of rows tid/8 + 32*i.
  const int a_chunk = tid & 7;
  const int a_row0 = tid >> 3;
  u32x4_t ra[T::A_chunks];
  // x2: int8 -> 16 columns per 16-byte chunk; int4 -> 32 columns per chunk.
  constexpr int kColsPerChunk = W4 ? 32 : 16;
  constexpr int kChunksPerRow = BN / kColsPerChunk;
  constexpr int kRowsPerPass = kThreads / kChunksPerRow;
  constexpr int kBPasses = kBK / kRowsPerPass;
  static_assert(kBPasses >= 1 && kRowsPerPass * kChunksPerRow == kThreads, "B staging shape");
  const int b_chunk = tid % kChunksPerRow;
  const int b_row0 = tid / kChunksPerRow;
  u32x4_t rb[kBPasses];
  const int64_t x2_pitch = W4 ? (N >> 1) : N;  // bytes per weight row

  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < T::A_chunks; ++i) {
      const int64_t row = m0 + a_row0 + 32 * i;
      const int kk = k0 + a_chunk * 8;
      if (row < M && kk < K)
        ra[i] = *(const u32x4_t*)(x1 + row * K + kk);
      else
        ra[i] = u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kBPasses; ++i) {
      const int kr = k0 + b_row0 + kRowsPerPass * i;
      const int col = n0 + b_chunk * kColsPerChunk;
      if (kr < K && col < N)
        rb[i] = *(const u32x4_t*)(x2 + (int64_t)kr * x2_pitch + (W4 ? (col >> 1) : col));
      else
        rb[i] = u32x4_t{0, 0, 0, 0};
    }
  };

  auto store_tiles = [&](int stage) {
    uint16_t* As = smem + stage * T::Stage;
    uint16_t* Bs = As + T::A_elems;
#pragma unroll
    for (int i = 0; i < T::A_chunks; ++i)
      *(u32x4_t*)(As + (a_row0 + 32 * i) * kApitch + a_chunk * 8) = ra[i];
#pragma unroll
    for (int i = 0; i < kBPasses; ++i) {
      uint16_t* dst = Bs + (b_row0 + kRowsPerPass * i) * Bp + b_chunk * kColsPerChunk;
      if constexpr (W4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t o[4];
          i4x8_to_act<BF16>(rb[i][q], o);
          *(u32x4_t*)(dst + 8 * q) = u32x4_t{o[0], o[1], o[2], o[3]};
        }
      } else {
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (BF16) i8x4_to_bf16(rb[i][q], o[2 * q], o[2 * q + 1]);
          else i8x4_to_f16(rb[i][q], o[2 * q], o[2 * q + 1]);
        }
        *(u32x4_t*)(dst) = u32x4_t{o[0], o[1], o[2], o[3]};
        *(u32x4_t*)(dst + 8) = u32x4_t{o[4], o[5], o[6], o[7]};
      }
    }
  };

  // ---------------------------------------------------------------- accumulators
  f32x16_t acc[WM][WN];
  f32x16_t tot[GROUPED ? WM : 1][GROUPED ? WN : 1];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x16_t{};
  if constexpr (GROUPED) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) tot[i][j] = f32x16_t{};
  }

  const uint16_t* __restrict__ scale = (const uint16_t*)a.scale;
  const uint16_t* __restrict__ offset = (const uint16_t*)a.offset;
  const float* __restrict__ rsum = a.rowsum;  // [groups][mp]
  const float cbias = a.code_bias;
  // lane's output column in block j and first output row of block i
  const int lane_col = n0 + wn * (32 * WN) + (lane & 31);
  const int64_t wave_row0 = m0 + wm * (32 * WM);

  // fold one finished group into the totals: tot += s * acc + s * (off - C) * S_g
  auto rescale = [&](int g) {
    float s[WN], q[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int col = lane_col + 32 * j;
      const bool ok = col < N;
      const float sv = ok ? act_to_f32<BF16>(scale[(int64_t)g * N + col]) : 0.f;
      const float ov = (ok && offset) ? act_to_f32<BF16>(offset[(int64_t)g * N + col]) : 0.f;
      s[j] = sv;
      q[j] = sv * (ov - cbias);
    }
    // rowsum rows are padded to a multiple of 256 with zeros, so every tile row is in bounds
    const float* sg = rsum + (int64_t)g * a.mp;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int64_t row = wave_row0 + 32 * i + 8 * rq + 4 * (lane >> 5);
        const f32x4_t sr = *(const f32x4_t*)(sg + row);
#pragma unroll
        for (int j = 0; j < WN; ++j) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rq + e;
            tot[i][j][r] = fmaf(s[j], acc[i][j][r], fmaf(q[j], sr[e], tot[i][j][r]));
          }
        }
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[i][j] = f32x16_t{};
    }
  };

  // ---------------------------------------------------------------- main loop
  const int nk = (K + kBK - 1) / kBK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int stage = ks & 1;
    const bool more = ks + 1 < nk;
    if (more) load_tiles((ks + 1) * kBK);

    const uint16_t* As = smem + stage * T::Stage;
    const uint16_t* Bs = As + T::A_elems;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4_t af[WM], bfr[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int row = wm * (32 * WM) + 32 * i + (lane & 31);
        af[i] = *(const u32x4_t*)(As + row * kApitch + kk * 16 + 8 * (lane >> 5));
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int kr = kk * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
        const int nc = wn * (32 * WN) + 32 * j + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const u32x2_t lo = lds_read_tr16(Bs + kr * Bp + nc);
        const u32x2_t hi = lds_read_tr16(Bs + (kr + 4) * Bp + nc);
        bfr[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = mfma32x32x16<BF16>(af[i], bfr[j], acc[i][j]);

      if constexpr (GROUPED) {
        if (kk & 1) {  // a 32-wide slice of k is done; groups end on multiples of 32
          const int kdone = ks * kBK + kk * 16 + 16;
          if (kdone <= K && (kdone % a.group == 0 || kdone == K)) rescale((kdone - 1) / a.group);
        }
      }
    }

    if (more) store_tiles(stage ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  const uint16_t* __restrict__ bias = (const uint16_t*)a.bias;
  const uint16_t* __restrict__ x3 = (const uint16_t*)a.x3;
  uint16_t* __restrict__ out = (uint16_t*)a.out;
  float s[WN], q[WN], bcol[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int col = lane_col + 32 * j;
    const bool ok = col < N;
    bcol[j] = (ok && bias) ? act_to_f32<BF16>(bias[col]) : 0.f;
    if constexpr (!GROUPED) {
      const int pc = a.per_tensor ? 0 : col;
      const float sv = ok ? act_to_f32<BF16>(scale[pc]) : 0.f;
      const float ov = (ok && offset) ? act_to_f32<BF16>(offset[pc]) : 0.f;
      s[j] = sv;
      q[j] = sv * (ov - cbias);
    }
  }
#pragma unroll
  for (int i = 0; i < WM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = wave_row0 + 32 * i + acc_row(r, lane);
      if (row >= M) continue;
      float srow = 0.f;
      if constexpr (!GROUPED) srow = rsum[row];
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int col = lane_col + 32 * j;
        if (col >= N) continue;
        float v;
        if constexpr (GROUPED) v = tot[i][j][r];
        else v = fmaf(s[j], acc[i][j][r], q[j] * srow);
        v += bcol[j];
        const int64_t idx = row * N + col;
        if (x3) v += act_to_f32<BF16>(x3[idx]);
        out[idx] = f32_to_act<BF16>(v);
      }
    }
  }
}

template <bool BF16, bool W4, int WM, int WN, bool GROUPED>
hipError_t launch_one(const AqArgs& a0, hipStream_t stream) {
  using T = AqTile<WM, WN>;
  AqArgs a = a0;
  a.tiles_m = (int)((a.m + T::BM - 1) / T::BM);
  a.tiles_n = (a.n + T::BN - 1) / T::BN;
  const size_t lds = 2 * (size_t)T::Stage * sizeof(uint16_t);
  auto kern = aq_gemm_kernel<BF16, W4, WM, WN, GROUPED>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

// Per-tensor / per-channel: 256 x 256 workgroup tiles (128 x 128 per wave).
// Per-group: the group rescale needs a second accumulator set, so 256 x 128 tiles.
hipError_t launch_aq_gemm(const AqArgs& a, hipStream_t stream) {
  const bool grouped = a.grouped;
  if (a.bf16) {
    if (a.w4) return grouped ? launch_one<true, true, 4, 2, true>(a, stream)
                             : launch_one<true, true, 4, 4, false>(a, stream);
    return grouped ? launch_one<true, false, 4, 2, true>(a, stream)
                   : launch_one<true, false, 4, 4, false>(a, stream);
  }
  if (a.w4) return grouped ? launch_one<false, true, 4, 2, true>(a, stream)
                           : launch_one<false, true, 4, 4, false>(a, stream);
  return grouped ? launch_one<false, false, 4, 2, true>(a, stream)
                 : launch_one<false, false, 4, 4, false>(a, stream);
}

}  // namespace wq

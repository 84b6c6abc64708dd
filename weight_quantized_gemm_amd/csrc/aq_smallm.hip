// Anti-quant matmul for small m (m <= 32): the weight stream dominates, so the kernel is
// shaped for HBM bandwidth rather than for matrix-core reuse.
//
//   out = x1 @ ((x2 + offset) * scale) + bias + x3
// ("CANN ops-transformer ... aclnnWeightQuantMatmulAllReduce 完全指南", section 计算公式),
// evaluated in the same factored form as the large-m kernel (aq_gemm.hip).
//
// Work split: a workgroup owns a 128-column slab of x2 and a contiguous range of k (split-k);
// its 4 waves take the 64-row blocks of that range round-robin.  Each wave streams its
// block (global -> registers -> wave-private LDS, row-major int8 / packed int4), reads MFMA
// B fragments back with tr8 transpose reads (8 consecutive k of one column per lane),
// turns them into exact 16-bit images and runs 32x32x16 MFMAs against the 32 rows of x1.
// Per-group parameters are folded at every group end; a group cut by the end of a wave's
// block is folded with its scale only, and its offset term is added once, by the block
// that holds the group's end.  The 4 waves are reduced through LDS in a fixed order, the
// splits by a finishing kernel in a fixed order: results are deterministic.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {
namespace {

constexpr int kThreads = 256;
constexpr int kSlab = 128;   // logical columns per workgroup
constexpr int kRows = 64;    // k rows per wave block

template <bool W4>
struct SmTile {
  static constexpr int RowBytes = W4 ? kSlab / 2 : kSlab;   // 64 or 128 bytes per k row
  static constexpr int Pitch = RowBytes + 32;                // 96 or 160: tr8 bank spread
  static constexpr int Buf = kRows * Pitch;                  // bytes of the wave's LDS tile
  static constexpr int Loads = kRows * RowBytes / 16 / 64;   // 16-byte loads per lane
  static constexpr int LanesPerRow = RowBytes / 16;
};

template <bool BF16, bool W4, bool GROUPED>
__global__ __launch_bounds__(kThreads, 1) void aq_smallm_kernel(const AqArgs a) {
  using T = SmTile<W4>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * T::Buf > 4 * 32 * kSlab * 4
                                                            ? 4 * T::Buf
                                                            : 4 * 32 * kSlab * 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slab = blockIdx.x, split = blockIdx.y;
  const int n0 = slab * kSlab;
  const int K = a.k, N = a.n;
  const int M = (int)a.m;
  const int kchunk = ((K + a.splits - 1) / a.splits + kRows - 1) / kRows * kRows;
  const int kbeg = split * kchunk;
  const int kend = min(K, kbeg + kchunk);
  const int nblocks = kend > kbeg ? (kend - kbeg + kRows - 1) / kRows : 0;

  const uint16_t* __restrict__ x1 = (const uint16_t*)a.x1;
  const uint8_t* __restrict__ x2 = (const uint8_t*)a.x2;
  const int64_t x2_pitch = W4 ? (N >> 1) : N;
  // One LDS tile per wave suffices: a wave's LDS instructions execute in issue order, so
  // the transpose reads of block b complete before the stores of block b + 4 land.
  uint8_t* wbuf = smem + wave * T::Buf;

  // ---- per-lane load pattern: LanesPerRow lanes cover one k row of the slab
  const int l_row = lane / T::LanesPerRow;
  const int l_byte = 16 * (lane % T::LanesPerRow);
  constexpr int kRowsPerLoad = 64 / T::LanesPerRow;
  const int col_bytes0 = (W4 ? n0 / 2 : n0) + l_byte;
  const bool col_ok = (W4 ? 2 * col_bytes0 : col_bytes0) < N;

  // two register sets: blocks b and b + 4 are in flight while block b - 4 is computed
  u32x4_t rb[2][T::Loads];
  u32x4_t ra[2][4];
  auto load_block = [&](int set, int blk) {
    const int k0 = kbeg + blk * kRows;
#pragma unroll
    for (int q = 0; q < T::Loads; ++q) {
      const int kr = k0 + l_row + kRowsPerLoad * q;
      rb[set][q] = (kr < kend && col_ok) ? *(const u32x4_t*)(x2 + (int64_t)kr * x2_pitch + col_bytes0)
                                         : u32x4_t{0, 0, 0, 0};
    }
    const int arow = lane & 31;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kc = k0 + 16 * kk + 8 * (lane >> 5);
      ra[set][kk] = (arow < M && kc < kend) ? *(const u32x4_t*)(x1 + (int64_t)arow * K + kc)
                                            : u32x4_t{0, 0, 0, 0};
    }
  };
  auto store_block = [&](int set) {
#pragma unroll
    for (int q = 0; q < T::Loads; ++q)
      *(u32x4_t*)(wbuf + (l_row + kRowsPerLoad * q) * T::Pitch + l_byte) = rb[set][q];
  };

  // accumulators: 4 blocks of 32 columns (int4: byte-column pair p, parity e -> block 2p+e)
  f32x16_t acc[4], tot[GROUPED ? 4 : 1];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16_t{};
  if constexpr (GROUPED) {
#pragma unroll
    for (int j = 0; j < 4; ++j) tot[j] = f32x16_t{};
  }
  // logical column of this lane in block j
  auto block_col = [&](int j) -> int {
    if constexpr (W4) return n0 + 64 * (j >> 1) + 2 * (lane & 31) + (j & 1);
    else return n0 + 32 * j + (lane & 31);
  };

  const uint16_t* __restrict__ scale = (const uint16_t*)a.scale;
  const uint16_t* __restrict__ offset = (const uint16_t*)a.offset;
  const float cbias = a.code_bias;
  // fold the running group g: tot += s*acc (+ s*(off-C)*S_g when the group ends here)
  auto fold = [&](int g, bool group_end) {
    float s[4], q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = block_col(j);
      const bool ok = col < N;
      const float sv = ok ? act_to_f32<BF16>(scale[(int64_t)g * N + col]) : 0.f;
      const float ov = (ok && offset) ? act_to_f32<BF16>(offset[(int64_t)g * N + col]) : 0.f;
      s[j] = sv;
      q[j] = group_end ? sv * (ov - cbias) : 0.f;
    }
    const float* sg = a.rowsum + (int64_t)g * a.mp;
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const f32x4_t sr = *(const f32x4_t*)(sg + 8 * rq + 4 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          tot[j][4 * rq + e] = fmaf(s[j], acc[j][4 * rq + e], fmaf(q[j], sr[e], tot[j][4 * rq + e]));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x16_t{};
  };

  // compute one block from the wave's LDS tile (already stored) with x1 fragments af
  auto compute_block = [&](const u32x4_t* af, int blk) {
    const int k0 = kbeg + blk * kRows;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int row = kk * 16 + 8 * (lane >> 5) + ((lane & 15) >> 1);
#pragma unroll
      for (int p = 0; p < (W4 ? 2 : 4); ++p) {
        const int cb = 32 * p + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
        const u32x2_t d = lds_read_tr8(wbuf + row * T::Pitch + cb);
        if constexpr (W4) {
          u32x4_t ev, od;
          i4_kpairs<BF16>(d, ev, od);
          acc[2 * p] = mfma32x32x16<BF16>(af[kk], ev, acc[2 * p]);
          acc[2 * p + 1] = mfma32x32x16<BF16>(af[kk], od, acc[2 * p + 1]);
        } else {
          acc[p] = mfma32x32x16<BF16>(af[kk], i8x8_to_act<BF16>(d), acc[p]);
        }
      }
      if constexpr (GROUPED) {
        if (kk & 1) {  // groups end on multiples of 32
          const int kdone = k0 + 16 * kk + 16;
          const bool ends = kdone <= kend && (kdone % a.group == 0 || kdone == K);
          const bool last = kdone >= min(kend, k0 + kRows);  // end of this block
          if (ends) fold((kdone - 1) / a.group, true);
          else if (last) fold((min(kdone, kend) - 1) / a.group, false);
        }
      }
    }
  };

  // ---- stream this wave's blocks: wave, wave + 4, ... with two blocks in flight
  int blk = wave;
  if (blk < nblocks) load_block(0, blk);
  if (blk + 4 < nblocks) load_block(1, blk + 4);
  while (blk < nblocks) {
    store_block(0);
    const u32x4_t a0[4] = {ra[0][0], ra[0][1], ra[0][2], ra[0][3]};
    if (blk + 8 < nblocks) load_block(0, blk + 8);
    compute_block(a0, blk);
    blk += 4;
    if (blk >= nblocks) break;
    store_block(1);
    const u32x4_t a1[4] = {ra[1][0], ra[1][1], ra[1][2], ra[1][3]};
    if (blk + 8 < nblocks) load_block(1, blk + 8);
    compute_block(a1, blk);
    blk += 4;
  }

  // ---- reduce the 4 waves in a fixed order, write this split's partial [split][m][n]
  __syncthreads();
  float* red = (float*)smem;  // [4][32][kSlab]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int lc = block_col(j) - n0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = acc_row(r, lane);
      red[(wave * 32 + row) * kSlab + lc] = GROUPED ? tot[j][r] : acc[j][r];
    }
  }
  __syncthreads();
  float* part = a.partial + (int64_t)split * a.m * N;
  for (int o = tid; o < 32 * kSlab; o += kThreads) {
    const int row = o / kSlab, lc = o % kSlab;
    if (row >= M || n0 + lc >= N) continue;
    const float v = red[(0 * 32 + row) * kSlab + lc] + red[(1 * 32 + row) * kSlab + lc] +
                    red[(2 * 32 + row) * kSlab + lc] + red[(3 * 32 + row) * kSlab + lc];
    part[(int64_t)row * N + n0 + lc] = v;
  }
}

// out = [s*P + s*(off-C)*S]  (per-tensor / per-channel)  or  T (per-group), + bias + x3,
// where P / T is the sum of the split partials in split order.
template <bool BF16, bool GROUPED>
__global__ __launch_bounds__(256) void aq_smallm_finish(const AqArgs a) {
  const int64_t total = a.m * a.n;
  const int N = a.n;
  const uint16_t* scale = (const uint16_t*)a.scale;
  const uint16_t* offset = (const uint16_t*)a.offset;
  const uint16_t* bias = (const uint16_t*)a.bias;
  const uint16_t* x3 = (const uint16_t*)a.x3;
  uint16_t* out = (uint16_t*)a.out;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / N;
    const int col = (int)(i - row * N);
    float v = 0.f;
    for (int s = 0; s < a.splits; ++s) v += a.partial[(int64_t)s * total + i];
    if constexpr (!GROUPED) {
      const int pc = a.per_tensor ? 0 : col;
      const float sv = act_to_f32<BF16>(scale[pc]);
      const float ov = offset ? act_to_f32<BF16>(offset[pc]) : 0.f;
      v = fmaf(sv, v, sv * (ov - a.code_bias) * a.rowsum[row]);
    }
    if (bias) v += act_to_f32<BF16>(bias[col]);
    if (x3) v += act_to_f32<BF16>(x3[i]);
    out[i] = f32_to_act<BF16>(v);
  }
}

template <bool BF16, bool W4, bool GROUPED>
hipError_t launch_sm(const AqArgs& a, hipStream_t stream) {
  const int slabs = (a.n + kSlab - 1) / kSlab;
  hipLaunchKernelGGL((aq_smallm_kernel<BF16, W4, GROUPED>), dim3(slabs, a.splits), dim3(kThreads),
                     0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = a.m * a.n;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 4096));
  hipLaunchKernelGGL((aq_smallm_finish<BF16, GROUPED>), dim3((unsigned)blocks), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

int aq_smallm_splits(int64_t m, int k, int n, int group, bool grouped) {
  (void)m; (void)group; (void)grouped;
  const int slabs = (n + kSlab - 1) / kSlab;
  int splits = std::max(1, 256 / std::max(1, slabs));  // about one workgroup per CU
  const int max_splits = std::max(1, (k + 4 * kRows - 1) / (4 * kRows));  // >= 4 blocks per split
  return std::min(splits, max_splits);
}

hipError_t launch_aq_smallm(const AqArgs& a, hipStream_t stream) {
  if (a.bf16) {
    if (a.w4) return a.grouped ? launch_sm<true, true, true>(a, stream) : launch_sm<true, true, false>(a, stream);
    return a.grouped ? launch_sm<true, false, true>(a, stream) : launch_sm<true, false, false>(a, stream);
  }
  if (a.w4) return a.grouped ? launch_sm<false, true, true>(a, stream) : launch_sm<false, true, false>(a, stream);
  return a.grouped ? launch_sm<false, false, true>(a, stream) : launch_sm<false, false, false>(a, stream);
}

}  // namespace wq

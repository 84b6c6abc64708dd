// W8A8 matmul for gfx950:
//
//   out = dequant_scale * pertoken_scale * (x1_int8 @ x2_int8 + bias_int32) + x3
//
// ("aclnnQuantMatmulAllReduceV2", section Function, formula case 2; case 1 has no pertoken).
//
// int8 x int8 products accumulate exactly in int32 on the matrix cores
// (v_mfma_i32_32x32x32_i8); bias joins the int32 accumulator before any scaling (two's
// complement wrap past the int32 range); scaling and x3 run in fp32 in the epilogue and the
// result is rounded once to the output dtype.  The int32 accumulator (with bias) can be
// stored as well.
//
// Pipeline: 8 waves (2 x 4, two per SIMD), wave tile 128 x 64, workgroup tile 256 x 256,
// BK = 64.  x1 and x2 tiles move global -> LDS by direct-to-LDS buffer loads through a
// 4-stage ring (three stages in flight), one barrier per k-step.  x1 rows (64 bytes) are
// read as MFMA A fragments by 16-byte loads; x2 rows (256 bytes, n-contiguous) give B
// fragments by two tr8 transpose reads (16 consecutive k of one column).  A transposed x2
// (stored (n, k), which the Parameters table allows) travels exactly like x1: 64-byte rows
// of k per column, 16-byte fragment loads, no transpose.  A packed x2 (wq_prepack_weight)
// travels as one contiguous 16 KiB run per stage and gives each B fragment in two 8-byte
// reads.  The epilogue
// stages the accumulators through LDS so that x3, the output and the int32 accumulator
// move in 16-byte row-contiguous accesses.  With few output tiles k is split (grid y):
// the splits write int32 partial tiles and qm_splitk_finish adds them, in split order.
#include <algorithm>

#include "wq_kernels.h"
#include "wq_pipeline.h"

namespace wq {
namespace {

constexpr int kBN = 256, kBK = 64;
constexpr int kStages = 4;
constexpr int kRA = kBK;                        // bytes per x1 row in a stage
constexpr int kRB = kBN;                        // bytes per x2 row in a stage
constexpr int kBbytes = kBK * kRB;              // 16 KiB
static_assert(kBN == kQmTileN, "the planner's tile is the kernel's");
// per workgroup-tile height BM (256, or 128 / 64 for short m or short split chunks): x1
// stage, stage, LDS
template <int BM> constexpr int qm_abytes() { return BM * kRA; }          // 16 / 8 / 4 KiB
template <int BM> constexpr int qm_stage() { return qm_abytes<BM>() + kBbytes; }
template <int BM> constexpr int qm_lds() { return kStages * qm_stage<BM>(); }  // 128 / 96 / 80 KiB

// Wave grid GM x GN with WM x WN 32x32 blocks per wave (BM x 256 per workgroup); XT: x2
// stored transposed, (n, k); PK: x2 in the packed layout (wq_prepack_weight: 64 k x 32
// column blocks holding, per 16-k step, each lane's 8 codes).  An int8 MFMA takes 32 k: a
// lane's 16 codes of a packed B fragment are the two 8-code pieces that the anti-quant
// layout gives to lanes c and c + 32 of one 16-k step.
template <bool OUT_BF16, int kGM, int kGN, bool XT, int BM = 256, bool PK = false>
__global__ __launch_bounds__(64 * kGM * kGN, 1) void qm_gemm_kernel(const QmArgs a) {
  static_assert(!(XT && PK), "one weight layout");
  constexpr int kWaves = kGM * kGN;
  constexpr int kBM = BM;
  constexpr int kAbytes = qm_abytes<BM>(), kStage = qm_stage<BM>();
  constexpr int kWM = BM / 32 / kGM, kWN = 8 / kGN;
  static_assert(kWM >= 1 && kWM * 32 * kGM == BM, "wave rows cover the tile");
  constexpr int kAper = kAbytes / 1024 / kWaves;  // DMA blocks per wave
  constexpr int kBper = kBbytes / 1024 / kWaves;
  constexpr int kDma = kAper + kBper;             // DMA loads per wave per stage
  static_assert(kAper >= 1 && kBper >= 1, "DMA split");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kGN, wn = wave % kGN;
  int tm, tn;
  tile_of(blockIdx.x, a.tiles_m, a.tiles_n, a.xcd_rm, tm, tn);
  const int64_t m0 = (int64_t)tm * kBM;
  const int n0 = tn * kBN;
  const int64_t M = a.m;
  const int K = a.k, N = a.n;
  // split k: this workgroup's k range (split starts are multiples of 64, so only the last
  // split can end in a partial k-step)
  const int split = blockIdx.y;
  const int kbeg = split * a.kchunk;
  const int kend = a.splits > 1 ? min(K, kbeg + a.kchunk) : K;
  const int nk = (kend - kbeg + kBK - 1) / kBK;

  // ------------------------------------------------------------------ DMA issue
  const uint8_t* x1b = (const uint8_t*)a.x1 + m0 * K;
  const int64_t x1_bytes = (M - m0) * K;
  const uint8_t* x2b = (const uint8_t*)a.x2 + (XT ? (int64_t)n0 * K : (int64_t)n0);
  // transposed x2: bytes from the tile's first column on that the tile may read
  const uint32_t x2t_bytes = (uint32_t)((N - n0 < kBN ? N - n0 : kBN) * (int64_t)K);
  uint32_t a_off[kAper];
  int a_chunk[kAper];
#pragma unroll
  for (int j = 0; j < kAper; ++j) {
    const int b = wave + kWaves * j;                 // 16 rows of 64 bytes
    const int r = 16 * b + (lane >> 2);
    a_chunk[j] = row_slot<kRA>(r, lane & 3);         // logical chunk in this physical slot
    a_off[j] = (uint32_t)(r * K + 16 * a_chunk[j]);
  }
  uint32_t b_off[kBper];
  int b_chunk[kBper];
#pragma unroll
  for (int j = 0; j < kBper; ++j) {
    const int b = wave + kWaves * j;
    if constexpr (PK) {                              // the stage's blocks are one contiguous run
      b_chunk[j] = 0;
      b_off[j] = 1024u * (uint32_t)b + 16u * (uint32_t)lane;
    } else if constexpr (XT) {                       // 16 columns of 64 bytes of k
      const int r = 16 * b + (lane >> 2);
      b_chunk[j] = row_slot<kRA>(r, lane & 3);
      b_off[j] = (uint32_t)(r * K + 16 * b_chunk[j]);
    } else {                                         // 4 k rows of 256 bytes
      const int r = 4 * b + (lane >> 4);
      const int p = lane & 15;
      b_chunk[j] = 0;
      b_off[j] = (uint32_t)(r * N + 16 * (2 * pair_slot<kRB>(r, p >> 1) + (p & 1)));
    }
  }
  // A stage's loads are formed once (stage_rsrc) and issued in two halves, one behind
  // each 32-k step of the k-step that issues them, so that the texture unit is not handed
  // a burst of loads that stalls the waves' matrix-core work.
  struct StageRsrc {
    u32x4_t ra, rb;
    uint8_t* st;
    int k0;
    bool tail;
  };
  auto stage_rsrc = [&](int ks) {
    StageRsrc r;
    r.k0 = kbeg + ks * kBK;
    r.st = smem + (ks % kStages) * kStage;
    // Every k-step issues the loads of the stage kStages - 1 ahead, also past the split's
    // range: those get empty resources, so they read nothing and write zeros into a stage no
    // wave reads any more.  The loop then has one wait count and no branches around its loads.
    const bool live = ks < nk;
    r.ra = make_rsrc(x1b + r.k0, live ? x1_bytes - r.k0 : 0);
    if constexpr (PK) {
      // the tile's column blocks of 64-k block k0 / 64; blocks past n read zero, and so do
      // codes past k (the packed layout pads them with zeros)
      const int nbl = N / 32, nbt = n0 / 32;
      const int valid = nbl - nbt < kBN / 32 ? nbl - nbt : kBN / 32;
      r.rb = make_rsrc((const uint8_t*)a.x2 + ((int64_t)(r.k0 / kBK) * nbl + nbt) * 2048,
                       live ? (int64_t)valid * 2048 : 0);
    } else if constexpr (XT) {
      r.rb = make_rsrc32(x2b + r.k0, live ? x2t_bytes - (uint32_t)r.k0 : 0u);
    } else {
      const int rows = K - r.k0 < kBK ? K - r.k0 : kBK;
      r.rb = make_rsrc32(x2b + (int64_t)r.k0 * N, live ? (uint32_t)(rows * N - n0) : 0u);
    }
    r.tail = r.k0 + kBK > K;
    return r;
  };
  // half h of a stage: x1 blocks j with j % 2 == h, weight blocks j with j % 2 == h
  auto issue_half = [&](const StageRsrc& r, int h) {
#pragma unroll
    for (int j = 0; j < kAper; ++j) {
      if (j % 2 != h) continue;
      uint8_t* dst = r.st + 1024 * (wave + kWaves * j);
      dma16(r.ra, dst, (r.tail && r.k0 + 16 * a_chunk[j] >= K) ? kOOB : a_off[j]);
    }
#pragma unroll
    for (int j = 0; j < kBper; ++j) {
      if (j % 2 != h) continue;
      uint8_t* dst = r.st + kAbytes + 1024 * (wave + kWaves * j);
      if constexpr (!XT) dma16(r.rb, dst, b_off[j]);
      else dma16(r.rb, dst, (r.tail && r.k0 + 16 * b_chunk[j] >= K) ? kOOB : b_off[j]);
    }
  };
  auto issue = [&](int ks) {
    const StageRsrc r = stage_rsrc(ks);
    issue_half(r, 0);
    issue_half(r, 1);
  };

  i32x16_t acc[kWM][kWN];
#pragma unroll
  for (int i = 0; i < kWM; ++i)
#pragma unroll
    for (int j = 0; j < kWN; ++j) acc[i][j] = i32x16_t{};

  // ------------------------------------------------------------------ epilogue geometry
  // The epilogue moves 8 consecutive columns of one row per lane.  Its x3 rows are
  // prefetched into registers while the last k-step's MFMAs run (two 32-row bands ahead).
  constexpr int WC = 32 * kWN;          // wave columns
  constexpr int EP = WC + 8;            // int32 pitch of the staging rows
  constexpr int LanesPerRow = WC / 8;   // lanes per row, 8 columns each
  constexpr int RowsPerPass = 64 / LanesPerRow;
  constexpr int kPasses = 32 / RowsPerPass;
  const int ecol = 8 * (lane % LanesPerRow);
  const int gcol = n0 + wn * WC + ecol;
  const bool col_ok = gcol < N;
  // with split k the epilogue writes int32 partials; bias, scales and x3 are applied when the
  // splits are added
  const bool split_out = a.splits > 1;
  const uint16_t* x3 = split_out ? nullptr : (const uint16_t*)a.x3;
  u32x4_t xpre[2][kPasses];
  auto prefetch_x3 = [&](int i, int slot) {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int er = p * RowsPerPass + lane / LanesPerRow;
      const int64_t grow = m0 + wm * (32 * kWM) + 32 * i + er;
      xpre[slot][p] = (x3 && col_ok && grow < M) ? *(const u32x4_t*)(x3 + grow * N + gcol)
                                                 : u32x4_t{0, 0, 0, 0};
    }
  };

  // ------------------------------------------------------------------ main loop
  // Fragments are double-buffered across the two 32-k steps, and across stages: the barrier
  // that publishes stage ks + 1 is taken before the MFMAs of stage ks's second step, and the
  // first fragment reads of stage ks + 1 follow it at once, so that their LDS latency and the
  // wait for the slowest wave hide behind those MFMAs.  The barrier also tells every wave
  // that all reads of stage ks - 1 are done: its buffer is the one the loads issued during
  // stage ks refill.
  constexpr int kEarly = (kAper + 1) / 2 + (kBper + 1) / 2;  // loads of a stage's first half
  u32x4_t af[2][kWM], bfr[2][kWN];
  auto load = [&](const uint8_t* As, int kk, int buf) {
    const uint8_t* Bs = As + kAbytes;
#pragma unroll
    for (int i = 0; i < kWM; ++i) {
      const int r = wm * (32 * kWM) + 32 * i + (lane & 31);
      af[buf][i] = *(const u32x4_t*)(As + r * kRA + 16 * row_slot<kRA>(r, 2 * kk + (lane >> 5)));
    }
    if constexpr (PK) {
      // lane (h, c) takes k 32 kk + 16 h + 0..15 of column c: the 16-k step 2 kk + h of the
      // packed block, where lane c holds its k 0..7 and lane c + 32 its k 8..15
      const int h = lane >> 5, c = lane & 31;
#pragma unroll
      for (int j = 0; j < kWN; ++j) {
        const uint8_t* q = Bs + (wn * kWN + j) * 2048 + (2 * kk + h) * 512 + 8 * c;
        const u32x2_t lo = *(const u32x2_t*)q;
        const u32x2_t hi = *(const u32x2_t*)(q + 256);
        bfr[buf][j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
      return;
    }
    if constexpr (XT) {
#pragma unroll
      for (int j = 0; j < kWN; ++j) {
        const int r = wn * WC + 32 * j + (lane & 31);
        bfr[buf][j] = *(const u32x4_t*)(Bs + r * kRA + 16 * row_slot<kRA>(r, 2 * kk + (lane >> 5)));
      }
    } else {
      const int kr = 32 * kk + 16 * (lane >> 5) + ((lane & 15) >> 1);
#pragma unroll
      for (int j = 0; j < kWN; ++j) {
        const int pair = wn * kWN + j;
        const int sub = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
        const u32x2_t lo = lds_read_tr8(Bs + kr * kRB + 32 * pair_slot<kRB>(kr, pair) + sub);
        const u32x2_t hi = lds_read_tr8(Bs + (kr + 8) * kRB + 32 * pair_slot<kRB>(kr + 8, pair) + sub);
        bfr[buf][j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
    }
  };
  static_assert(kStages == 4, "three stages ahead");
  issue(0);
  issue(1);
  issue(2);
  stage_barrier<2 * kDma>();  // stage 0 complete; stages 1 and 2 may stay in flight
  load(smem, 0, 0);
  for (int ks = 0; ks < nk; ++ks) {
    const StageRsrc nr = stage_rsrc(ks + kStages - 1);
    if (ks == nk - 1) {  // only loads past the range left: start the epilogue's x3 reads
      prefetch_x3(0, 0);
      if (kWM > 1) prefetch_x3(1, 1);
    }
    const uint8_t* As = smem + (ks % kStages) * kStage;
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      static_assert(kBK / 32 == 2, "two 32-k steps per stage");
      if (kk == 0) {
        load(As, 1, 1);
      } else if (ks + 1 < nk) {
        // stage ks + 1 complete: in flight may stay stage ks + 2 and the first-half loads
        // of stage ks + 3
        stage_barrier<kDma + kEarly>();
        load(smem + ((ks + 1) % kStages) * kStage, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kWM; ++i)
#pragma unroll
        for (int j = 0; j < kWN; ++j) acc[i][j] = mfma32x32x32_i8(af[kk][i], bfr[kk][j], acc[i][j]);
      issue_half(nr, kk);  // behind this step's matrix-core work
    }
  }

  // ------------------------------------------------------------------ epilogue
  wave_wait<0>();   // the loads past the range (zeros) have landed
  __syncthreads();
  int32_t* E = (int32_t*)smem + wave * (32 * EP);
  int32_t cb[8];
  float cdq[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { cb[e] = 0; cdq[e] = 0.f; }
  if (col_ok) {
    if (a.bias) {
      const i32x4_t b0 = *(const i32x4_t*)(a.bias + gcol), b1 = *(const i32x4_t*)(a.bias + gcol + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { cb[e] = b0[e]; cb[e + 4] = b1[e]; }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dc = a.dq_per_tensor ? 0 : gcol + e;
      cdq[e] = a.dq_bf16 ? bf16_bits_to_f32(((const uint16_t*)a.dq)[dc]) : ((const float*)a.dq)[dc];
    }
  }
  uint16_t* out = (uint16_t*)a.out;
#pragma unroll
  for (int i = 0; i < kWM; ++i) {
#pragma unroll
    for (int j = 0; j < kWN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) E[acc_row(r, lane) * EP + 32 * j + (lane & 31)] = acc[i][j][r];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int er = p * RowsPerPass + lane / LanesPerRow;
      const int64_t grow = m0 + wm * (32 * kWM) + 32 * i + er;
      const u32x4_t xv = xpre[i & 1][p];
      const i32x4_t v0 = *(const i32x4_t*)(E + er * EP + ecol);
      const i32x4_t v1 = *(const i32x4_t*)(E + er * EP + ecol + 4);
      if (grow >= M || !col_ok) continue;
      if (split_out) {
        int32_t* part = a.partial + (int64_t)split * M * N + grow * N + gcol;
        *(i32x4_t*)part = v0;
        *(i32x4_t*)(part + 4) = v1;
        continue;
      }
      int32_t v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = (int32_t)((uint32_t)v0[e] + (uint32_t)cb[e]);
        v[e + 4] = (int32_t)((uint32_t)v1[e] + (uint32_t)cb[e + 4]);
      }
      const int64_t idx = grow * N + gcol;
      if (a.acc_out) {
        *(i32x4_t*)(a.acc_out + idx) = i32x4_t{v[0], v[1], v[2], v[3]};
        *(i32x4_t*)(a.acc_out + idx + 4) = i32x4_t{v[4], v[5], v[6], v[7]};
      }
      const float pt = a.pt ? a.pt[grow] : 1.f;
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float y0 = (float)v[e] * cdq[e] * pt, y1 = (float)v[e + 1] * cdq[e + 1] * pt;
        if (x3) {
          const uint32_t xw = xv[e >> 1];
          y0 += OUT_BF16 ? bf16_bits_to_f32(xw & 0xffffu) : f16_bits_to_f32(xw & 0xffffu);
          y1 += OUT_BF16 ? bf16_bits_to_f32(xw >> 16) : f16_bits_to_f32(xw >> 16);
        }
        o[e >> 1] = (uint32_t)(OUT_BF16 ? f32_to_bf16_rne(y0) : f32_to_f16_rne(y0)) |
                    ((uint32_t)(OUT_BF16 ? f32_to_bf16_rne(y1) : f32_to_f16_rne(y1)) << 16);
      }
      *(u32x4_t*)(out + idx) = u32x4_t{o[0], o[1], o[2], o[3]};
    }
    if (i + 2 < kWM) prefetch_x3(i + 2, i & 1);
  }
}

// Split-k finish: acc = the int32 partials added in split order (two's complement wrap, so
// the sum is the single-pass accumulator bit for bit) + bias; the optional accumulator
// output, then out = acc * dequant_scale * pertoken_scale + x3, rounded once.  A thread
// handles four consecutive columns of one row (n is a multiple of 32).
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void qm_splitk_finish(const QmArgs a) {
  const int N = a.n;
  const int64_t quads = a.m * (N / 4);
  const int64_t plane = a.m * N;
  const uint16_t* x3 = (const uint16_t*)a.x3;
  uint16_t* out = (uint16_t*)a.out;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = q / (N / 4);
    const int col = 4 * (int)(q - row * (N / 4));
    const int64_t idx = row * N + col;
    // every operand is loaded ahead of its use; partials four splits at a time, at clamped
    // split indices so that no load waits behind a branch
    const i32x4_t b = a.bias ? *(const i32x4_t*)(a.bias + col) : i32x4_t{0, 0, 0, 0};
    const float pt = a.pt ? a.pt[row] : 1.f;
    u32x2_t xv{0u, 0u};
    if (x3) xv = *(const u32x2_t*)(x3 + idx);
    i32x4_t v = *(const i32x4_t*)(a.partial + idx);
    for (int s0 = 1; s0 < a.splits; s0 += 4) {
      i32x4_t p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = *(const i32x4_t*)(a.partial + (int64_t)min(s0 + j, a.splits - 1) * plane + idx);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (s0 + j < a.splits) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (int32_t)((uint32_t)v[e] + (uint32_t)p[j][e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (int32_t)((uint32_t)v[e] + (uint32_t)b[e]);
    if (a.acc_out) *(i32x4_t*)(a.acc_out + idx) = v;
    uint32_t o[2];
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      float dq[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int dc = a.dq_per_tensor ? 0 : col + e + h;
        dq[h] = a.dq_bf16 ? bf16_bits_to_f32(((const uint16_t*)a.dq)[dc]) : ((const float*)a.dq)[dc];
      }
      float y0 = (float)v[e] * dq[0] * pt, y1 = (float)v[e + 1] * dq[1] * pt;
      if (x3) {
        const uint32_t xw = xv[e >> 1];
        y0 += OUT_BF16 ? bf16_bits_to_f32(xw & 0xffffu) : f16_bits_to_f32(xw & 0xffffu);
        y1 += OUT_BF16 ? bf16_bits_to_f32(xw >> 16) : f16_bits_to_f32(xw >> 16);
      }
      o[e >> 1] = (uint32_t)(OUT_BF16 ? f32_to_bf16_rne(y0) : f32_to_f16_rne(y0)) |
                  ((uint32_t)(OUT_BF16 ? f32_to_bf16_rne(y1) : f32_to_f16_rne(y1)) << 16);
    }
    *(u32x2_t*)(out + idx) = u32x2_t{o[0], o[1]};
  }
}

}  // namespace

hipError_t launch_qm_gemm(const QmArgs& a0, hipStream_t stream) {
  QmArgs a = a0;
  // 2 x 4 waves of 128 x 64 (two per SIMD), a 256 x 256 tile, or with the planner's shorter
  // tile rows (qm_gemm_tile_m: short m, or short split chunks) 2 x 4 waves of 64 x 64, a
  // 128 x 256 tile, or 2 x 2 waves of 32 x 128, a 64 x 256 tile (its x1 stage is one 16-row
  // block per wave; its 80 KiB of LDS let two workgroups share a CU)
  const int bm = a.bm;
  a.tiles_m = (int)((a.m + bm - 1) / bm);
  a.tiles_n = (a.n + kBN - 1) / kBN;
  a.xcd_rm = xcd_region_rows(a.tiles_m, a.tiles_n, (double)bm * a.kchunk, (double)kBN * a.kchunk);
  void (*kern)(const QmArgs);
  if (a.x2p) {  // packed weights
    if (bm == 64)
      kern = a.out_bf16 ? qm_gemm_kernel<true, 2, 2, false, 64, true> : qm_gemm_kernel<false, 2, 2, false, 64, true>;
    else if (bm == 128)
      kern = a.out_bf16 ? qm_gemm_kernel<true, 2, 4, false, 128, true> : qm_gemm_kernel<false, 2, 4, false, 128, true>;
    else
      kern = a.out_bf16 ? qm_gemm_kernel<true, 2, 4, false, 256, true> : qm_gemm_kernel<false, 2, 4, false, 256, true>;
  } else if (bm == 64)
    kern = a.x2t ? (a.out_bf16 ? qm_gemm_kernel<true, 2, 2, true, 64> : qm_gemm_kernel<false, 2, 2, true, 64>)
                 : (a.out_bf16 ? qm_gemm_kernel<true, 2, 2, false, 64> : qm_gemm_kernel<false, 2, 2, false, 64>);
  else if (bm == 128)
    kern = a.x2t ? (a.out_bf16 ? qm_gemm_kernel<true, 2, 4, true, 128> : qm_gemm_kernel<false, 2, 4, true, 128>)
                 : (a.out_bf16 ? qm_gemm_kernel<true, 2, 4, false, 128> : qm_gemm_kernel<false, 2, 4, false, 128>);
  else
    kern = a.x2t ? (a.out_bf16 ? qm_gemm_kernel<true, 2, 4, true> : qm_gemm_kernel<false, 2, 4, true>)
                 : (a.out_bf16 ? qm_gemm_kernel<true, 2, 4, false> : qm_gemm_kernel<false, 2, 4, false>);
  const int threads = bm == 64 ? 256 : 512;
  const int kLds = bm == 64 ? qm_lds<64>() : bm == 128 ? qm_lds<128>() : qm_lds<256>();
  hipError_t e = raise_lds_limit((const void*)kern, kLds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
  const int splits = a.splits > 1 ? a.splits : 1;
  e = launch_main((const void*)kern, dim3((unsigned)blocks, (unsigned)splits), dim3(threads), (size_t)kLds, stream, &a);
  if (e != hipSuccess) return e;
  if (splits == 1) return hipSuccess;
  const int64_t quads = a.m * (a.n / 4);
  const int64_t fblocks = std::max<int64_t>(1, std::min<int64_t>((quads + 255) / 256, 8192));
  hipLaunchKernelGGL(a.out_bf16 ? qm_splitk_finish<true> : qm_splitk_finish<false>, dim3((unsigned)fblocks),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace wq

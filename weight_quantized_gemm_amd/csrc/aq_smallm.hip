// Anti-quant matmul for small m (m <= 32): the weight stream dominates, so the kernel is
// shaped for HBM bandwidth rather than for matrix-core reuse.
//
//   out = x1 @ ((x2 + offset) * scale) + bias + x3
// ("CANN ops-transformer ... aclnnWeightQuantMatmulAllReduce 完全指南", section 计算公式),
// evaluated in the same factored form as the large-m kernel (aq_gemm.h).
//
// Work split: a workgroup owns a 128-column slab of x2 and a contiguous k range (split-k).
// Its 8 waves (two per SIMD, so that one wave's LDS, matrix-core and VALU latencies hide
// behind the other's work) take the range's 64-row blocks round-robin.  Each block --
// weights, the matching 32 x 64 slice of x1 (full 128-byte rows) and, per-group, the scale
// / offset rows of its two 32-row halves -- streams into the wave's own LDS stage by
// direct-to-LDS loads (no barriers; vmcnt waits only).  The wave copies the block into
// registers (A fragments by ds_read_b128, B fragments by tr8 transpose reads), hands the
// stage to its next block at once, and then converts the codes to exact 16-bit images and
// runs 32x32x16 MFMAs while that block streams in.  Row sums of x1 come from the A
// fragments (v_dot2).  Per-group parameters are applied at each group end and at each
// block end: the fold is linear in the accumulators and row sums, so a group split between
// waves or workgroups is folded piecewise with its own scale and offset.  The 8 waves are
// reduced through LDS in a fixed order and the splits by a finishing kernel in a fixed
// order: results are deterministic.
#include "wq_kernels.h"
#include "wq_pipeline.h"

namespace wq {
namespace {

constexpr int kWaves = kSmWaves;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlab = kSmSlab;  // logical columns per workgroup
constexpr int kRows = kSmRows;  // k rows per block, a wave's unit of work

template <bool W4, bool GROUPED>
struct SmTile {
  static constexpr int RB = W4 ? kSlab / 2 : kSlab;   // weight bytes per k row
  // transposed weights: per column a row of the block's 64 k (int4: 32 bytes)
  static constexpr int RowT = W4 ? kRows / 2 : kRows;
  static constexpr int ColsPerKB = 1024 / RowT;
  static constexpr int Wbytes = kRows * RB;           // 8 or 4 KiB
  static constexpr int Xbytes = 32 * kRows * 2;       // 4 KiB of x1 (32 rows x 64 k)
  static constexpr int Pbytes = GROUPED ? 1024 : 0;   // scale / offset rows of the block's groups
  static constexpr int Stage = Wbytes + Xbytes + Pbytes;  // one per wave
  static constexpr int WDma = Wbytes / 1024;
  static constexpr int XDma = Xbytes / 1024;
  static constexpr int RedPitch = 36;                 // floats per column (32 rows + bank pad)
  static constexpr int Red = kWaves * kSlab * RedPitch * 4;  // column-major wave reduction
  static constexpr int Body = kWaves * Stage > Red ? kWaves * Stage : Red;
  static constexpr int GOff = Body;                   // per-wave group row-sum scratch
  static constexpr int SOff = GOff + kWaves * 32 * 4; // per-wave row sums (per-channel)
  static constexpr int Lds = SOff + kWaves * 32 * 4;
  static_assert(Lds <= 160 * 1024, "one workgroup per CU");
};

// XT: the weights are stored transposed, (n, k) (int4: (n, k/2) bytes packed along k).
// PK: the weights are in the packed layout (wq_prepack_weight): a block's four 32-column
// pieces are adjacent 2 KiB runs of B fragments in lane order (int4: two 2 KiB runs, each
// holding two pieces in the low and high nibbles), so the whole block is one contiguous DMA
// and each fragment read one contiguous 8-byte LDS read.
template <bool BF16, int WF, bool GROUPED, bool XT, bool PK = false>
__global__ __launch_bounds__(kThreads, 1) void aq_smallm_kernel(const AqArgs a) {
  constexpr bool W4 = WF == kWInt4;
  using T = SmTile<W4, GROUPED>;
  constexpr int RB = T::RB;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * kSlab, split = blockIdx.y;
  const int K = a.k, N = a.n, M = (int)a.m;
  const int kbeg = split * a.kchunk;
  const int kend = min(K, kbeg + a.kchunk);
  const int nblocks = kend > kbeg ? (kend - kbeg + kRows - 1) / kRows : 0;
  // this wave's blocks: wave, wave + 8, ... of the workgroup's k range
  const int nb = wave < nblocks ? (nblocks - wave + kWaves - 1) / kWaves : 0;
  auto block_k0 = [&](int t) { return kbeg + (wave + kWaves * t) * kRows; };

  // bytes per weight row: a k row of n codes, or (transposed) a column row of k codes
  const int64_t x2_pitch = XT ? (W4 ? (K >> 1) : K) : (W4 ? (N >> 1) : N);
  const int nb0 = W4 ? n0 / 2 : n0;
  uint8_t* const st = smem + wave * T::Stage;  // the wave's one LDS stage

  // per-lane DMA offsets inside a block
  uint32_t w_off[T::WDma];
  int w_k[T::WDma];  // transposed weights: first k (within the block) of this lane's chunk
  constexpr int kPkBlock = W4 ? 1024 : 2048;     // packed: bytes of a 64 k x 32 column block
#pragma unroll
  for (int j = 0; j < T::WDma; ++j) {
    if constexpr (PK) {
      w_k[j] = 0;
      w_off[j] = 1024u * (uint32_t)j + 16u * (uint32_t)lane;
    } else if constexpr (XT) {
      constexpr int L = T::RowT / 16;
      const int r = T::ColsPerKB * j + lane / L;
      const int c = row_slot<T::RowT>(r, lane % L);
      w_k[j] = W4 ? 32 * c : 16 * c;
      w_off[j] = (uint32_t)(r * x2_pitch + 16 * c);
    } else {
      const int r = (1024 / RB) * j + lane / (RB / 16);
      const int p = lane % (RB / 16);
      w_k[j] = 0;
      w_off[j] = (uint32_t)(r * x2_pitch + 16 * (2 * pair_slot<RB>(r, p >> 1) + (p & 1)));
    }
  }
  uint32_t x_off[T::XDma];
  int x_k[T::XDma];  // first k (within the block) of the x1 chunk this lane loads
#pragma unroll
  for (int j = 0; j < T::XDma; ++j) {
    const int r = 8 * j + (lane >> 3);
    const int c = row_slot<128>(r, lane & 7);
    x_k[j] = 8 * c;
    x_off[j] = (uint32_t)(r * K * 2 + 16 * c);
  }
  const bool has_offset = a.offset != nullptr;
  u32x4_t rsc{}, rof{};
  if constexpr (GROUPED) {
    const int64_t pbytes = ((int64_t)a.groups * N - n0) * 2;
    rsc = make_rsrc((const uint8_t*)a.scale + 2 * (int64_t)n0, pbytes);
    rof = has_offset ? make_rsrc((const uint8_t*)a.offset + 2 * (int64_t)n0, pbytes) : rsc;
  }
  auto issue = [&](int t) {
    const int k0 = block_k0(t);
    if constexpr (PK) {
      // the slab's four column blocks of 64-k block k0 / 64, side by side; blocks past n
      // read zero, and so do codes past k (the packed layout pads them with zeros)
      const int nbl = N / 32, nbt = n0 / 32;
      const int valid = nbl - nbt < kSlab / 32 ? nbl - nbt : kSlab / 32;
      const u32x4_t rw = make_rsrc((const uint8_t*)a.x2 + ((int64_t)(k0 / kRows) * nbl + nbt) * kPkBlock,
                                   (int64_t)valid * kPkBlock);
#pragma unroll
      for (int j = 0; j < T::WDma; ++j) dma16(rw, st + 1024 * j, w_off[j]);
    } else if constexpr (XT) {
      // the slab's column rows from k0 on; k >= kend (the split's end) is masked per chunk
      const int64_t kb = W4 ? k0 / 2 : k0;
      const int cols = N - n0 < kSlab ? N - n0 : kSlab;
      const u32x4_t rw = make_rsrc((const uint8_t*)a.x2 + (int64_t)n0 * x2_pitch + kb,
                                   (int64_t)cols * x2_pitch - kb);
#pragma unroll
      for (int j = 0; j < T::WDma; ++j) dma16(rw, st + 1024 * j, k0 + w_k[j] < kend ? w_off[j] : kOOB);
    } else {
      const u32x4_t rw = make_rsrc((const uint8_t*)a.x2 + (int64_t)k0 * x2_pitch + nb0,
                                   (int64_t)(kend - k0) * x2_pitch - nb0);
#pragma unroll
      for (int j = 0; j < T::WDma; ++j) dma16(rw, st + 1024 * j, w_off[j]);
    }
    // rows >= m lie past the resource; k >= kend (a 32-row tail block) is masked per chunk
    const u32x4_t rx = make_rsrc((const uint8_t*)a.x1 + (int64_t)k0 * 2, (int64_t)M * K * 2 - (int64_t)k0 * 2);
#pragma unroll
    for (int j = 0; j < T::XDma; ++j)
      dma16(rx, st + T::Wbytes + 1024 * j, k0 + x_k[j] < kend ? x_off[j] : kOOB);
    if constexpr (GROUPED) {
      const int ga = min(k0 / a.group, a.groups - 1);
      const int gb = min((k0 + 32) / a.group, a.groups - 1);
      dma_group_params<kSlab>(st + T::Wbytes + T::Xbytes, rsc, rof, has_offset, ga, gb, N, lane);
    }
  };

  f32x16_t acc[4], tot[GROUPED ? 4 : 1];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16_t{};
  if constexpr (GROUPED) {
#pragma unroll
    for (int j = 0; j < 4; ++j) tot[j] = f32x16_t{};
  }
  float ssum = 0.f;  // row sum of x1 (row lane % 32, k half lane / 32)
  // logical column of this lane in block j (int4: byte pair p = j >> 1, parity j & 1)
  auto block_col = [&](int j) -> int {
    if constexpr (W4 && !XT && !PK) return n0 + 64 * (j >> 1) + 2 * (lane & 31) + (j & 1);
    else return n0 + 32 * j + (lane & 31);
  };
  const float cbias = a.code_bias;
  float* gscr = (float*)(smem + T::GOff) + wave * 32;

  // fold the accumulators of the current group with the group's scale / offset values of
  // this lane's four column blocks: tot += s * acc + s * (off - C) * S, S the row sums
  // since the last fold
  auto fold = [&](const uint16_t (&ps)[4], const uint16_t (&po)[4]) {
    const float t = ssum + __shfl_xor(ssum, 32, 64);
    if (lane < 32) gscr[lane] = t;
    ssum = 0.f;
    float s[4], q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sv = act_to_f32<BF16>(ps[j]);
      s[j] = sv;
      q[j] = sv * (act_to_f32<BF16>(po[j]) - cbias);
    }
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const f32x4_t sr = *(const f32x4_t*)(gscr + 8 * rq + 4 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          tot[j][4 * rq + e] = fmaf(s[j], acc[j][4 * rq + e], fmaf(q[j], sr[e], tot[j][4 * rq + e]));
    }
    // acc is not cleared: the next MFMA of each column block starts from a zero operand
  };

  // ------------------------------------------------------------------ stream
  // One block in flight per wave in LDS, one in registers: the wave reads block t out of
  // its stage, hands the stage to block t + 1 at once, then computes on block t while
  // block t + 1 streams in.  Eight waves keep 96-104 KiB in flight per CU.
  if (nb > 0) issue(0);
  for (int t = 0; t < nb; ++t) {
    wave_wait<0>();
    const uint8_t* W = st;
    const uint8_t* X = st + T::Wbytes;
    // B fragment reads per 16-k step: int4 row-major (tr8) and packed reads feed two column
    // blocks each; one-byte codes and transposed int4 (4-byte reads) one block each
    constexpr int kP = (W4 && !XT) ? 2 : 4;
    u32x4_t af[kRows / 16];
    u32x2_t braw[kRows / 16][kP];
#pragma unroll
    for (int kk = 0; kk < kRows / 16; ++kk) {
      const int r = lane & 31;
      af[kk] = *(const u32x4_t*)(X + r * 128 + 16 * row_slot<128>(r, 2 * kk + (lane >> 5)));
      if constexpr (PK) {
#pragma unroll
        for (int p = 0; p < kP; ++p) braw[kk][p] = *(const u32x2_t*)(W + p * 2048 + kk * 512 + 8 * lane);
      } else if constexpr (XT) {
        constexpr int RowT = T::RowT;
        const int c = 2 * kk + (lane >> 5);  // 8-k piece within the column row
#pragma unroll
        for (int p = 0; p < kP; ++p) {
          const int cr = 32 * p + (lane & 31);
          if constexpr (RowT == 64)
            braw[kk][p] = *(const u32x2_t*)(W + cr * RowT + 16 * row_slot<RowT>(cr, c >> 1) + 8 * (c & 1));
          else
            braw[kk][p] = u32x2_t{*(const uint32_t*)(W + cr * RowT + 16 * row_slot<RowT>(cr, c >> 2) + 4 * (c & 3)), 0u};
        }
      } else {
        const int kr = 16 * kk + 8 * (lane >> 5) + ((lane & 15) >> 1);
        const int sub = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
#pragma unroll
        for (int p = 0; p < kP; ++p) braw[kk][p] = lds_read_tr8(W + kr * RB + 32 * pair_slot<RB>(kr, p) + sub);
      }
    }
    // the parameter rows of the block's first (e = 0) and second (e = 1) 32-row halves
    uint16_t ps[2][4], po[2][4];
    if constexpr (GROUPED) {
      const uint16_t* Ps = (const uint16_t*)(X + T::Xbytes);
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int lc = block_col(j) - n0;
          ps[e][j] = Ps[e * kSlab + lc];
          po[e][j] = Ps[2 * kSlab + e * kSlab + lc];
        }
    }
    // the stage's LDS reads have completed (the direct-to-LDS writes land whenever their
    // data returns, so they must not be issued earlier): hand it to the next block
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (t + 1 < nb) issue(t + 1);
    __builtin_amdgcn_sched_barrier(0);
    const int k0 = block_k0(t);
#pragma unroll
    for (int kk = 0; kk < kRows / 16; ++kk) {
      // zero: start each column block's accumulator from a zero operand
      auto step = [&](bool zero) {
#pragma unroll
        for (int p = 0; p < kP; ++p) {
          if constexpr (W4 && XT) {
            acc[p] = mfma32x32x16<BF16>(af[kk], i4x8_k_to_act<BF16>(braw[kk][p][0]), zero ? f32x16_t{} : acc[p]);
          } else if constexpr (W4) {
            u32x4_t ev, od;
            i4_kpairs<BF16>(braw[kk][p], ev, od);
            acc[2 * p] = mfma32x32x16<BF16>(af[kk], ev, zero ? f32x16_t{} : acc[2 * p]);
            acc[2 * p + 1] = mfma32x32x16<BF16>(af[kk], od, zero ? f32x16_t{} : acc[2 * p + 1]);
          } else {
            acc[p] = mfma32x32x16<BF16>(af[kk], w8x8_to_act<BF16, WF>(braw[kk][p]), zero ? f32x16_t{} : acc[p]);
          }
        }
      };
      // Per-group: a fold leaves the accumulators spent, so the MFMAs after one start from
      // zero: at kk = 0 always (a block ends in a fold, and the first starts from zero), at
      // kk = 2 after a fold at kk = 1.  The condition is uniform: one of two code paths runs.
      bool fresh = false;
      if constexpr (GROUPED) fresh = kk == 0 || (kk == 2 && ((k0 + 32) % a.group == 0 || k0 + 32 >= kend));
      if (fresh) step(true);
      else step(false);
#pragma unroll
      for (int q = 0; q < 4; ++q) ssum = dot2_ones<BF16>(af[kk][q], ssum);
      if constexpr (GROUPED) {
        // folds: where a group ends inside the block (group sizes are multiples of 32), and
        // at the block end, after which the wave continues elsewhere in k
        if (kk == 1 && ((k0 + 32) % a.group == 0 || k0 + 32 >= kend)) fold(ps[0], po[0]);
        if (kk == 3 && k0 + 32 < kend) fold(ps[1], po[1]);
      }
    }
  }

  // ------------------------------------------------------------------ wave reduction
  // The eight waves' tiles are staged column-major (32 rows per column, padded): a lane
  // moves its 16 accumulators of a column block as four 16-byte writes, and thread t then
  // sums, in wave order, rows 8*(t/128) .. +7 of column t % 128 with 16-byte reads.
  __syncthreads();  // every wave has left the stream: the stages are free
  constexpr int RP = T::RedPitch;
  float* red = (float*)smem;
  float* sred = (float*)(smem + T::SOff);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int lc = block_col(j) - n0;
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const f32x16_t& v = GROUPED ? tot[j] : acc[j];
      *(f32x4_t*)(red + (wave * kSlab + lc) * RP + 8 * rq + 4 * (lane >> 5)) =
          f32x4_t{v[4 * rq], v[4 * rq + 1], v[4 * rq + 2], v[4 * rq + 3]};
    }
  }
  if constexpr (!GROUPED) {
    const float t = ssum + __shfl_xor(ssum, 32, 64);
    if (lane < 32) sred[wave * 32 + lane] = t;
  }
  __syncthreads();
  const int c = tid & (kSlab - 1), r0 = 8 * (tid >> 7);
  const int gcol = n0 + c;
  const bool col_ok = gcol < N;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const f32x4_t lo = *(const f32x4_t*)(red + (w * kSlab + c) * RP + r0);
    const f32x4_t hi = *(const f32x4_t*)(red + (w * kSlab + c) * RP + r0 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] += lo[i];
      v[4 + i] += hi[i];
    }
  }
  float srow[8];  // per-channel: this workgroup's row sums of rows r0 .. r0 + 7
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    srow[i] = 0.f;
    if constexpr (!GROUPED) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) srow[i] += sred[w * 32 + r0 + i];
    }
  }

  // ------------------------------------------------------------------ split-k
  // With several k splits every workgroup writes its partial sums (and, per-channel, its
  // row sums); the finishing kernel adds the splits in split order and writes the output.
  const int S = a.splits;
  if (S > 1) {
    float* part = a.partial + (int64_t)split * a.m * N;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (r0 + i < M && col_ok) part[(int64_t)(r0 + i) * N + gcol] = v[i];
    if constexpr (!GROUPED) {
      if (c == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (r0 + i < M) a.rowsum_part[(int64_t)split * a.m + r0 + i] = srow[i];
      }
    }
    return;
  }

  // ------------------------------------------------------------------ output (one split)
  // out = [s*P + s*(off-C)*S] (per-tensor / per-channel) or T (per-group), + bias + x3
  if (!col_ok) return;
  float cs = 1.f, cq = 0.f;
  if constexpr (!GROUPED) {
    const uint16_t* scale = (const uint16_t*)a.scale;
    const uint16_t* offset = (const uint16_t*)a.offset;
    const int pc = a.per_tensor ? 0 : gcol;
    cs = act_to_f32<BF16>(scale[pc]);
    cq = cs * ((offset ? act_to_f32<BF16>(offset[pc]) : 0.f) - cbias);
  }
  const float cb = a.bias ? act_to_f32<BF16>(((const uint16_t*)a.bias)[gcol]) : 0.f;
  const uint16_t* x3 = (const uint16_t*)a.x3;
  uint16_t* out = (uint16_t*)a.out;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r0 + i;
    if (row >= M) continue;
    const int64_t idx = (int64_t)row * N + gcol;
    float y = GROUPED ? v[i] : fmaf(cs, v[i], cq * srow[i]);
    y += cb;
    if (x3) y += act_to_f32<BF16>(x3[idx]);
    out[idx] = f32_to_act<BF16>(y);
  }
}

// Split-k finish, for this kernel and for the large-m kernel (aq_gemm.h):
// out = [s*P + s*(off-C)*S] (per-tensor / per-channel) or T (per-group), + bias + x3, where
// P / T and S are the sums of the split partials in split order.  A thread handles four
// consecutive columns of one row (n is a multiple of 32).  The kernel streams the partials
// (8 x 4 MiB at m = 128, n = 8192), so its loads are issued ahead of their use: the
// partials four splits at a time, at clamped split indices so that no load waits behind a
// branch, and the other operands before the first partial.
template <bool BF16, bool GROUPED>
__global__ __launch_bounds__(256) void aq_splitk_finish(const AqArgs a) {
  const int N = a.n, S = a.splits;
  const int64_t quads = a.m * (N / 4);
  const int64_t plane = a.m * N;
  const uint16_t* scale = (const uint16_t*)a.scale;
  const uint16_t* offset = (const uint16_t*)a.offset;
  const uint16_t* bias = (const uint16_t*)a.bias;
  const uint16_t* x3 = (const uint16_t*)a.x3;
  uint16_t* out = (uint16_t*)a.out;
  auto half = [](const u32x2_t& w, int e) { return (uint16_t)(w[e >> 1] >> (16 * (e & 1))); };
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = q / (N / 4);
    const int col = 4 * (int)(q - row * (N / 4));
    const int64_t idx = row * N + col;
    const u32x2_t xv = x3 ? *(const u32x2_t*)(x3 + idx) : u32x2_t{0u, 0u};
    const u32x2_t bv = bias ? *(const u32x2_t*)(bias + col) : u32x2_t{0u, 0u};
    u32x2_t sv{0u, 0u}, ov{0u, 0u};
    if constexpr (!GROUPED) {
      if (a.per_tensor) {
        const uint32_t s1 = scale[0], o1 = offset ? offset[0] : 0u;
        sv = u32x2_t{s1 | (s1 << 16), s1 | (s1 << 16)};
        ov = u32x2_t{o1 | (o1 << 16), o1 | (o1 << 16)};
      } else {
        sv = *(const u32x2_t*)(scale + col);
        if (offset) ov = *(const u32x2_t*)(offset + col);
      }
    }
    f32x4_t v = *(const f32x4_t*)(a.partial + idx);
    float srow = 0.f;
    if constexpr (!GROUPED) srow = a.rowsum_part[row];
    for (int s0 = 1; s0 < S; s0 += 4) {
      f32x4_t p[4];
      float r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int sj = min(s0 + j, S - 1);
        p[j] = *(const f32x4_t*)(a.partial + (int64_t)sj * plane + idx);
        if constexpr (!GROUPED) r[j] = a.rowsum_part[(int64_t)sj * a.m + row];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (s0 + j < S) {
          v[0] += p[j][0]; v[1] += p[j][1]; v[2] += p[j][2]; v[3] += p[j][3];
          if constexpr (!GROUPED) srow += r[j];
        }
      }
    }
    float y[4] = {v[0], v[1], v[2], v[3]};
    if constexpr (!GROUPED) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float s = act_to_f32<BF16>(half(sv, e));
        const float o = offset ? act_to_f32<BF16>(half(ov, e)) : 0.f;
        y[e] = fmaf(s, y[e], s * (o - a.code_bias) * srow);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (bias) y[e] += act_to_f32<BF16>(half(bv, e));
      if (x3) y[e] += act_to_f32<BF16>(half(xv, e));
    }
    *(u32x2_t*)(out + idx) = u32x2_t{(uint32_t)f32_to_act<BF16>(y[0]) | ((uint32_t)f32_to_act<BF16>(y[1]) << 16),
                                     (uint32_t)f32_to_act<BF16>(y[2]) | ((uint32_t)f32_to_act<BF16>(y[3]) << 16)};
  }
}

template <bool BF16, int WF, bool GROUPED>
hipError_t launch_sm(const AqArgs& a, hipStream_t stream) {
  using T = SmTile<WF == kWInt4, GROUPED>;
  const int slabs = (a.n + kSlab - 1) / kSlab;
  auto kern = a.x2p ? aq_smallm_kernel<BF16, WF, GROUPED, false, true>
            : a.x2t ? aq_smallm_kernel<BF16, WF, GROUPED, true> : aq_smallm_kernel<BF16, WF, GROUPED, false>;
  hipError_t e = raise_lds_limit((const void*)kern, T::Lds);
  if (e != hipSuccess) return e;
  AqArgs args = a;
  e = launch_main((const void*)kern, dim3(slabs, a.splits), dim3(kThreads), (size_t)T::Lds, stream, &args);
  if (e != hipSuccess) return e;
  if (a.splits == 1) return hipSuccess;  // the kernel wrote the output
  return launch_aq_splitk_finish(a, stream);
}

}  // namespace

hipError_t launch_aq_splitk_finish(const AqArgs& a, hipStream_t stream) {
  const int64_t quads = a.m * (a.n / 4);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((quads + 255) / 256, 8192));
  auto kern = a.bf16 ? (a.grouped ? aq_splitk_finish<true, true> : aq_splitk_finish<true, false>)
                     : (a.grouped ? aq_splitk_finish<false, true> : aq_splitk_finish<false, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_aq_smallm(const AqArgs& a, hipStream_t stream) {
  // FLOAT8_E4M3FN weights come per-channel only
  if (a.f8) return a.bf16 ? launch_sm<true, kWFp8, false>(a, stream) : launch_sm<false, kWFp8, false>(a, stream);
  if (a.bf16) {
    if (a.w4) return a.grouped ? launch_sm<true, kWInt4, true>(a, stream) : launch_sm<true, kWInt4, false>(a, stream);
    return a.grouped ? launch_sm<true, kWInt8, true>(a, stream) : launch_sm<true, kWInt8, false>(a, stream);
  }
  if (a.w4) return a.grouped ? launch_sm<false, kWInt4, true>(a, stream) : launch_sm<false, kWInt4, false>(a, stream);
  return a.grouped ? launch_sm<false, kWInt8, true>(a, stream) : launch_sm<false, kWInt8, false>(a, stream);
}

}  // namespace wq

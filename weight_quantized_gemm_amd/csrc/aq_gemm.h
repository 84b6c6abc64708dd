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
// C is the constant bias of the fed weight images (136 for bf16/int4, 0 otherwise).  The
// matrix cores see only exact 16-bit images of the weight codes (int8, int4 or
// FLOAT8_E4M3FN, all exact in fp16 and bf16) and x1; scale and offset
// are applied in fp32 on the accumulators, or once in the epilogue for per-tensor /
// per-channel parameters.  Per-channel S is summed in-kernel from the x1 fragments (v_dot2
// against ones), each row by one wave.  Per group, the scale part is folded at each group
// end (tot += s * acc), with the group's scale row travelling with the weight tile of the
// k-step in which the group ends, so a fold reads it from LDS and never waits on a global
// load (which would also wait for every stage in flight).  The offset part,
// sum_g s[g,n] * (off[g,n] - C) * S_g[m], is a product of depth G between the per-group row
// sums of x1 and the parameter rows: it runs once per tile after the k loop, on the matrix
// cores in fp32.  The S_g come from a pass before the product (group_rowsums_kernel,
// aq_prep.hip): summed in the k-loop they cost every wave of a row band the same work,
// about a sixth of the kernel's time.
//
// Pipeline: GM x GN waves, wave tile (32*WM) x (32*WN), workgroup tile (32*WM*GM) x (32*WN*GN),
// BK = 64.  Operands travel global -> LDS by direct-to-LDS buffer loads
// (no registers, out-of-range lanes read zero) through 3 to 6 LDS stages (as many as fit),
// one barrier per k-step; every k-step issues a full stage of loads, those past the k range
// from empty resources, so that the loop needs no branches around them.  x1 tiles are row-major with a 16-byte-chunk XOR swizzle and are read as MFMA A
// fragments by ds_read_b128.  Weight tiles stay raw (one-byte codes or packed int4, n-contiguous,
// 32-byte-pair XOR swizzle); B fragments come from ds_read_b64_tr_b8 (8 consecutive k of
// one column per lane) and are turned into exact 16-bit images in registers.  The
// epilogue stages fp32 results through LDS so that x3, bias and the output move in
// 16-byte row-contiguous accesses.
//
// Split k: when the output tiles alone would leave CUs idle, the grid's y index is a k
// split; each split runs the same pipeline over its k range (whole groups, per-group) and
// writes its fp32 tile (per-group: the folded total) and, per-tensor / per-channel, its
// partial row sums; aq_splitk_finish adds the splits in split order and applies the
// parameters, bias and x3.
//
// This header holds the kernel templates; aq_gemm_int8.hip, aq_gemm_int4.hip and
// aq_gemm_fp8.hip instantiate them, one weight format per translation unit.
#pragma once
#include <type_traits>

#include "wq_kernels.h"
#include "wq_pipeline.h"

namespace wq {
namespace {

constexpr int kBK = 64;
constexpr int kArow = 128;                 // bytes per x1 row in a stage (64 x 16-bit)

// XT: the weights are stored transposed, (n, k) (int4: (n, k/2) bytes packed along k).
// PK: the weights are in the packed layout (wq_prepack_weight): 64 k x 32 column blocks in
// MFMA B-fragment order, int4 blocks in pairs that share each byte.
template <bool W4, int GM, int GN, int WM, int WN, bool GROUPED, bool XT = false, bool PK = false>
struct Tile {
  static constexpr int Waves = GM * GN;              // wave grid GM x GN
  static constexpr int Threads = 64 * Waves;
  static constexpr int BM = 32 * WM * GM;            // rows of the workgroup tile
  static constexpr int Abytes = BM * kArow;          // x1 stage
  static constexpr int BN = 32 * WN * GN;            // logical columns
  static constexpr int RB = W4 ? BN / 2 : BN;        // weight bytes per k row
  static constexpr int Bbytes = kBK * RB;
  // per-group scale and offset rows of the two groups a k-step can close
  static constexpr int Pbytes = GROUPED ? (BN > 128 ? 2048 : 1024) : 0;
  static constexpr int Stage = Abytes + Bbytes + Pbytes;
  static constexpr int Win = 256 / RB;               // k rows per 256-byte bank window
  static constexpr int PairMask = 8 / Win - 1;       // swizzle span of 32-byte pairs
  static constexpr int RowsPerKB = 1024 / RB;        // k rows per 1 KiB DMA block
  // transposed weights: per column a row of the stage's 64 k (64 bytes, int4 32 bytes)
  static constexpr int RowT = W4 ? kBK / 2 : kBK;
  static constexpr int ColsPerKB = 1024 / RowT;      // columns per 1 KiB DMA block
  static constexpr int Ablocks = Abytes / 1024;      // 1 KiB DMA blocks of x1
  static constexpr int Bblocks = Bbytes / 1024;      // DMA blocks per stage (weights)
  static constexpr int Aper = Ablocks / Waves;
  // weights: Bblocks spread over the first Bblocks waves when there are fewer blocks
  static constexpr int Bper = Bblocks >= Waves ? Bblocks / Waves : 1;
  static constexpr int Bwaves = Bblocks >= Waves ? Waves : Bblocks;
  static constexpr int Pwave = Waves - 1;            // issues the group-parameter loads
  static constexpr int WCols = 32 * WN;              // logical columns per wave
  static constexpr bool XTile = XT;
  static constexpr bool PKed = PK;
  // packed weights: bytes of a 64 k x 32 column block; a B fragment read takes 8 bytes per
  // lane from a 2048-byte unit (a block of one-byte codes, a pair of int4 blocks)
  static constexpr int PkBlock = W4 ? 1024 : 2048;
  // B fragment reads per wave per 16-k step: int4 row-major (tr8) and packed reads feed two
  // blocks each; one-byte codes and transposed int4 (4-byte reads) one block each
  static constexpr int Reads = (W4 && !XT) ? WN / 2 : WN;
  // LDS layout: stages (x1 | weights | group scale / offset rows) | per-channel S rows
  // (BM fp32).  As many stages as fit (3 to 6): a deeper pipeline hides more load
  // latency where a stage is small.
  static constexpr int Extra = BM * 4;
  static constexpr int FitStages = (160 * 1024 - Extra) / Stage;
  static constexpr int Stages = FitStages > 6 ? 6 : FitStages;
  static constexpr int SOff = Stages * Stage;
  static constexpr int Total = SOff + BM * 4;
  static_assert(Stages >= 3, "at least three stages");
  static_assert(BM == 64 || BM == 128 || BM == 256, "x1 stage holds 64, 128 or 256 rows");
  static_assert(Ablocks % Waves == 0, "x1 DMA blocks split evenly over the waves");
  static_assert(Bblocks % Waves == 0 || Bblocks < Waves, "weight DMA blocks split");
  static_assert(Win >= 1 && Win <= 4, "weight row bytes 64..256");
  static_assert(!W4 || XT || WN % 2 == 0, "an int4 read feeds an even and an odd block");
  static_assert(!(XT && PK), "one weight layout");
};

// One 16-k step of MFMA operands for a wave: WM x1 fragments (16-byte reads) and the raw
// weight bytes of its tr8 reads.
template <int WM, int R>
struct Frag {
  u32x4_t a[WM];
  u32x2_t raw[R];
};

template <class T, int WM>
__device__ __forceinline__ void load_frag(const uint8_t* As, const uint8_t* Bs, int kk, int wm, int wn,
                                          int lane, Frag<WM, T::Reads>& f) {
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int r = wm * (32 * WM) + 32 * i + (lane & 31);
    const int c = 2 * kk + (lane >> 5);
    f.a[i] = *(const u32x4_t*)(As + r * kArow + 16 * row_slot<kArow>(r, c));
  }
  if constexpr (T::PKed) {
    // the stage holds the tile's 2048-byte units of one 64-k block side by side; the codes
    // of 16-k step kk of unit u are lane-ordered, 8 bytes a lane, at u * 2048 + kk * 512
#pragma unroll
    for (int j = 0; j < T::Reads; ++j)
      f.raw[j] = *(const u32x2_t*)(Bs + (wn * T::Reads + j) * 2048 + kk * 512 + 8 * lane);
    return;
  }
  if constexpr (T::XTile) {
    // column row r holds the stage's k for one column, 16-byte chunks swizzled like x1
    // rows; lane half h = lane / 32 takes k 16 kk + 8 h .. + 7
    constexpr int RowT = T::RowT;
    const int c = 2 * kk + (lane >> 5);  // 8-k piece within the row
#pragma unroll
    for (int j = 0; j < T::Reads; ++j) {
      const int r = wn * T::WCols + 32 * j + (lane & 31);
      if constexpr (RowT == 64) {        // 8 bytes per piece
        f.raw[j] = *(const u32x2_t*)(Bs + r * RowT + 16 * row_slot<RowT>(r, c >> 1) + 8 * (c & 1));
      } else {                           // int4: 4 bytes per piece
        f.raw[j] = u32x2_t{*(const uint32_t*)(Bs + r * RowT + 16 * row_slot<RowT>(r, c >> 2) + 4 * (c & 3)), 0u};
      }
    }
    return;
  }
  const int kr = 16 * kk + 8 * (lane >> 5) + ((lane & 15) >> 1);
#pragma unroll
  for (int j = 0; j < T::Reads; ++j) {
    const int pair = wn * T::Reads + j;  // 32-byte pair within the weight row
    const int off = kr * T::RB + 32 * pair_slot<T::RB>(kr, pair) + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
    f.raw[j] = lds_read_tr8(Bs + off);
  }
}

// The kernel body, specialised on the wave's column index WNI in the GM x GN wave grid:
// column offsets and the per-channel row-sum block become compile-time constants.
template <bool BF16, int WF, int GM, int GN, int WM, int WN, bool GROUPED, bool XT, bool PK, int WNI>
__device__ __forceinline__ void aq_gemm_body(const AqArgs& a, uint8_t* smem, int wave) {
  constexpr bool W4 = WF == kWInt4;
  using T = Tile<W4, GM, GN, WM, WN, GROUPED, XT, PK>;
  constexpr int BN = T::BN, RB = T::RB, WC = T::WCols;
  const int lane = threadIdx.x & 63;
  const int wm = wave / GN;
  constexpr int wn = WNI;
  int tm, tn;
  tile_of(blockIdx.x, a.tiles_m, a.tiles_n, a.xcd_rm, tm, tn);
  const int64_t m0 = (int64_t)tm * T::BM;
  const int n0 = tn * BN;
  const int64_t M = a.m;
  const int K = a.k, N = a.n;
  // bytes per weight row: a k row of n codes, or (transposed) a column row of k codes
  const int64_t x2_pitch = XT ? (W4 ? (K >> 1) : K) : (W4 ? (N >> 1) : N);
  // split k: this workgroup's k range.  Split starts are multiples of 64, and per-group of
  // the group size too, so a split holds whole groups and only the last one has a tail.
  const int split = blockIdx.y;
  const int kbeg = split * a.kchunk;
  const int kend = a.splits > 1 ? min(K, kbeg + a.kchunk) : K;
  const int klen = kend - kbeg;
  const int nk = (klen + kBK - 1) / kBK;

  // ---------------------------------------------------------------- DMA issue
  // x1: wave w fills 1 KiB blocks b = w + Waves*j (8 rows each); lane -> (row, physical
  // slot).  The per-lane byte offsets inside a stage do not depend on k: they are formed
  // once, and each k-step only moves the (scalar) buffer base.
  const uint8_t* x1b = (const uint8_t*)a.x1 + m0 * K * 2;
  // bytes of x1 from the tile's first row on that the tile may read (at most BM rows)
  const uint32_t x1_bytes = (uint32_t)((M - m0 < T::BM ? M - m0 : T::BM) * K * 2);
  const int nb0 = W4 ? n0 / 2 : n0;
  const uint8_t* x2b = (const uint8_t*)a.x2 + (XT ? (int64_t)n0 * x2_pitch : (int64_t)nb0);
  // transposed weights: bytes from the tile's first column row on that the tile may read
  const uint32_t x2t_bytes = (uint32_t)((N - n0 < BN ? N - n0 : BN) * x2_pitch);
  uint32_t a_off[T::Aper];
  int a_k[T::Aper];  // first k (within the stage) of the chunk this lane loads
#pragma unroll
  for (int j = 0; j < T::Aper; ++j) {
    const int b = wave + T::Waves * j;
    const int r = 8 * b + (lane >> 3);
    const int c = row_slot<kArow>(r, lane & 7);  // logical chunk held by this physical slot
    a_k[j] = 8 * c;
    a_off[j] = (uint32_t)(r * K * 2 + 16 * c);
  }
  uint32_t b_off[T::Bper];
  int b_k[T::Bper];  // transposed weights: first k (within the stage) of the chunk this lane loads
#pragma unroll
  for (int j = 0; j < T::Bper; ++j) {
    const int b = wave + T::Waves * j;
    if constexpr (PK) {                // the stage's blocks are one contiguous run
      b_k[j] = 0;
      b_off[j] = 1024u * (uint32_t)b + 16u * (uint32_t)lane;
    } else if constexpr (XT) {
      constexpr int L = T::RowT / 16;  // 16-byte chunks per column row
      const int r = T::ColsPerKB * b + lane / L;
      const int c = row_slot<T::RowT>(r, lane % L);
      b_k[j] = W4 ? 32 * c : 16 * c;
      b_off[j] = (uint32_t)(r * x2_pitch + 16 * c);
    } else {
      const int r = T::RowsPerKB * b + lane / (RB / 16);
      const int p = lane % (RB / 16);
      b_k[j] = 0;
      b_off[j] = (uint32_t)(r * x2_pitch + 16 * (2 * pair_slot<RB>(r, p >> 1) + (p & 1)));
    }
  }
  // per-group parameters: buffer resources over scale / offset from column n0 on
  const bool has_offset = a.offset != nullptr;
  u32x4_t rsc{}, rof{};
  if constexpr (GROUPED) {
    const int64_t pbytes = ((int64_t)a.groups * N - n0) * 2;
    rsc = make_rsrc((const uint8_t*)a.scale + 2 * (int64_t)n0, pbytes);
    rof = has_offset ? make_rsrc((const uint8_t*)a.offset + 2 * (int64_t)n0, pbytes) : rsc;
  }
  // per-group: the precomputed S_g, (groups, m) fp32, read after the k loop
  const float* gsum = a.gsum;
  // loads this wave issues per stage (the parameter wave: 2 parameter-row loads)
  constexpr int kOwnA = T::Aper, kOwnB = T::Bper, kOwnP = GROUPED ? 2 : 0;
  const bool has_b = wave < T::Bwaves, has_p = GROUPED && wave == T::Pwave;

  // The loads of one stage, as items that can be issued separately: x1 blocks j (kind 0),
  // weight blocks j (kind 1) and the group-parameter rows (kind 2).  A stage's resources
  // are formed once by stage_rsrc; the items are then spread over the four 16-k steps of
  // the k-step that issues them, so that the texture unit is not handed a burst of loads
  // that stalls the waves' matrix-core work.
  struct StageRsrc {
    u32x4_t ra, rb;
    uint8_t* st;
    int k0;
    bool tail;
  };
  auto stage_rsrc = [&](int ks) {
    StageRsrc r;
    r.k0 = kbeg + ks * kBK;
    r.st = smem + (ks % T::Stages) * T::Stage;
    // Every k-step issues the loads of the stage S - 1 ahead, also past the split's range:
    // those get empty resources, so they read nothing and write zeros into a stage no wave
    // reads any more.  The loop then has one wait count and no branches around its loads.
    const bool live = ks < nk;
    r.ra = make_rsrc32(x1b + (int64_t)r.k0 * 2, live ? x1_bytes - (uint32_t)r.k0 * 2 : 0u);
    if constexpr (PK) {
      // the tile's column blocks of 64-k block k0 / 64; blocks past n read zero (the
      // packed layout pads k past the end with zero codes)
      const int nbl = N / 32, nbt = n0 / 32;
      const int valid = nbl - nbt < BN / 32 ? nbl - nbt : BN / 32;
      r.rb = make_rsrc((const uint8_t*)a.x2 + ((int64_t)(r.k0 / kBK) * nbl + nbt) * T::PkBlock,
                       live ? (int64_t)valid * T::PkBlock : 0);
    } else if constexpr (XT) {
      const uint32_t kb = W4 ? (uint32_t)r.k0 / 2 : (uint32_t)r.k0;
      r.rb = make_rsrc32(x2b + kb, live ? x2t_bytes - kb : 0u);
    } else {
      const int rows = K - r.k0 < kBK ? K - r.k0 : kBK;
      r.rb = make_rsrc32(x2b + (int64_t)r.k0 * x2_pitch, live ? (uint32_t)(rows * x2_pitch - nb0) : 0u);
    }
    r.tail = r.k0 + kBK > K;  // only the last k-step can reach past k
    return r;
  };
  auto issue_a = [&](const StageRsrc& r, int j) {
    uint8_t* dst = r.st + 1024 * (wave + T::Waves * j);
    dma16(r.ra, dst, (r.tail && r.k0 + a_k[j] >= K) ? kOOB : a_off[j]);
  };
  auto issue_b = [&](const StageRsrc& r, int j) {
    uint8_t* dst = r.st + T::Abytes + 1024 * (wave + T::Waves * j);
    if constexpr (!XT) dma16(r.rb, dst, b_off[j]);
    else dma16(r.rb, dst, (r.tail && r.k0 + b_k[j] >= K) ? kOOB : b_off[j]);  // k past the end reads 0
  };
  auto issue_p = [&](const StageRsrc& r) {
    if constexpr (GROUPED) {
      const int ga = min((r.k0 + 31) / a.group, a.groups - 1);
      const int gb = min((r.k0 + 63) / a.group, a.groups - 1);
      uint8_t* pd = r.st + T::Abytes + T::Bbytes;
      dma_group_params<BN>(pd, rsc, rof, has_offset, ga, gb, N, lane);
    }
  };
  // the items of 16-k step kk: x1 blocks j with j % 4 == kk, weight blocks j with
  // (j + 2) % 4 == kk, the parameter rows at kk == 1
  auto issue_step = [&](const StageRsrc& r, int kk) {
#pragma unroll
    for (int j = 0; j < T::Aper; ++j)
      if (j % 4 == kk) issue_a(r, j);
    if (has_b) {
#pragma unroll
      for (int j = 0; j < T::Bper; ++j)
        if ((j + 2) % 4 == kk) issue_b(r, j);
    }
    if (has_p && kk == 1) issue_p(r);
  };
  auto issue = [&](int ks) {
    const StageRsrc r = stage_rsrc(ks);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) issue_step(r, kk);
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
  // per-channel row sums of x1 (lane half l>>5 of row 32i + l%32 of the wave's band): the
  // GN waves of a row band share its WM i-blocks, wave wn summing blocks
  // wn*SB .. wn*SB + SB - 1
  constexpr int SB = WM / GN > 0 ? WM / GN : 1;  // blocks summed per wave
  static_assert(GROUPED || WM % GN == 0 || GN % WM == 0, "row-sum split");
  float ssum[SB];
#pragma unroll
  for (int i = 0; i < SB; ++i) ssum[i] = 0.f;
  // the wave's first summed block
  constexpr int sb0 = WM >= GN ? wn * SB : (wn < WM ? wn : WM);

  const uint16_t* __restrict__ scale = (const uint16_t*)a.scale;
  const uint16_t* __restrict__ offset = (const uint16_t*)a.offset;
  const float cbias = a.code_bias;
  (void)has_offset;

  // logical column of lane's block j (int4: block 2p + e covers byte pair p, parity e)
  auto block_col = [&](int j) -> int {
    if constexpr (W4 && !XT && !PK) return n0 + wn * WC + 64 * (j >> 1) + 2 * (lane & 31) + (j & 1);
    else return n0 + wn * WC + 32 * j + (lane & 31);
  };

  // fold the group that ends at row 32 (e = 0) or 64 (e = 1) of the k-step whose
  // parameter rows are at Ps: tot += s * acc.  The group's offset term s * (off - C) * S_g is
  // added after the k loop, for all groups at once (offset_product).
  auto rescale = [&](const uint16_t* Ps, int e) {
    float s[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) s[j] = act_to_f32<BF16>(Ps[e * BN + block_col(j) - n0]);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) tot[i][j][r] = fmaf(s[j], acc[i][j][r], tot[i][j][r]);
    // acc is not cleared: the next group's first MFMA starts from zero
  };

  // The offset terms of this split's groups g0 .. g1 - 1, sum_g S_g[row] * q_g[col] with
  // q_g = s_g * (off_g - C): a product of depth g1 - g0 between the precomputed row sums
  // (groups, m) and the parameter rows, on the matrix cores in fp32 (32x32x2 MFMAs, two
  // groups each: lane l holds group g + l / 32 of row or column l % 32), added to tot.
  auto offset_product = [&]() {
    if constexpr (GROUPED) {
      if (!has_offset && cbias == 0.f) return;
      const int g0 = kbeg / a.group;
      const int g1 = min(a.groups, (kend + a.group - 1) / a.group);
      const uint16_t* sp = (const uint16_t*)a.scale;
      const uint16_t* op = (const uint16_t*)a.offset;
      int64_t rows[WM];
#pragma unroll
      for (int i = 0; i < WM; ++i) rows[i] = m0 + wm * (32 * WM) + 32 * i + (lane & 31);
      int cols[WN];
#pragma unroll
      for (int j = 0; j < WN; ++j) cols[j] = block_col(j);
#pragma unroll 4
      for (int g = g0; g < g1; g += 2) {
        const int gl = g + (lane >> 5);
        const bool gv = gl < g1;
        float av[WM], bv[WN];
#pragma unroll
        for (int i = 0; i < WM; ++i) av[i] = (gv && rows[i] < M) ? gsum[(int64_t)gl * M + rows[i]] : 0.f;
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          float q = 0.f;
          if (gv && cols[j] < N) {
            const int64_t pi = (int64_t)gl * N + cols[j];
            const float sv = act_to_f32<BF16>(sp[pi]);
            q = sv * ((has_offset ? act_to_f32<BF16>(op[pi]) : 0.f) - cbias);
          }
          bv[j] = q;
        }
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            tot[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[j], tot[i][j], 0, 0, 0);
      }
    }
  };

  // ---------------------------------------------------------------- epilogue geometry
  // The epilogue moves 8 consecutive columns of one row per lane.  Its x3 rows are
  // prefetched into registers while the last k-step's MFMAs run (two 32-row bands ahead).
  constexpr int EP = WC + 8;            // fp32 pitch of the staging rows (bank spread)
  constexpr int LanesPerRow = WC / 8;
  constexpr int RowsPerPass = 64 / LanesPerRow;
  constexpr int kPasses = 32 / RowsPerPass;
  const int ecol = 8 * (lane % LanesPerRow);
  const int gcol = n0 + wn * WC + ecol;   // first of this lane's 8 output columns
  const bool col_ok = gcol < N;
  // with split k the epilogue writes fp32 partials; x3, bias and the parameters are applied
  // when the splits are added
  const bool split_out = a.splits > 1;
  const uint16_t* __restrict__ x3 = split_out ? nullptr : (const uint16_t*)a.x3;
  // bands of x3 held in registers ahead of use: one where the accumulators leave little room
  constexpr int XP = (!GROUPED && WM * WN >= 8) ? 1 : 2;
  u32x4_t xpre[XP][kPasses];
  auto prefetch_x3 = [&](int i, int slot) {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int er = p * RowsPerPass + lane / LanesPerRow;
      const int64_t grow = m0 + wm * (32 * WM) + 32 * i + er;
      xpre[slot][p] = (x3 && col_ok && grow < M) ? *(const u32x4_t*)(x3 + grow * N + gcol)
                                                 : u32x4_t{0, 0, 0, 0};
    }
  };

  // ---------------------------------------------------------------- main loop
  constexpr int S = T::Stages;
  for (int ks = 0; ks < S - 1; ++ks) issue(ks);
  // The k loop, in two versions: with the per-channel row sums (RS) where the offset term
  // needs them, without where that term is zero (no offset and exact images, C = 0).
  auto k_loop = [&](auto rs_c) {
    constexpr bool RS = decltype(rs_c)::value;
    for (int ks = 0; ks < nk; ++ks) {
      // stage ks is complete once only the S - 2 stages issued after it may still be in flight
      if (has_b && has_p) stage_barrier<(kOwnA + kOwnB + kOwnP) * (S - 2)>();
      else if (has_b) stage_barrier<(kOwnA + kOwnB) * (S - 2)>();
      else if (has_p) stage_barrier<(kOwnA + kOwnP) * (S - 2)>();
      else stage_barrier<kOwnA * (S - 2)>();
      const StageRsrc nr = stage_rsrc(ks + S - 1);
      if (ks == nk - 1) {  // only loads past the range left: start the epilogue's x3 reads
        prefetch_x3(0, 0);
        if (XP > 1 && WM > 1) prefetch_x3(1, 1 % XP);
      }

      const uint8_t* As = smem + (ks % T::Stages) * T::Stage;
      const uint8_t* Bs = As + T::Abytes;
      // Fragments are double-buffered across the four 16-k steps: the reads of step kk + 1
      // are issued before the MFMAs of step kk, so LDS latency hides behind them.
      Frag<WM, T::Reads> f0, f1;
      load_frag<T, WM>(As, Bs, 0, wm, wn, lane, f0);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        Frag<WM, T::Reads>& cur = (kk & 1) ? f1 : f0;
        Frag<WM, T::Reads>& nxt = (kk & 1) ? f0 : f1;
        if (kk < 3) load_frag<T, WM>(As, Bs, kk + 1, wm, wn, lane, nxt);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!GROUPED && RS) {
#pragma unroll
          for (int t = 0; t < SB; ++t) {
            // sb0 is a constant and t an unrolled index: the block is chosen at compile time
            constexpr int kLast = WM - 1;
            const int blk = sb0 + t < WM ? sb0 + t : kLast;
            if (sb0 + t < WM) {
#pragma unroll
              for (int q = 0; q < 4; ++q) ssum[t] = dot2_ones<BF16>(cur.a[blk][q], ssum[t]);
            }
          }
        }
        u32x4_t bfr[WN];
#pragma unroll
        for (int j = 0; j < T::Reads; ++j) {
          if constexpr (W4 && XT) bfr[j] = i4x8_k_to_act<BF16>(cur.raw[j][0]);
          else if constexpr (W4) i4_kpairs<BF16>(cur.raw[j], bfr[2 * j], bfr[2 * j + 1]);
          else bfr[j] = w8x8_to_act<BF16, WF>(cur.raw[j]);
        }
        // Per-group: a group's first 16-k step (group starts fall on multiples of 32, so on
        // steps 0 and 2; k is counted from the split's start, a group boundary) starts its
        // accumulators from zero through the MFMA's own operand instead of clearing them
        // after the previous group's fold.
        bool fresh = false;
        if constexpr (GROUPED) {
          if (kk % 2 == 0) fresh = (ks * kBK + kk * 16) % a.group == 0;
        }
        if (fresh) {
#pragma unroll
          for (int i = 0; i < WM; ++i)
#pragma unroll
            for (int j = 0; j < WN; ++j) acc[i][j] = mfma32x32x16<BF16>(cur.a[i], bfr[j], f32x16_t{});
        } else {
#pragma unroll
          for (int i = 0; i < WM; ++i)
#pragma unroll
            for (int j = 0; j < WN; ++j) acc[i][j] = mfma32x32x16<BF16>(cur.a[i], bfr[j], acc[i][j]);
        }
        issue_step(nr, kk);  // behind this step's matrix-core work

        if constexpr (GROUPED) {
          if (kk & 1) {  // groups end on multiples of 32
            const int kdone = ks * kBK + kk * 16 + 16;
            if (kdone <= klen && (kdone % a.group == 0 || kdone == klen))
              rescale((const uint16_t*)(Bs + T::Bbytes), kk >> 1);
          }
        }
      }
    }
  };
  if constexpr (GROUPED) {
    k_loop(std::false_type{});
  } else {
    if (a.offset != nullptr || cbias != 0.f) k_loop(std::true_type{});
    else k_loop(std::false_type{});  // the row sums stay zero: the term they feed is zero
  }

  offset_product();

  // ---------------------------------------------------------------- epilogue
  wave_wait<0>();   // the loads past the range (zeros) have landed
  __syncthreads();  // every wave is done with the stage buffers
  float* srow = (float*)(smem + T::SOff);
  if constexpr (!GROUPED) {
#pragma unroll
    for (int t = 0; t < SB; ++t) {
      const float v = ssum[t] + __shfl_xor(ssum[t], 32, 64);
      if (lane < 32 && sb0 + t < WM) srow[wm * (32 * WM) + 32 * (sb0 + t) + lane] = v;
    }
    __syncthreads();
    // split k: this split's row sums of the tile's rows, from the first column of tiles
    if (split_out && tn == 0) {
      for (int r = threadIdx.x; r < T::BM; r += T::Threads)
        if (m0 + r < M) a.rowsum_part[(int64_t)split * M + m0 + r] = srow[r];
    }
  }
  float* __restrict__ part = split_out ? a.partial + (int64_t)split * M * N : nullptr;
  // Each wave stages one 32-row band of its tile at a time in its own LDS region, then
  // moves 8 consecutive columns per lane with 16-byte accesses.
  float* E = (float*)smem + wave * (32 * EP);
  const uint16_t* __restrict__ bias = (const uint16_t*)a.bias;
  uint16_t* __restrict__ out = (uint16_t*)a.out;
  // per-column parameters of this lane's 8 columns
  float cs[8], cq[8], cb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { cs[e] = 0.f; cq[e] = 0.f; cb[e] = 0.f; }
  if (col_ok) {
    if (bias) {
      const u32x4_t bv = *(const u32x4_t*)(bias + gcol);
#pragma unroll
      for (int e = 0; e < 8; ++e) cb[e] = act_to_f32<BF16>((uint16_t)(bv[e >> 1] >> (16 * (e & 1))));
    }
    if constexpr (!GROUPED) {
      if (a.per_tensor) {
        const float sv = act_to_f32<BF16>(scale[0]);
        const float ov = offset ? act_to_f32<BF16>(offset[0]) : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) { cs[e] = sv; cq[e] = sv * (ov - cbias); }
      } else {
        const u32x4_t sv = *(const u32x4_t*)(scale + gcol);
        u32x4_t ov = u32x4_t{0, 0, 0, 0};
        if (offset) ov = *(const u32x4_t*)(offset + gcol);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float s = act_to_f32<BF16>((uint16_t)(sv[e >> 1] >> (16 * (e & 1))));
          const float o = offset ? act_to_f32<BF16>((uint16_t)(ov[e >> 1] >> (16 * (e & 1)))) : 0.f;
          cs[e] = s;
          cq[e] = s * (o - cbias);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < WM; ++i) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int lc = block_col(j) - (n0 + wn * WC);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        E[acc_row(r, lane) * EP + lc] = GROUPED ? tot[i][j][r] : acc[i][j][r];
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int er = p * RowsPerPass + lane / LanesPerRow;
      const int64_t grow = m0 + wm * (32 * WM) + 32 * i + er;
      const u32x4_t xv = xpre[i % XP][p];
      const f32x4_t v0 = *(const f32x4_t*)(E + er * EP + ecol);
      const f32x4_t v1 = *(const f32x4_t*)(E + er * EP + ecol + 4);
      if (grow >= M || !col_ok) continue;
      if (split_out) {
        *(f32x4_t*)(part + grow * N + gcol) = v0;
        *(f32x4_t*)(part + grow * N + gcol + 4) = v1;
        continue;
      }
      const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      float sr = 0.f;
      if constexpr (!GROUPED) sr = srow[wm * (32 * WM) + 32 * i + er];
      const int64_t idx = grow * N + gcol;
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float y0 = v[e], y1 = v[e + 1];
        if constexpr (!GROUPED) {
          y0 = fmaf(cs[e], y0, cq[e] * sr);
          y1 = fmaf(cs[e + 1], y1, cq[e + 1] * sr);
        }
        y0 += cb[e];
        y1 += cb[e + 1];
        if (x3) {
          y0 += act_to_f32<BF16>((uint16_t)(xv[e >> 1] & 0xffffu));
          y1 += act_to_f32<BF16>((uint16_t)(xv[e >> 1] >> 16));
        }
        o[e >> 1] = (uint32_t)f32_to_act<BF16>(y0) | ((uint32_t)f32_to_act<BF16>(y1) << 16);
      }
      *(u32x4_t*)(out + idx) = u32x4_t{o[0], o[1], o[2], o[3]};
    }
    if (i + XP < WM) prefetch_x3(i + XP, i % XP);
  }
}

template <bool BF16, int WF, int GM, int GN, int WM, int WN, bool GROUPED, bool XT, bool PK>
__global__ __launch_bounds__(64 * GM * GN, 1) void aq_gemm_kernel(const AqArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
  const int wn = wave % GN;
#define WQ_WAVE_COLUMN(c)                                                      \
  if constexpr (GN > c) {                                                     \
    if (wn == c) {                                                            \
      aq_gemm_body<BF16, WF, GM, GN, WM, WN, GROUPED, XT, PK, c>(a, smem, wave); \
      return;                                                                 \
    }                                                                         \
  }
  WQ_WAVE_COLUMN(0) WQ_WAVE_COLUMN(1) WQ_WAVE_COLUMN(2) WQ_WAVE_COLUMN(3)
  WQ_WAVE_COLUMN(4) WQ_WAVE_COLUMN(5) WQ_WAVE_COLUMN(6) WQ_WAVE_COLUMN(7)
#undef WQ_WAVE_COLUMN
}

template <bool BF16, int WF, int GM, int GN, int WM, int WN, bool GROUPED, bool XT = false, bool PK = false>
hipError_t launch_one(const AqArgs& a0, hipStream_t stream) {
  static_assert(GN <= 8, "wave grids have at most 8 columns");
  using T = Tile<WF == kWInt4, GM, GN, WM, WN, GROUPED, XT, PK>;
  AqArgs a = a0;
  a.tiles_m = (int)((a.m + T::BM - 1) / T::BM);
  a.tiles_n = (a.n + T::BN - 1) / T::BN;
  // operand bytes per tile row (x1) and per tile column (weights) over the k range
  a.xcd_rm = xcd_region_rows(a.tiles_m, a.tiles_n, (double)T::BM * a.kchunk * 2.0,
                             (double)T::BN * a.kchunk * (WF == kWInt4 ? 0.5 : 1.0));
  const size_t lds = (size_t)T::Total;
  auto kern = aq_gemm_kernel<BF16, WF, GM, GN, WM, WN, GROUPED, XT, PK>;
  hipError_t e = raise_lds_limit((const void*)kern, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
  const int splits = a.splits > 1 ? a.splits : 1;
  e = launch_main((const void*)kern, dim3((unsigned)blocks, (unsigned)splits), dim3(T::Threads), lds, stream, &a);
  if (e != hipSuccess) return e;
  return splits > 1 ? launch_aq_splitk_finish(a, stream) : hipSuccess;
}

// Tile configurations (wave grid GM x GN, blocks per wave WM x WN).  The matrix cores and
// the VALU hardly overlap on gfx950, and one wave per SIMD leaves LDS latency exposed, so
// every configuration runs two waves per SIMD.  Per-group tiles are wide in n and short in
// m: the x1 tile (16-bit) costs more load bandwidth per MFMA than the packed weights, and
// the per-group accumulators (current group + folded total) leave room for 64x64 wave
// tiles only.
//   per-tensor / per-channel: 2x4 waves of 128x64 (256x256)
//   per-group:                2x4 waves of 64x64 (128x256)
// The planner's shorter tiles (aq_gemm_tile_m: short m, or short split chunks): 2x4 waves
// of 32x64 (64x256) at 64 rows in every mode, and per-tensor / per-channel 2x4 waves of
// 64x64 (128x256) at 128 rows.
template <bool BF16, int WF>
hipError_t launch_mode(const AqArgs& a, hipStream_t stream) {
  const bool tiny_m = a.bm == 64, short_m = a.bm == 128;
  constexpr bool kGroupedOk = WF != kWFp8;  // FLOAT8_E4M3FN weights come per-channel only
  if (a.x2p) {  // packed weights
    if constexpr (kGroupedOk) {
      if (a.grouped) {
        if (tiny_m) return launch_one<BF16, WF, 2, 4, 1, 2, true, false, true>(a, stream);
        return launch_one<BF16, WF, 2, 4, 2, 2, true, false, true>(a, stream);
      }
    }
    if (tiny_m) return launch_one<BF16, WF, 2, 4, 1, 2, false, false, true>(a, stream);
    if (short_m) return launch_one<BF16, WF, 2, 4, 2, 2, false, false, true>(a, stream);
    return launch_one<BF16, WF, 2, 4, 4, 2, false, false, true>(a, stream);
  }
  if (a.x2t) {  // transposed weights
    if constexpr (kGroupedOk) {
      if (a.grouped) {
        if (tiny_m) return launch_one<BF16, WF, 2, 4, 1, 2, true, true>(a, stream);
        return launch_one<BF16, WF, 2, 4, 2, 2, true, true>(a, stream);
      }
    }
    if (tiny_m) return launch_one<BF16, WF, 2, 4, 1, 2, false, true>(a, stream);
    if (short_m) return launch_one<BF16, WF, 2, 4, 2, 2, false, true>(a, stream);
    return launch_one<BF16, WF, 2, 4, 4, 2, false, true>(a, stream);
  }
  if constexpr (kGroupedOk) {
    if (a.grouped) {
      if (tiny_m) return launch_one<BF16, WF, 2, 4, 1, 2, true>(a, stream);
      return launch_one<BF16, WF, 2, 4, 2, 2, true>(a, stream);
    }
  }
  if (tiny_m) return launch_one<BF16, WF, 2, 4, 1, 2, false>(a, stream);
  if (short_m) return launch_one<BF16, WF, 2, 4, 2, 2, false>(a, stream);
  return launch_one<BF16, WF, 2, 4, 4, 2, false>(a, stream);
}

}  // namespace
}  // namespace wq

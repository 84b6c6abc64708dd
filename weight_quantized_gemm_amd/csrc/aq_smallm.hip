// Anti-quant matmul for small m (m <= 32): the weight stream dominates, so the kernel is
// shaped for HBM bandwidth rather than for matrix-core reuse.
//
//   out = x1 @ ((x2 + offset) * scale) + bias + x3
// ("CANN ops-transformer ... aclnnWeightQuantMatmulAllReduce 完全指南", section 计算公式),
// evaluated in the same factored form as the large-m kernel (aq_gemm.hip).
//
// Work split: a workgroup owns a 128-column slab of x2 and a contiguous k range (split-k).
// Its 8 waves (two per SIMD, so that one wave's LDS, matrix-core and VALU latencies hide
// behind the other's work) take 64-row units of the range round-robin.  Each wave streams
// its 32-row blocks -- weights, the matching 32 x 32 slice of x1 and, per-group, the
// block's scale / offset row -- into its own 3-stage LDS ring with direct-to-LDS loads (no
// barriers; vmcnt waits only), reads B fragments with tr8 transpose reads, converts them to
// exact 16-bit images and runs 32x32x16 MFMAs.  Row sums of x1 come from the A fragments
// (v_dot2).  Per-group parameters are applied at each group end and at each unit end: the
// fold is linear in the accumulators and row sums, so a group split between waves or
// workgroups is folded piecewise with its own scale and offset.  The 8 waves are reduced
// through LDS in a fixed order and the splits by a finishing kernel in a fixed order:
// results are deterministic.
#include "wq_kernels.h"
#include "wq_pipeline.h"

namespace wq {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlab = 128;    // logical columns per workgroup
constexpr int kRows = 32;     // k rows per block
constexpr int kUnit = 64;     // k rows per work unit (blocks of one unit run back to back)
constexpr int kStages = 3;    // blocks in flight per wave

template <bool W4, bool GROUPED>
struct SmTile {
  static constexpr int RB = W4 ? kSlab / 2 : kSlab;   // weight bytes per k row
  static constexpr int Wbytes = kRows * RB;           // 4 or 2 KiB
  static constexpr int Xbytes = 32 * kRows * 2;       // 2 KiB of x1 (32 rows x 32 k)
  static constexpr int Pbytes = GROUPED ? 512 : 0;    // the block's scale / offset row
  static constexpr int Stage = Wbytes + Xbytes + Pbytes;
  static constexpr int WDma = Wbytes / 1024;
  static constexpr int XDma = Xbytes / 1024;
  static constexpr int Dma = WDma + XDma + (GROUPED ? 2 : 0);  // loads per block
  static constexpr int Ring = kStages * Stage;        // per wave
  static constexpr int Red = kWaves * 32 * kSlab * 4; // wave reduction buffer
  static constexpr int Body = kWaves * Ring > Red ? kWaves * Ring : Red;
  static constexpr int GOff = Body;                   // per-wave group row-sum scratch
  static constexpr int SOff = GOff + kWaves * 32 * 4; // per-wave row sums (per-channel)
  static constexpr int Lds = SOff + kWaves * 32 * 4;
  static_assert(Lds <= 160 * 1024, "one workgroup per CU");
  static_assert(2 * Dma <= 63, "vmcnt range");
};

template <bool BF16, bool W4, bool GROUPED>
__global__ __launch_bounds__(kThreads, 1) void aq_smallm_kernel(const AqArgs a) {
  using T = SmTile<W4, GROUPED>;
  constexpr int RB = T::RB;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * kSlab, split = blockIdx.y;
  const int K = a.k, N = a.n, M = (int)a.m;
  const int kbeg = split * a.kchunk;
  const int kend = min(K, kbeg + a.kchunk);
  constexpr int bpu = kUnit / kRows;                      // blocks per unit
  const int nunits = kend > kbeg ? (kend - kbeg + kUnit - 1) / kUnit : 0;
  // this wave's blocks: units wave, wave + 8, ...; the blocks of a unit in order
  const int my_units = wave < nunits ? (nunits - wave + kWaves - 1) / kWaves : 0;
  auto block_k0 = [&](int t) { return kbeg + (wave + kWaves * (t / bpu)) * kUnit + (t % bpu) * kRows; };
  int nb = my_units * bpu;
  while (nb > 0 && block_k0(nb - 1) >= kend) --nb;         // a trailing block past the range

  const int64_t x2_pitch = W4 ? (N >> 1) : N;
  const int nb0 = W4 ? n0 / 2 : n0;
  uint8_t* ring = smem + wave * T::Ring;

  // per-lane DMA offsets inside a block
  uint32_t w_off[T::WDma];
#pragma unroll
  for (int j = 0; j < T::WDma; ++j) {
    const int r = (1024 / RB) * j + lane / (RB / 16);
    const int p = lane % (RB / 16);
    w_off[j] = (uint32_t)(r * x2_pitch + 16 * (2 * pair_slot<RB>(r, p >> 1) + (p & 1)));
  }
  uint32_t x_off[T::XDma];
#pragma unroll
  for (int j = 0; j < T::XDma; ++j) {
    const int r = 16 * j + (lane >> 2);
    x_off[j] = (uint32_t)(r * K * 2 + 16 * row_slot<64>(r, lane & 3));
  }
  const bool has_offset = a.offset != nullptr;
  u32x4_t rsc{}, rof{};
  if constexpr (GROUPED) {
    const int64_t pbytes = ((int64_t)a.groups * N - n0) * 2;
    rsc = make_rsrc((const uint8_t*)a.scale + 2 * (int64_t)n0, pbytes);
    rof = has_offset ? make_rsrc((const uint8_t*)a.offset + 2 * (int64_t)n0, pbytes) : rsc;
  }
  auto issue = [&](int t) {
    uint8_t* st = ring + (t % kStages) * T::Stage;
    const int k0 = block_k0(t);
    const u32x4_t rw = make_rsrc((const uint8_t*)a.x2 + (int64_t)k0 * x2_pitch + nb0,
                                 (int64_t)(kend - k0) * x2_pitch - nb0);
#pragma unroll
    for (int j = 0; j < T::WDma; ++j) dma16(rw, st + 1024 * j, w_off[j]);
    // blocks never straddle kend (both are multiples of 32): only rows >= m read zeros
    const u32x4_t rx = make_rsrc((const uint8_t*)a.x1 + (int64_t)k0 * 2, (int64_t)M * K * 2 - (int64_t)k0 * 2);
#pragma unroll
    for (int j = 0; j < T::XDma; ++j) dma16(rx, st + T::Wbytes + 1024 * j, x_off[j]);
    if constexpr (GROUPED)
      dma_group_row<kSlab>(st + T::Wbytes + T::Xbytes, rsc, rof, has_offset, k0 / a.group, N, lane);
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
    if constexpr (W4) return n0 + 64 * (j >> 1) + 2 * (lane & 31) + (j & 1);
    else return n0 + 32 * j + (lane & 31);
  };
  const float cbias = a.code_bias;
  float* gscr = (float*)(smem + T::GOff) + wave * 32;

  // fold the accumulators of the current group with the group's parameter rows at Ps:
  // tot += s * acc + s * (off - C) * S, S the row sums since the last fold
  auto fold = [&](const uint16_t* Ps) {
    const float t = ssum + __shfl_xor(ssum, 32, 64);
    if (lane < 32) gscr[lane] = t;
    ssum = 0.f;
    float s[4], q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lc = block_col(j) - n0;
      const float sv = act_to_f32<BF16>(Ps[lc]);
      const float ov = act_to_f32<BF16>(Ps[128 + lc]);
      s[j] = sv;
      q[j] = sv * (ov - cbias);
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
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x16_t{};
  };

  // ------------------------------------------------------------------ stream
  for (int t = 0; t < nb && t < kStages; ++t) issue(t);
  for (int t = 0; t < nb; ++t) {
    const int ahead = min(kStages - 1, nb - 1 - t);  // blocks issued after block t
    if (ahead == 2) wave_wait<2 * T::Dma>();
    else if (ahead == 1) wave_wait<T::Dma>();
    else wave_wait<0>();
    const uint8_t* W = ring + (t % kStages) * T::Stage;
    const uint8_t* X = W + T::Wbytes;
#pragma unroll
    for (int kk = 0; kk < kRows / 16; ++kk) {
      const int r = lane & 31;
      const u32x4_t af = *(const u32x4_t*)(X + r * 64 + 16 * row_slot<64>(r, 2 * kk + (lane >> 5)));
      const int kr = 16 * kk + 8 * (lane >> 5) + ((lane & 15) >> 1);
      const int sub = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
#pragma unroll
      for (int p = 0; p < (W4 ? 2 : 4); ++p) {
        const u32x2_t d = lds_read_tr8(W + kr * RB + 32 * pair_slot<RB>(kr, p) + sub);
        if constexpr (W4) {
          u32x4_t ev, od;
          i4_kpairs<BF16>(d, ev, od);
          acc[2 * p] = mfma32x32x16<BF16>(af, ev, acc[2 * p]);
          acc[2 * p + 1] = mfma32x32x16<BF16>(af, od, acc[2 * p + 1]);
        } else {
          acc[p] = mfma32x32x16<BF16>(af, i8x8_to_act<BF16>(d), acc[p]);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) ssum = dot2_ones<BF16>(af[q], ssum);
    }
    if constexpr (GROUPED) {
      // fold at a group end, and wherever the wave's next block does not continue this one
      const int kdone = block_k0(t) + kRows;
      if (kdone % a.group == 0 || kdone == kend || t % bpu == bpu - 1 || t == nb - 1)
        fold((const uint16_t*)(X + T::Xbytes));
    }
    // refill the slot of block t: its LDS reads must have completed first, since the
    // direct-to-LDS writes land whenever their data returns
    if (t + kStages < nb) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(t + kStages);
    }
  }

  // ------------------------------------------------------------------ wave reduction
  __syncthreads();
  float* red = (float*)smem;  // [kWaves][32][kSlab]
  float* sred = (float*)(smem + T::SOff);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int lc = block_col(j) - n0;
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 32 + acc_row(r, lane)) * kSlab + lc] = GROUPED ? tot[j][r] : acc[j][r];
  }
  if constexpr (!GROUPED) {
    const float t = ssum + __shfl_xor(ssum, 32, 64);
    if (lane < 32) sred[wave * 32 + lane] = t;
  }
  __syncthreads();
  float* part = a.partial + (int64_t)split * a.m * N;
  for (int o = tid; o < 32 * kSlab; o += kThreads) {
    const int row = o / kSlab, lc = o % kSlab;
    if (row >= M || n0 + lc >= N) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[(w * 32 + row) * kSlab + lc];
    part[(int64_t)row * N + n0 + lc] = v;
  }
  if constexpr (!GROUPED) {
    if (blockIdx.x == 0 && tid < M) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += sred[w * 32 + tid];
      a.rowsum_part[(int64_t)split * a.m + tid] = v;
    }
  }
}

// out = [s*P + s*(off-C)*S]  (per-tensor / per-channel)  or  T (per-group), + bias + x3,
// where P / T and S are the sums of the split partials in split order.
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
      float srow = 0.f;
      for (int s = 0; s < a.splits; ++s) srow += a.rowsum_part[(int64_t)s * a.m + row];
      const int pc = a.per_tensor ? 0 : col;
      const float sv = act_to_f32<BF16>(scale[pc]);
      const float ov = offset ? act_to_f32<BF16>(offset[pc]) : 0.f;
      v = fmaf(sv, v, sv * (ov - a.code_bias) * srow);
    }
    if (bias) v += act_to_f32<BF16>(bias[col]);
    if (x3) v += act_to_f32<BF16>(x3[i]);
    out[i] = f32_to_act<BF16>(v);
  }
}

template <bool BF16, bool W4, bool GROUPED>
hipError_t launch_sm(const AqArgs& a, hipStream_t stream) {
  using T = SmTile<W4, GROUPED>;
  const int slabs = (a.n + kSlab - 1) / kSlab;
  auto kern = aq_smallm_kernel<BF16, W4, GROUPED>;
  hipError_t e = raise_lds_limit((const void*)kern, T::Lds);
  if (e != hipSuccess) return e;
  if ((e = profile_begin(stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(slabs, a.splits), dim3(kThreads), (size_t)T::Lds, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = profile_end(stream)) != hipSuccess) return e;
  const int64_t total = a.m * a.n;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 4096));
  hipLaunchKernelGGL((aq_smallm_finish<BF16, GROUPED>), dim3((unsigned)blocks), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

SmallmPlan aq_smallm_plan(int64_t m, int k, int n, int group, bool grouped) {
  (void)m; (void)group; (void)grouped;
  SmallmPlan p;
  const int slabs = (n + kSlab - 1) / kSlab;
  const int want = std::max(1, 256 / std::max(1, slabs));  // about one workgroup per CU
  // whole units per split, a multiple of kWaves units when the range allows (balance)
  const int per = (k + want - 1) / want;
  const int step = per >= kWaves * kUnit ? kWaves * kUnit : kUnit;
  p.kchunk = std::max(kUnit, (per + step - 1) / step * step);
  p.splits = std::max(1, (k + p.kchunk - 1) / p.kchunk);
  return p;
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

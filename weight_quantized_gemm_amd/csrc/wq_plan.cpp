// Planning and the size-query half of the C ABI.  Host-only C++: no HIP call is made here
// (the compute-unit count comes from device_cu_count, defined with the launch code).
//
// Two-phase shape after the pages ("CANN ops-transformer ... aclnnWeightQuantMatmulAllReduce
// 完全指南", section 两段式接口与函数原型; "aclnnQuantMatmulAllReduceV2", Function
// Prototype): the size query validates the arguments and returns the workspace the run call
// needs; both phases are stateless and repeatable.
#include "wq_plan.h"

#include <algorithm>
#include <cstdint>

namespace wq {

// Split k when the tiles alone would leave compute units idle: as many splits as bring the
// workgroups (one per CU: each takes most of a CU's LDS) up to at most the CU count, each
// at least 256 k long (4 k-steps; 512 was up to 20% slower on short k), in whole units of k.
SplitPlan gemm_split_plan(int64_t tiles, int k, int unit, int cus) {
  SplitPlan p;
  p.kchunk = k;
  p.splits = 1;
  const int64_t want = std::max(1, cus) / std::max<int64_t>(1, tiles);
  if (want < 2) return p;
  const int min_chunk = (256 + unit - 1) / unit * unit;
  int per = (int)((k + want - 1) / want);
  per = std::max(min_chunk, (per + unit - 1) / unit * unit);
  const int splits = (k + per - 1) / per;
  if (splits < 2) return p;
  p.kchunk = per;
  p.splits = splits;
  return p;
}

namespace {

// Workgroup tile rows of a tiled kernel's default configuration for an m x k x n product:
// its tallest tile (`tallest` rows), or the next shorter one while m fits it, or while the
// taller tiles would split k into chunks of at most 512.  Such short chunks cost the taller
// workgroups more in pipeline fill and drain than the shorter tiles lose by reading each x2
// tile from twice as many workgroups: 128 rows instead of 256 measured 6-30% faster at
// m = 144-1024, 64 instead of 128 6-17% faster at m = 80-128 (both with k * n up to
// 2048 x 8192); with chunks of 1024 and more the taller tiles are level or ahead by up to
// 7%.  64 rows are taken only up to m = 128.
int tile_rows(int64_t m, int k, int n, int tallest, int cus) {
  const int64_t tiles_n = (n + kAqTileN - 1) / kAqTileN;
  auto short_chunks = [&](int bm) {
    const SplitPlan s = gemm_split_plan((m + bm - 1) / bm * tiles_n, k, 64, cus);
    return s.splits > 1 && s.kchunk <= 512;
  };
  if (m <= 64) return 64;
  if (m <= 128) return short_chunks(128) ? 64 : 128;
  if (tallest == 128) return 128;
  return short_chunks(256) ? 128 : 256;
}

constexpr int64_t kAlign = 256;
int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

}  // namespace

static_assert(kAqTileN == kQmTileN, "both tiled kernels' tiles are equally wide");

int xcd_region_rows(int64_t tiles_m, int64_t tiles_n, double mtile_bytes, double ntile_bytes) {
  int best = 0;
  double best_bytes = 0;
  for (int rm = 8; rm >= 1; rm /= 2) {  // taller rectangles first: they win ties
    const int rn = 8 / rm;
    if (tiles_m % rm != 0 || tiles_n % rn != 0) continue;
    const double bytes = (double)(tiles_m / rm) * mtile_bytes + (double)(tiles_n / rn) * ntile_bytes;
    if (best == 0 || bytes < best_bytes) {
      best = rm;
      best_bytes = bytes;
    }
  }
  return best;
}

// The anti-quant kernel: tallest tiles of 256 rows per-tensor / per-channel, 128 per-group.
int aq_gemm_tile_m(int64_t m, int k, int n, bool grouped, int cus) {
  return tile_rows(m, k, n, grouped ? 128 : 256, cus);
}

// The W8A8 kernel: tallest tiles of 256 rows.
int qm_gemm_tile_m(int64_t m, int k, int n, int cus) { return tile_rows(m, k, n, 256, cus); }

SplitPlan aq_smallm_plan(int64_t m, int k, int n, int group, bool grouped, int cus) {
  (void)m; (void)group; (void)grouped;
  SplitPlan p;
  // A split costs a second launch and a pass over the partials: none for k <= 1024 (a
  // slab's rows then stream in a few microseconds), and otherwise at least one 64-row block
  // per wave (512 k) in each split.  At k = n = 1024 this took 10.5 us down to 7.6 us, and
  // at k = 4096, n = 256 (64 splits of 64 k before) 18.9 us down to 9.3 us.
  if (k <= 1024) {
    p.kchunk = std::max(kSmRows, (k + kSmRows - 1) / kSmRows * kSmRows);
    p.splits = 1;
    return p;
  }
  const int slabs = (n + kSmSlab - 1) / kSmSlab;
  const int want = std::max(1, std::max(1, cus) / std::max(1, slabs));  // about one workgroup per CU
  // whole multiples of kSmWaves blocks per split (every wave gets a block: balance)
  const int per = (k + want - 1) / want;
  constexpr int step = kSmWaves * kSmRows;
  p.kchunk = std::max(step, (per + step - 1) / step * step);
  p.splits = std::max(1, (k + p.kchunk - 1) / p.kchunk);
  return p;
}

float code_bias(const AntiquantProblem& p) { return (p.act == WQ_BF16 && p.w4) ? 136.f : 0.f; }

AqPlan plan_antiquant(const AntiquantProblem& p, int cus) {
  AqPlan pl;
  if (p.k == 0) {
    pl.empty_k = true;
    return pl;
  }
  pl.small_m = p.m <= kSmallM;
  const bool grouped = p.mode == QuantMode::kGroup;
  if (pl.small_m) {
    pl.split = aq_smallm_plan(p.m, (int)p.k, (int)p.n, (int)p.group, grouped, cus);
  } else {
    // per-group splits end on group boundaries (the precomputed S_g cover whole groups)
    const int unit = grouped ? (p.group % 64 == 0 ? (int)p.group : 2 * (int)p.group) : 64;
    pl.bm = aq_gemm_tile_m(p.m, (int)p.k, (int)p.n, grouped, cus);
    const int64_t tiles = (p.m + pl.bm - 1) / pl.bm * ((p.n + kAqTileN - 1) / kAqTileN);
    pl.split = gemm_split_plan(tiles, (int)p.k, unit, cus);
  }
  if (pl.split.splits > 1) {
    pl.partial_bytes = align_up((int64_t)pl.split.splits * p.m * p.n * (int64_t)sizeof(float));
    pl.rowsum_bytes = grouped ? 0 : align_up((int64_t)pl.split.splits * p.m * (int64_t)sizeof(float));
  }
  if (p.params_t) pl.param_bytes = align_up(p.groups * p.n * 2);
  // per-group row sums S_g feed only the offset term s * (off - C) * S_g: none without an
  // offset and with exact images
  if (!pl.small_m && p.mode == QuantMode::kGroup && (p.has_offset || code_bias(p) != 0.f))
    pl.gsum_bytes = align_up(p.groups * p.m * 4);
  pl.workspace = pl.partial_bytes + pl.rowsum_bytes + 2 * pl.param_bytes + pl.gsum_bytes;
  return pl;
}

QmPlan plan_quant(const QuantProblem& p, int cus) {
  QmPlan pl;
  if (p.k == 0) return pl;
  pl.bm = qm_gemm_tile_m(p.m, (int)p.k, (int)p.n, cus);
  const int64_t tiles = (p.m + pl.bm - 1) / pl.bm * ((p.n + kQmTileN - 1) / kQmTileN);
  pl.split = gemm_split_plan(tiles, (int)p.k, 64, cus);
  if (pl.split.splits > 1) pl.workspace = align_up((int64_t)pl.split.splits * p.m * p.n * (int64_t)sizeof(int32_t));
  return pl;
}

}  // namespace wq

extern "C" {

int wq_antiquant_matmul_get_workspace_size(const wq_tensor* x1, const wq_tensor* x2,
                                           const wq_tensor* bias, const wq_tensor* antiquant_scale,
                                           const wq_tensor* antiquant_offset, const wq_tensor* x3,
                                           int64_t antiquant_group_size, const wq_tensor* output,
                                           uint64_t* workspace_size) {
  wq::AntiquantProblem p;
  int st = wq::validate_antiquant(x1, x2, bias, antiquant_scale, antiquant_offset, x3,
                                  antiquant_group_size, output, &p);
  if (st != WQ_OK) return st;
  if (!workspace_size) return WQ_ERR_PARAM_NULLPTR;
  *workspace_size = (uint64_t)wq::plan_antiquant(p, wq::device_cu_count()).workspace;
  return WQ_OK;
}

int wq_quant_matmul_get_workspace_size(const wq_tensor* x1, const wq_tensor* x2,
                                       const wq_tensor* bias, const wq_tensor* x3,
                                       const wq_tensor* dequant_scale,
                                       const wq_tensor* pertoken_scale, const wq_tensor* output,
                                       const wq_tensor* acc_out, uint64_t* workspace_size) {
  wq::QuantProblem p;
  int st = wq::validate_quant(x1, x2, bias, x3, dequant_scale, pertoken_scale, output, acc_out, &p);
  if (st != WQ_OK) return st;
  if (!workspace_size) return WQ_ERR_PARAM_NULLPTR;
  *workspace_size = (uint64_t)wq::plan_quant(p, wq::device_cu_count()).workspace;
  return WQ_OK;
}

int wq_prepack_weight_get_size(const wq_tensor* x2, uint64_t* packed_bytes) {
  wq::PrepackProblem p;
  const int st = wq::validate_prepack(x2, nullptr, &p);
  if (st != WQ_OK) return st;
  if (!packed_bytes) return WQ_ERR_PARAM_NULLPTR;
  *packed_bytes = (uint64_t)p.bytes;
  return WQ_OK;
}

const char* wq_status_string(int status) {
  switch (status) {
    case WQ_OK: return "WQ_OK";
    case WQ_ERR_PARAM_NULLPTR: return "WQ_ERR_PARAM_NULLPTR: a required argument is a null pointer";
    case WQ_ERR_PARAM_INVALID: return "WQ_ERR_PARAM_INVALID: an argument breaks a dtype, attribute, shape, layout or workspace rule";
    case WQ_ERR_RUNTIME: return "WQ_ERR_RUNTIME: a HIP runtime call or kernel launch failed";
    case WQ_ERR_SCRATCH_LIMIT:
      return "WQ_ERR_SCRATCH_LIMIT: the call needs more workspace than the no-allocation entry point's "
             "scratch area (WQ_NOALLOC_SCRATCH_BYTES) holds";
    default: return "unknown status";
  }
}

int wq_version(void) { return 200; }  // 0.2.0

}  // extern "C"

// C ABI entry points: validate, plan (kernel choice, workspace layout), launch.
//
// Two-phase shape after the pages ("CANN ops-transformer ... aclnnWeightQuantMatmulAllReduce
// 完全指南", section 两段式接口与函数原型; "aclnnQuantMatmulAllReduceV2", Function
// Prototype), without an executor object: both phases are stateless and repeatable.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <tuple>
#include <vector>

#include "wq_kernels.h"
#include "wq_problem.h"

namespace wq {

static_assert(kAqTileN == kQmTileN, "both tiled kernels' tiles are equally wide");

// Workgroup tile rows of a tiled kernel's default configuration for an m x k x n product:
// its tallest tile (`tallest` rows), or the next shorter one while m fits it, or while the
// taller tiles would split k into chunks of at most 512.  Such short chunks cost the taller
// workgroups more in pipeline fill and drain than the shorter tiles lose by reading each x2
// tile from twice as many workgroups: 128 rows instead of 256 measured 6-30% faster at
// m = 144-1024, 64 instead of 128 6-17% faster at m = 80-128 (both with k * n up to
// 2048 x 8192); with chunks of 1024 and more the taller tiles are level or ahead by up to
// 7%.  64 rows are taken only up to m = 128.
static int tile_rows(int64_t m, int k, int n, int tallest) {
  const int64_t tiles_n = (n + kAqTileN - 1) / kAqTileN;
  auto short_chunks = [&](int bm) {
    const SplitPlan s = gemm_split_plan((m + bm - 1) / bm * tiles_n, k, 64);
    return s.splits > 1 && s.kchunk <= 512;
  };
  if (m <= 64) return 64;
  if (m <= 128) return short_chunks(128) ? 64 : 128;
  if (tallest == 128) return 128;
  return short_chunks(256) ? 128 : 256;
}

// The anti-quant kernel (see aq_gemm.h): tallest tiles of 256 rows per-tensor /
// per-channel, 128 per-group.
int aq_gemm_tile_m(int64_t m, int k, int n, bool grouped) {
  return tile_rows(m, k, n, grouped ? 128 : 256);
}

// Split k when the tiles alone would leave CUs idle: as many splits as bring the workgroups
// (one per CU: each takes most of a CU's LDS) up to at most the CU count of an MI355X, each
// at least 256 k long (4 k-steps; 512 was up to 20% slower on short k), in whole units of k.
SplitPlan gemm_split_plan(int64_t tiles, int k, int unit) {
  constexpr int64_t kCUs = 256;
  SplitPlan p;
  p.kchunk = k;
  p.splits = 1;
  const int64_t want = kCUs / std::max<int64_t>(1, tiles);
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

// The W8A8 kernel (qm_gemm.hip): tallest tiles of 256 rows.
int qm_gemm_tile_m(int64_t m, int k, int n) { return tile_rows(m, k, n, 256); }

namespace {

constexpr int64_t kAlign = 256;
int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// The small-m split-k kernel serves m <= 32; larger m use the tiled kernel.
constexpr int64_t kSmallM = 32;

struct AqPlan {
  bool empty_k = false;
  bool small_m = false;
  SplitPlan split;           // k splits of the small-m or the tiled kernel
  int bm = 0;                // tiled kernel: tile rows (aq_gemm_tile_m)
  int64_t partial_bytes = 0;
  int64_t rowsum_bytes = 0;
  int64_t param_bytes = 0;   // per-group scale / offset given transposed: row-major copies
  int64_t gsum_bytes = 0;    // large m, per-group: row sums of x1 per group, (groups, m) fp32
  int64_t workspace = 0;
};

AqPlan plan_antiquant(const AntiquantProblem& p) {
  AqPlan pl;
  if (p.k == 0) {
    pl.empty_k = true;
    return pl;
  }
  pl.small_m = p.m <= kSmallM;
  const bool grouped = p.mode == QuantMode::kGroup;
  if (pl.small_m) {
    pl.split = aq_smallm_plan(p.m, (int)p.k, (int)p.n, (int)p.group, grouped);
  } else {
    // per-group splits end on group boundaries (the precomputed S_g cover whole groups)
    const int unit = grouped ? (p.group % 64 == 0 ? (int)p.group : 2 * (int)p.group) : 64;
    pl.bm = aq_gemm_tile_m(p.m, (int)p.k, (int)p.n, grouped);
    const int64_t tiles = (p.m + pl.bm - 1) / pl.bm * ((p.n + kAqTileN - 1) / kAqTileN);
    pl.split = gemm_split_plan(tiles, (int)p.k, unit);
  }
  if (pl.split.splits > 1) {
    pl.partial_bytes = align_up((int64_t)pl.split.splits * p.m * p.n * (int64_t)sizeof(float));
    pl.rowsum_bytes = grouped ? 0 : align_up((int64_t)pl.split.splits * p.m * (int64_t)sizeof(float));
  }
  if (p.params_t) pl.param_bytes = align_up(p.groups * p.n * 2);
  if (!pl.small_m && p.mode == QuantMode::kGroup) pl.gsum_bytes = align_up(p.groups * p.m * 4);
  pl.workspace = pl.partial_bytes + pl.rowsum_bytes + 2 * pl.param_bytes + pl.gsum_bytes;
  return pl;
}

// Tuning knob: WQ_AQ_TILE selects a non-default tile configuration of the large-m
// kernels.  Read once per process; never consulted on the launch path itself.
int tile_override() {
  static const int v = [] {
    const char* e = std::getenv("WQ_AQ_TILE");
    return e ? std::atoi(e) : 0;
  }();
  return v;
}

// The W8A8 kernel's k splits and int32 partials.
struct QmPlan {
  SplitPlan split;
  int bm = 128;
  int64_t workspace = 0;
};
QmPlan plan_quant(const QuantProblem& p) {
  QmPlan pl;
  if (p.k == 0) return pl;
  pl.bm = qm_gemm_tile_m(p.m, (int)p.k, (int)p.n);
  const int64_t tiles = (p.m + pl.bm - 1) / pl.bm * ((p.n + kQmTileN - 1) / kQmTileN);
  pl.split = gemm_split_plan(tiles, (int)p.k, 64);
  if (pl.split.splits > 1) pl.workspace = align_up((int64_t)pl.split.splits * p.m * p.n * (int64_t)sizeof(int32_t));
  return pl;
}

float code_bias(const AntiquantProblem& p) {
  // bf16 images of int4 codes are code + 136 (see wq_device.h); all other images are exact
  return (p.act == WQ_BF16 && p.w4) ? 136.f : 0.f;
}

// the events armed by wq_profile_next_call on this host thread
struct ProfileHook {
  hipEvent_t before = nullptr;
  hipEvent_t after = nullptr;
};
thread_local ProfileHook g_hook;

}  // namespace

hipError_t raise_lds_limit(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::vector<std::tuple<const void*, int, int>> done;  // (kernel, device, bytes)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& d : done)
    if (std::get<0>(d) == kernel && std::get<1>(d) == dev && std::get<2>(d) >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.emplace_back(kernel, dev, bytes);
  return e;
}

hipError_t profile_begin(hipStream_t stream) {
  return g_hook.before ? hipEventRecord(g_hook.before, stream) : hipSuccess;
}

hipError_t profile_end(hipStream_t stream) {
  hipError_t e = g_hook.after ? hipEventRecord(g_hook.after, stream) : hipSuccess;
  g_hook = ProfileHook{};
  return e;
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
  *workspace_size = (uint64_t)wq::plan_antiquant(p).workspace;
  return WQ_OK;
}

int wq_antiquant_matmul(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                        const wq_tensor* antiquant_scale, const wq_tensor* antiquant_offset,
                        const wq_tensor* x3, int64_t antiquant_group_size, const wq_tensor* output,
                        void* workspace, uint64_t workspace_size, void* stream) {
  wq::AntiquantProblem p;
  int st = wq::validate_antiquant(x1, x2, bias, antiquant_scale, antiquant_offset, x3,
                                  antiquant_group_size, output, &p);
  if (st != WQ_OK) return st;
  const wq::AqPlan pl = wq::plan_antiquant(p);
  if (workspace_size < (uint64_t)pl.workspace) return WQ_ERR_PARAM_INVALID;
  if (pl.workspace > 0 && !workspace) return WQ_ERR_PARAM_NULLPTR;
  if (pl.workspace > 0 && ((uintptr_t)workspace & 255u) != 0) return WQ_ERR_PARAM_INVALID;
  hipStream_t s = (hipStream_t)stream;

  wq::AqArgs a{};
  a.x1 = p.x1; a.x2 = p.x2; a.scale = p.scale; a.offset = p.offset; a.bias = p.bias;
  a.x3 = p.x3; a.out = p.out;
  a.m = p.m; a.k = (int32_t)p.k; a.n = (int32_t)p.n;
  a.group = (int32_t)p.group; a.groups = (int32_t)p.groups;
  a.bf16 = p.act == WQ_BF16; a.w4 = p.w4; a.f8 = p.f8; a.x2t = p.x2t;
  a.grouped = p.mode == wq::QuantMode::kGroup;
  a.per_tensor = p.mode == wq::QuantMode::kTensor;
  a.code_bias = wq::code_bias(p);
  a.splits = pl.split.splits;
  a.kchunk = pl.split.kchunk;
  a.tile = wq::tile_override();
  a.bm = pl.bm;

  hipError_t e;
  if (pl.param_bytes) {
    // transposed per-group parameters (n, groups) -> row-major (groups, n) copies
    // (scale and offset in one launch)
    char* pb = (char*)workspace + pl.partial_bytes + pl.rowsum_bytes;
    char* po = p.offset ? pb + pl.param_bytes : nullptr;
    if ((e = wq::launch_transpose16(p.scale, pb, p.offset, po, (int)p.groups, (int)p.n, s)) != hipSuccess)
      return WQ_ERR_RUNTIME;
    a.scale = pb;
    if (p.offset) a.offset = po;
  }
  if (pl.empty_k) {
    e = wq::launch_aq_bias_x3(a, s);
    return e == hipSuccess ? WQ_OK : WQ_ERR_RUNTIME;
  }
  {
    char* w = (char*)workspace;
    a.partial = pl.partial_bytes ? (float*)w : nullptr;
    a.rowsum_part = pl.rowsum_bytes ? (float*)(w + pl.partial_bytes) : nullptr;
  }
  if (pl.small_m) {
    e = wq::launch_aq_smallm(a, s);
  } else {
    if (pl.gsum_bytes) {  // per-group row sums first (the tiled kernel reads them per stage)
      a.gsum = (float*)((char*)workspace + pl.partial_bytes + pl.rowsum_bytes + 2 * pl.param_bytes);
      if ((e = wq::launch_group_rowsums(a, s)) != hipSuccess) return WQ_ERR_RUNTIME;
    }
    e = wq::launch_aq_gemm(a, s);
  }
  return e == hipSuccess ? WQ_OK : WQ_ERR_RUNTIME;
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
  *workspace_size = (uint64_t)wq::plan_quant(p).workspace;
  return WQ_OK;
}

int wq_quant_matmul(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                    const wq_tensor* x3, const wq_tensor* dequant_scale,
                    const wq_tensor* pertoken_scale, const wq_tensor* output,
                    const wq_tensor* acc_out, void* workspace, uint64_t workspace_size,
                    void* stream) {
  wq::QuantProblem p;
  int st = wq::validate_quant(x1, x2, bias, x3, dequant_scale, pertoken_scale, output, acc_out, &p);
  if (st != WQ_OK) return st;
  const wq::QmPlan pl = wq::plan_quant(p);
  if (workspace_size < (uint64_t)pl.workspace) return WQ_ERR_PARAM_INVALID;
  if (pl.workspace > 0 && !workspace) return WQ_ERR_PARAM_NULLPTR;
  if (pl.workspace > 0 && ((uintptr_t)workspace & 255u) != 0) return WQ_ERR_PARAM_INVALID;
  wq::QmArgs a{};
  a.x1 = (const int8_t*)p.x1; a.x2 = (const int8_t*)p.x2; a.bias = (const int32_t*)p.bias;
  a.x3 = p.x3; a.dq = p.dq; a.pt = (const float*)p.pt; a.out = p.out;
  a.acc_out = (int32_t*)p.acc_out;
  a.m = p.m; a.k = (int32_t)p.k; a.n = (int32_t)p.n;
  a.out_bf16 = p.out_dtype == WQ_BF16; a.dq_bf16 = p.dq_dtype == WQ_BF16;
  a.dq_per_tensor = p.dq_per_tensor;
  a.x2t = p.x2t;
  a.splits = pl.split.splits;
  a.kchunk = pl.split.kchunk;
  a.partial = pl.workspace ? (int32_t*)workspace : nullptr;
  a.tile = wq::tile_override();
  a.bm = pl.bm;
  hipError_t e = wq::launch_qm_gemm(a, (hipStream_t)stream);
  return e == hipSuccess ? WQ_OK : WQ_ERR_RUNTIME;
}

int wq_profile_next_call(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return WQ_ERR_PARAM_NULLPTR;
  wq::g_hook.before = (hipEvent_t)before;
  wq::g_hook.after = (hipEvent_t)after;
  return WQ_OK;
}

const char* wq_status_string(int status) {
  switch (status) {
    case WQ_OK: return "WQ_OK";
    case WQ_ERR_PARAM_NULLPTR: return "WQ_ERR_PARAM_NULLPTR: a required argument is a null pointer";
    case WQ_ERR_PARAM_INVALID: return "WQ_ERR_PARAM_INVALID: an argument breaks a dtype, attribute, shape, layout or workspace rule";
    case WQ_ERR_RUNTIME: return "WQ_ERR_RUNTIME: a HIP runtime call or kernel launch failed";
    default: return "unknown status";
  }
}

int wq_version(void) { return 100; }  // 0.1.0

}  // extern "C"

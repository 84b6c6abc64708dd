// C ABI run entry points: validate, plan (wq_plan.cpp), launch; the device property cache
// and the launch helpers the kernels' translation units share.
//
// Two-phase shape after the pages ("CANN ops-transformer ... aclnnWeightQuantMatmulAllReduce
// 完全指南", section 两段式接口与函数原型; "aclnnQuantMatmulAllReduceV2", Function
// Prototype), without an executor object: both phases are stateless and repeatable.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <tuple>
#include <vector>

#include "wq_kernels.h"
#include "wq_plan.h"

namespace wq {

int device_cu_count() {
  static std::mutex mu;
  static std::vector<std::pair<int, int>> known;  // (device, compute units)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kDefaultCUs;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& d : known)
    if (d.first == dev) return d.second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = kDefaultCUs;
  known.emplace_back(dev, cus);
  return cus;
}

namespace {

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

hipError_t launch_main(const void* kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream, void* args) {
  void* argv[1] = {args};
  const ProfileHook h = g_hook;
  g_hook = ProfileHook{};
  if (h.before) {
    // the events take the kernel's own start and end (they are part of its launch)
    hipError_t e = hipExtLaunchKernel(kernel, grid, block, argv, lds, stream, h.before, h.after, 0);
    if (e != hipSuccess) return e;
    return hipGetLastError();
  }
  hipError_t e = hipLaunchKernel(kernel, grid, block, argv, lds, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace wq

extern "C" {

int wq_antiquant_matmul(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                        const wq_tensor* antiquant_scale, const wq_tensor* antiquant_offset,
                        const wq_tensor* x3, int64_t antiquant_group_size, const wq_tensor* output,
                        void* workspace, uint64_t workspace_size, void* stream) {
  wq::AntiquantProblem p;
  int st = wq::validate_antiquant(x1, x2, bias, antiquant_scale, antiquant_offset, x3,
                                  antiquant_group_size, output, &p);
  if (st != WQ_OK) return st;
  const wq::AqPlan pl = wq::plan_antiquant(p, wq::device_cu_count());
  if (workspace_size < (uint64_t)pl.workspace) return WQ_ERR_PARAM_INVALID;
  if (pl.workspace > 0 && !workspace) return WQ_ERR_PARAM_NULLPTR;
  if (pl.workspace > 0 && ((uintptr_t)workspace & 255u) != 0) return WQ_ERR_PARAM_INVALID;
  hipStream_t s = (hipStream_t)stream;

  wq::AqArgs a{};
  a.x1 = p.x1; a.x2 = p.x2; a.scale = p.scale; a.offset = p.offset; a.bias = p.bias;
  a.x3 = p.x3; a.out = p.out;
  a.m = p.m; a.k = (int32_t)p.k; a.n = (int32_t)p.n;
  a.group = (int32_t)p.group; a.groups = (int32_t)p.groups;
  a.bf16 = p.act == WQ_BF16; a.w4 = p.w4; a.f8 = p.f8; a.x2t = p.x2t; a.x2p = p.x2p;
  a.grouped = p.mode == wq::QuantMode::kGroup;
  a.per_tensor = p.mode == wq::QuantMode::kTensor;
  a.code_bias = wq::code_bias(p);
  a.splits = pl.split.splits;
  a.kchunk = pl.split.kchunk;
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
    if (pl.gsum_bytes) {  // per-group row sums first (read by the tiled kernel's offset product)
      a.gsum = (float*)((char*)workspace + pl.partial_bytes + pl.rowsum_bytes + 2 * pl.param_bytes);
      if ((e = wq::launch_group_rowsums(a, s)) != hipSuccess) return WQ_ERR_RUNTIME;
    }
    e = wq::launch_aq_gemm(a, s);
  }
  return e == hipSuccess ? WQ_OK : WQ_ERR_RUNTIME;
}

int wq_quant_matmul(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                    const wq_tensor* x3, const wq_tensor* dequant_scale,
                    const wq_tensor* pertoken_scale, const wq_tensor* output,
                    const wq_tensor* acc_out, void* workspace, uint64_t workspace_size,
                    void* stream) {
  wq::QuantProblem p;
  int st = wq::validate_quant(x1, x2, bias, x3, dequant_scale, pertoken_scale, output, acc_out, &p);
  if (st != WQ_OK) return st;
  const wq::QmPlan pl = wq::plan_quant(p, wq::device_cu_count());
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
  a.x2p = p.x2p;
  a.splits = pl.split.splits;
  a.kchunk = pl.split.kchunk;
  a.partial = pl.workspace ? (int32_t*)workspace : nullptr;
  a.bm = pl.bm;
  hipError_t e = wq::launch_qm_gemm(a, (hipStream_t)stream);
  return e == hipSuccess ? WQ_OK : WQ_ERR_RUNTIME;
}

int wq_prepack_weight(const wq_tensor* x2, const wq_tensor* packed, void* stream) {
  if (!packed) return WQ_ERR_PARAM_NULLPTR;
  wq::PrepackProblem p;
  const int st = wq::validate_prepack(x2, packed, &p);
  if (st != WQ_OK) return st;
  return wq::launch_prepack(p, (hipStream_t)stream) == hipSuccess ? WQ_OK : WQ_ERR_RUNTIME;
}

int wq_profile_next_call(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return WQ_ERR_PARAM_NULLPTR;
  wq::g_hook.before = (hipEvent_t)before;
  wq::g_hook.after = (hipEvent_t)after;
  return WQ_OK;
}

}  // extern "C"

// wq_antiquant_matmul_noalloc: the anti-quant matmul with its workspace in a fixed scratch
// area inside the library, for callers that cannot allocate device memory.
//
// The scratch area is a file-scope device array; each GPU the library runs on holds its own
// copy at its own address until the process ends.  Host code never passes the array's name
// to a kernel (on the host it only stands for the symbol): the device address is looked up
// once per device, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <utility>
#include <vector>

#include "wqgemm.h"

namespace wq {
namespace {

static __device__ __align__(256) uint8_t scratch[WQ_NOALLOC_SCRATCH_BYTES];

// The current device's address of `scratch`, looked up on the first call on that device.
// Returns nullptr if the lookup fails.
void* scratch_ptr() {
  static std::mutex mu;
  static std::vector<std::pair<int, void*>> known;  // (device, address)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& d : known)
    if (d.first == dev) return d.second;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
  known.emplace_back(dev, ptr);
  return ptr;
}

}  // namespace
}  // namespace wq

extern "C" int wq_antiquant_matmul_noalloc(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                                           const wq_tensor* antiquant_scale, const wq_tensor* antiquant_offset,
                                           const wq_tensor* x3, int64_t antiquant_group_size,
                                           const wq_tensor* output, void* stream) {
  uint64_t need = 0;
  int st = wq_antiquant_matmul_get_workspace_size(x1, x2, bias, antiquant_scale, antiquant_offset, x3,
                                                  antiquant_group_size, output, &need);
  if (st != WQ_OK) return st;
  if (need > (uint64_t)WQ_NOALLOC_SCRATCH_BYTES) return WQ_ERR_SCRATCH_LIMIT;
  void* ws = wq::scratch_ptr();
  if (ws == nullptr) return WQ_ERR_RUNTIME;
  return wq_antiquant_matmul(x1, x2, bias, antiquant_scale, antiquant_offset, x3, antiquant_group_size, output,
                             ws, (uint64_t)WQ_NOALLOC_SCRATCH_BYTES, stream);
}

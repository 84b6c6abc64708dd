// Resolved problem descriptions shared by validation, planning and the kernels' launchers.
// Host-only C++ (no HIP types), so that validation builds and runs without a GPU.
#pragma once
#include <cstdint>

#include "wqgemm.h"

namespace wq {

enum class QuantMode : int { kTensor = 0, kChannel = 1, kGroup = 2 };

struct AntiquantProblem {
  int64_t m = 0, k = 0, n = 0;
  int32_t act = WQ_F16;      // WQ_F16 | WQ_BF16 (x1, scale, offset, bias, x3, output)
  bool w4 = false;           // x2 is packed int4
  bool f8 = false;           // x2 is FLOAT8_E4M3FN (per-channel, no offset)
  bool x2t = false;          // x2 is stored transposed: row-major (n, k) (int4: (n, k/2) bytes)
  bool x2p = false;          // x2 is in the packed layout (wq_prepack_weight)
  bool params_t = false;     // per-group scale / offset stored transposed: row-major (n, groups)
  QuantMode mode = QuantMode::kTensor;
  int64_t group = 0;         // group size along k (per-group); k for tensor/channel
  int64_t groups = 1;        // ceil(k / group)
  const void* x1 = nullptr;
  const void* x2 = nullptr;
  const void* scale = nullptr;
  const void* offset = nullptr;  // may be null
  const void* bias = nullptr;    // may be null
  const void* x3 = nullptr;      // may be null
  void* out = nullptr;
  bool has_offset = false;       // an offset tensor is given
};

struct QuantProblem {
  int64_t m = 0, k = 0, n = 0;
  int32_t out_dtype = WQ_BF16;   // WQ_F16 | WQ_BF16 (output and x3)
  int32_t dq_dtype = WQ_F32;     // WQ_F32 | WQ_BF16
  bool dq_per_tensor = false;
  bool x2t = false;              // x2 stored transposed: row-major (n, k)
  bool x2p = false;              // x2 in the packed layout (wq_prepack_weight)
  const void* x1 = nullptr;
  const void* x2 = nullptr;
  const void* bias = nullptr;      // int32, may be null
  const void* x3 = nullptr;        // may be null
  const void* dq = nullptr;
  const void* pt = nullptr;        // fp32 (m), may be null
  void* out = nullptr;
  void* acc_out = nullptr;         // int32 (m, n), may be null
};

// wq_prepack_weight: a weight and the buffer of its packed layout.
struct PrepackProblem {
  int64_t k = 0, n = 0;
  bool w4 = false;           // int4 (else one byte per code: int8 or FLOAT8_E4M3FN)
  bool x2t = false;          // x2 stored transposed
  const void* x2 = nullptr;
  void* packed = nullptr;
  int64_t bytes = 0;         // size of the packed layout
};

// Bytes of the packed layout of a (k, n) weight: ceil(k / 64) x (n / 32) blocks of 64 k x
// 32 columns, 2 KiB each (1 KiB for int4).
inline int64_t packed_weight_bytes(int64_t k, int64_t n, bool w4) {
  return (k + 63) / 64 * (n / 32) * (w4 ? 1024 : 2048);
}

// Validation in the pages' order (null -> dtype -> attribute -> shape).  Returns a WQ_* code.
int validate_antiquant(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                       const wq_tensor* scale, const wq_tensor* offset, const wq_tensor* x3,
                       int64_t group_size, const wq_tensor* output, AntiquantProblem* p);

int validate_prepack(const wq_tensor* x2, const wq_tensor* packed, PrepackProblem* p);

int validate_quant(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                   const wq_tensor* x3, const wq_tensor* dq, const wq_tensor* pt,
                   const wq_tensor* output, const wq_tensor* acc_out, QuantProblem* p);

}  // namespace wq

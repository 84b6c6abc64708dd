// Kernel argument blocks and launchers (host side of the HIP translation units).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#include "wq_plan.h"

namespace wq {

// Anti-quant matmul.  All 16-bit tensors are fp16 or bf16 bit patterns (act dtype).
struct AqArgs {
  const void* x1;        // (m, k)
  const void* x2;        // int8 (k, n) or packed int4 (k, n/2) bytes
  const void* scale;     // (groups, n), (n) or (1)
  const void* offset;    // like scale, or null
  const void* bias;      // (n) or null
  const void* x3;        // (m, n) or null
  void* out;             // (m, n)
  float* partial;        // split k: partial products [splits][m][n] (per-group: folded)
  float* rowsum_part;    // split k, per-tensor / per-channel: row sums of x1 [splits][m]
  float* gsum;           // large-m per-group path: row sums of x1 per group, (groups, m)
  int64_t m;
  int32_t k, n;
  int32_t group;         // group size along k (per-group); k otherwise
  int32_t groups;        // parameter rows (1 unless per-group)
  int32_t splits;        // k splits (1: the main kernel writes the output)
  int32_t kchunk;        // k rows per split (a multiple of 64; per-group large m: of the group too)
  int32_t tiles_m, tiles_n;
  int32_t xcd_rm;        // rows of the per-XCD rectangle grid (xcd_region_rows), 0: bands
  int32_t bm;            // tile rows of the default configuration (aq_gemm_tile_m)
  float code_bias;       // C: the fed weight image is code + C
  bool bf16, w4, f8, grouped, per_tensor;  // f8: FLOAT8_E4M3FN weights
  bool x2t;              // x2 stored transposed: (n, k) (int4: (n, k/2) bytes along k)
  bool x2p;              // x2 in the packed layout (wq_prepack_weight)
};

// W8A8 matmul.
struct QmArgs {
  const int8_t* x1;      // (m, k)
  const int8_t* x2;      // (k, n)
  const int32_t* bias;   // (n) or null
  const void* x3;        // (m, n) out dtype or null
  const void* dq;        // (1) or (n), fp32 or bf16
  const float* pt;       // (m) or null
  void* out;             // (m, n) fp16 / bf16
  int32_t* acc_out;      // (m, n) or null
  int32_t* partial;      // split k: int32 partial products [splits][m][n]
  int64_t m;
  int32_t k, n;
  int32_t splits;        // k splits (1: the main kernel writes the output)
  int32_t kchunk;        // k rows per split (a multiple of 64)
  int32_t tiles_m, tiles_n;
  int32_t xcd_rm;        // rows of the per-XCD rectangle grid (xcd_region_rows), 0: bands
  int32_t bm;            // tile rows of the default configuration (qm_gemm_tile_m)
  bool out_bf16, dq_bf16, dq_per_tensor;
  bool x2t;              // x2 stored transposed, (n, k)
  bool x2p;              // x2 in the packed layout (wq_prepack_weight)
};

// Raise a kernel's dynamic LDS limit; done once per (kernel, device, size) in a process.
hipError_t raise_lds_limit(const void* kernel, int bytes);

// Launch a call's main kernel, whose one argument is the block at `args`.  When
// wq_profile_next_call has armed two events on this host thread, they are passed with the
// launch (hipExtLaunchKernel), so that they take the kernel's own start and end, and the
// hook is disarmed.
hipError_t launch_main(const void* kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream, void* args);

// large-m kernels, one translation unit per weight format
hipError_t launch_aq_gemm_int8(const AqArgs& a, hipStream_t stream);
hipError_t launch_aq_gemm_int4(const AqArgs& a, hipStream_t stream);
hipError_t launch_aq_gemm_fp8(const AqArgs& a, hipStream_t stream);
inline hipError_t launch_aq_gemm(const AqArgs& a, hipStream_t stream) {
  if (a.f8) return launch_aq_gemm_fp8(a, stream);
  return a.w4 ? launch_aq_gemm_int4(a, stream) : launch_aq_gemm_int8(a, stream);
}
hipError_t launch_aq_smallm(const AqArgs& a, hipStream_t stream);
// split k (either path): out from the a.splits partials, added in split order
hipError_t launch_aq_splitk_finish(const AqArgs& a, hipStream_t stream);
hipError_t launch_aq_bias_x3(const AqArgs& a, hipStream_t stream);  // k == 0
// large m, per-group: a.gsum[g][r] = sum of x1[r, k] over the k of group g (fp32, fixed order)
hipError_t launch_group_rowsums(const AqArgs& a, hipStream_t stream);
// dst0 (rows, cols) = transpose of src0 (cols, rows), 16-bit elements, and the same for
// src1 / dst1 in the same launch unless src1 is null
hipError_t launch_transpose16(const void* src0, void* dst0, const void* src1, void* dst1, int rows,
                              int cols, hipStream_t stream);
hipError_t launch_qm_gemm(const QmArgs& a, hipStream_t stream);
// the offline weight prepack (wq_prepack_weight)
hipError_t launch_prepack(const PrepackProblem& p, hipStream_t stream);

}  // namespace wq

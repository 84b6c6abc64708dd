// Large-m anti-quant matmul for FLOAT8_E4M3FN weights (per-channel only): the instantiations of the kernel
// templates in aq_gemm.h for this weight format, fp16 and bf16 activations.
#include "aq_gemm.h"

namespace wq {

hipError_t launch_aq_gemm_fp8(const AqArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_mode<true, kWFp8>(a, stream) : launch_mode<false, kWFp8>(a, stream);
}

}  // namespace wq

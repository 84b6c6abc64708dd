// Large-m anti-quant matmul for packed int4 weights: the instantiations of the kernel
// templates in aq_gemm.h for this weight format, fp16 and bf16 activations.
#include "aq_gemm.h"

namespace wq {

hipError_t launch_aq_gemm_int4(const AqArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_mode<true, kWInt4>(a, stream) : launch_mode<false, kWInt4>(a, stream);
}

}  // namespace wq

"""CPU oracle for the weight-anti-quant matmul and its W8A8 sibling.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
anything in this package; only the test suite, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the GPU library (no kernels, headers,
helpers, tables or pre/post-processing) and imports nothing from it.

What it computes is the plain definition of each operator, in fp64, applied literally:

* anti-quant matmul -- the formula of the aclnnWeightQuantMatmulAllReduce guide
  (discosf.com), section "计算公式" (computation formula), and of the
  torch_npu.npu_mm_all_reduce_base page, "计算公式": the weight is restored as
  (x2 + antiquantOffset) * antiquantScale, multiplied by x1, then bias and x3 are added.
  The AllReduce over ranks is the identity at one rank.
* W8A8 sibling -- the aclnnQuantMatmulAllReduceV2 page, "Function" (formula, case 2):
  dequantScale * pertokenScale * (x1_int8 @ x2_int8 + bias_int32) + x3.

Pages cited in this package:
  [guide]   "CANN ops-transformer 通算融合算子 aclnnWeightQuantMatmulAllReduce 完全指南"
            (discosf.com blog post)
  [npu_mm]  "torch_npu.npu_mm_all_reduce_base" (hiascend.com API reference)
  [qmmV2]   "aclnnQuantMatmulAllReduceV2" (hiascend.com API reference)

Every function is pinned by tests that do not re-type its formula: exact rational brute
force on tiny inputs, the pages' all-ones samples in closed form, identity and
granularity reductions, invariants and decoding of hand-written bit patterns.
"""
from .storage import decode, decode_bf16, decode_fp16, decode_fp8e4m3, unpack_int4
from .antiquant import resolve_mode, expand_params, ref_antiquant
from .w8a8 import ref_w8a8_acc, ref_w8a8
from .compare import compare, TOLERANCE

__all__ = ["decode", "decode_bf16", "decode_fp16", "decode_fp8e4m3", "unpack_int4", "resolve_mode",
           "expand_params", "ref_antiquant", "ref_w8a8_acc", "ref_w8a8", "compare",
           "TOLERANCE"]

/*
 * wqgemm -- weight-anti-quant matmul and its W8A8 sibling for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; no framework types cross this boundary.
 *
 * Operations (one rank's local result; the pages' AllReduce over ranks is the identity at
 * world size 1 and is not part of this library):
 *
 *   anti-quant:  output = x1 @ ((x2 + antiquant_offset) * antiquant_scale) + bias + x3
 *     -- "CANN ops-transformer ... aclnnWeightQuantMatmulAllReduce 完全指南" (discosf.com),
 *        section 计算公式 (formula); torch_npu.npu_mm_all_reduce_base, section 计算公式.
 *
 *   W8A8:        output = dequant_scale * pertoken_scale * (x1_int8 @ x2_int8 + bias_int32) + x3
 *     -- "aclnnQuantMatmulAllReduceV2" (hiascend.com), section Function, formula case 2
 *        (case 1 is case 2 with no pertoken scale).
 *
 * Calling convention (after the pages' two-phase interface, "两段式接口与函数原型" of the
 * guide and "Function Prototype" of aclnnQuantMatmulAllReduceV2): first ask for the workspace
 * size, allocate it (device memory, owned by the caller), then launch.  Unlike the pages,
 * there is no executor object: both calls are stateless and may be repeated with the same
 * arguments any number of times.
 *
 * Ownership: the caller owns every buffer, including the workspace.  The library allocates
 * and frees no device memory on these calls.  Launches are asynchronous on the caller's
 * stream and return once enqueued; the caller synchronises.  `output` must not alias an
 * input.  Calls that share a workspace on overlapping streams race.
 *
 * Errors: status codes only (nothing is printed, thrown or aborted).  Checks run in the
 * pages' order: null pointers, then dtypes, then attributes, then shapes (guide section
 * 返回值与错误码 (return codes)).  Numeric codes for the two parameter errors are the pages'
 * (aclnnQuantMatmulAllReduceV2, "Return Value" table).
 */
#ifndef WQGEMM_H
#define WQGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  WQ_I4 is a packed signed 4-bit type: see wq_tensor.  WQ_F8E4M3 is
 * FLOAT8_E4M3FN, one byte per element: sign, 4-bit exponent of bias 7, 3-bit mantissa,
 * no infinities, S.1111.111 the only NaN (largest finite value 448). */
typedef enum wq_dtype {
  WQ_F16 = 1,
  WQ_BF16 = 2,
  WQ_F32 = 3,
  WQ_I8 = 4,
  WQ_I4 = 5,
  WQ_I32 = 6,
  WQ_F8E4M3 = 7
} wq_dtype;

/* Layout flag, or-ed into the dtype of a weight (anti-quant: WQ_I8, WQ_I4 or WQ_F8E4M3;
 * W8A8: WQ_I8):
 * the tensor holds the packed layout wq_prepack_weight writes (the role of the pages'
 * FRACTAL_NZ weight format), not an ND array.  Its descriptor keeps the logical shape
 * (k, n); its strides are not read. */
#define WQ_PACKED 0x100

/*
 * Tensor descriptor (the role of the pages' aclTensor).
 *   data    device address of the first element, 16-byte aligned (for an empty tensor it
 *           may be NULL).
 *   dtype   a wq_dtype.
 *   ndim    1, 2 or 3.
 *   shape   logical shape; entries past ndim are ignored.
 *   stride  element strides of the logical shape.  Tensors must be row-major contiguous
 *           (stride[ndim-1] == 1, stride[i] == stride[i+1]*shape[i+1]; strides of extents 1
 *           are ignored), with one exception: the weight x2 (and, per-group, the anti-quant
 *           scale and offset with it) may be the transpose of a row-major tensor, i.e. logical
 *           shape (k, n) with strides (1, k).  Anything else is WQ_ERR_PARAM_INVALID.
 * WQ_I4 weights: logical shape (k, n); two signed two's-complement nibbles per byte along the
 * storage's contiguous axis, the even index in bits 0-3.  Row-major: k rows of n/2 bytes,
 * nibbles along n.  Transposed: n rows of k/2 bytes, nibbles along k (this library's choice;
 * the pages fix no int4 packing).  Strides of a WQ_I4 tensor are given in logical elements
 * ((n, 1) row-major, (1, k) transposed).
 * An optional input is absent when its descriptor pointer is NULL.
 */
typedef struct wq_tensor {
  void* data;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[3];
  int64_t stride[3];
} wq_tensor;

#define WQ_OK 0
#define WQ_ERR_PARAM_NULLPTR 161001 /* a required input/output or its data pointer is NULL */
#define WQ_ERR_PARAM_INVALID 161002 /* dtype, attribute, shape, layout or workspace rule broken */
#define WQ_ERR_RUNTIME 561001       /* a HIP runtime or kernel-launch failure (library's own code) */
#define WQ_ERR_SCRATCH_LIMIT 561002 /* the call needs more workspace than WQ_NOALLOC_SCRATCH_BYTES */

/*
 * Workspace size of wq_antiquant_matmul for these arguments, written to *workspace_size.
 *
 * Arguments (guide, "aclnnWeightQuantMatmulAllReduceGetWorkspaceSize 参数详解" and
 * "约束说明 / 形状与范围约束" (shape constraints)):
 *   x1               required; WQ_F16 or WQ_BF16; (m, k) or (b, s, k); m = b*s in [1, 2^31-1].
 *   x2               required; WQ_I8, WQ_I4 or WQ_F8E4M3, alone or with WQ_PACKED (the
 *                    output of wq_prepack_weight); (k, n); k in [0, 65535],
 *                    n in [1, 65535].  Alignment (guide, 950 format/alignment rules): int8
 *                    needs k and n multiples of 32, int4 multiples of 64 (k = 0 is allowed);
 *                    FLOAT8_E4M3FN, one byte per element like int8, multiples of 32.
 *                    WQ_F8E4M3 weights (guide, 支持矩阵 (support matrix), 950 row, and the
 *                    note under the 950 dtype table): per-channel scale only, no
 *                    antiquant_offset (it must be NULL), antiquant_group_size 0.  Their
 *                    values enter the formula as decoded; a NaN code gives NaN outputs.
 *                    x2 may be transposed (strides (1, k): storage (n, k), or (n, k/2)
 *                    bytes for int4) (guide, 参数说明 and its notes on contiguity).
 *   bias             optional; x1's dtype; (n).
 *   antiquant_scale  required; x1's dtype.  Per-tensor (1); per-channel (n) or (1, n);
 *                    per-group (ceil(k / g), n) (guide, attribute notes on
 *                    IsAntiquantScaleShapeValid).  Per-group with a transposed x2, scale and
 *                    offset are transposed too (strides (1, ceil(k / g))); per-group with a
 *                    row-major x2 they are row-major (guide, 参数说明).
 *   antiquant_offset optional; x1's dtype; the scale's shape and layout.  Absent means 0.
 *   x3               optional; x1's dtype; the output's shape.
 *   antiquant_group_size  0 = not per-group; otherwise a multiple of 32 in
 *                    [32, min(k - 1, INT32_MAX)].  Not checked when k == 0.
 *   output           required; x1's dtype; (m, n) or (b, s, n) following x1.
 * k == 0 is the empty-K case: output = bias + x3 (absent terms are 0)
 * (guide, "空 tensor 支持度" (empty tensors)); m == 0 or n == 0 is WQ_ERR_PARAM_INVALID.
 * Returns WQ_OK, WQ_ERR_PARAM_NULLPTR or WQ_ERR_PARAM_INVALID.  Touches no device.
 */
int wq_antiquant_matmul_get_workspace_size(const wq_tensor* x1, const wq_tensor* x2,
                                           const wq_tensor* bias, const wq_tensor* antiquant_scale,
                                           const wq_tensor* antiquant_offset, const wq_tensor* x3,
                                           int64_t antiquant_group_size, const wq_tensor* output,
                                           uint64_t* workspace_size);

/*
 * Enqueue the anti-quant matmul on `stream` (a hipStream_t; NULL = the null stream).
 * Same arguments as above, plus the caller's device workspace of workspace_size bytes
 * (at least what the size query returned, 256-byte aligned; NULL allowed when that is 0).
 * Repeats every check of the size query; a workspace smaller than required is
 * WQ_ERR_PARAM_INVALID.  Returns WQ_ERR_RUNTIME if a launch fails.

 *
 * Workspace contents: none are expected on entry.  The call uses it for: fp32 split-k
 * partial sums (and per-tensor / per-channel, partial row sums of x1), until a finishing
 * kernel of the same call has added them in split order -- at m <= 32 when k > 1024, and at
 * larger m when the output tiles alone would leave compute units idle; per-group scale and
 * offset given transposed, copied row-major; and, per-group with m > 32 when an offset is
 * given or the weight images carry a bias (bf16 activations with int4 weights), the fp32
 * row sums of x1 over each group, (groups, m), written before the product.
 */
int wq_antiquant_matmul(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                        const wq_tensor* antiquant_scale, const wq_tensor* antiquant_offset,
                        const wq_tensor* x3, int64_t antiquant_group_size, const wq_tensor* output,
                        void* workspace, uint64_t workspace_size, void* stream);

/*
 * wq_antiquant_matmul for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments and
 * checks, without a workspace argument.  The workspace is a fixed scratch area inside the
 * library, WQ_NOALLOC_SCRATCH_BYTES per device, held by each device the library runs on
 * until the process ends; its device address is looked up on the first call on a device.
 * The call allocates nothing.
 * A call whose workspace (wq_antiquant_matmul_get_workspace_size) exceeds the scratch area
 * returns WQ_ERR_SCRATCH_LIMIT and enqueues nothing.  Every call on a device shares that
 * device's scratch area: calls that overlap on one device (other streams, other host
 * threads) race and must be ordered by the caller.  Nothing in the area needs to be zero on
 * entry; it keeps the last call's contents.  Returns WQ_ERR_RUNTIME if the scratch lookup or
 * a launch fails.
 */
#define WQ_NOALLOC_SCRATCH_BYTES (64u << 20)
int wq_antiquant_matmul_noalloc(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                                const wq_tensor* antiquant_scale, const wq_tensor* antiquant_offset,
                                const wq_tensor* x3, int64_t antiquant_group_size, const wq_tensor* output,
                                void* stream);

/*
 * Offline weight prepack, after the pages' two-call weight conversion
 * ("aclnnQuantMatmulAllReduceV2", Parameters table, x2 in FRACTAL_NZ format, produced by
 * aclnnCalculateMatmulWeightSizeV2 then aclnnTransMatmulWeight; guide,
 * 产品相关的格式与对齐约束).  The packed layout is this library's, made for the gfx950
 * matrix cores rather than the pages' NZ tiles:
 *   the (k, n) weight is cut into blocks of 64 k x 32 columns, stored block row by block row
 *   (k blocks outer, n blocks inner); a block holds, for each of its four 16-k steps s, the
 *   64 lanes of an MFMA B fragment in lane order: lane l is column l % 32 and k
 *   16 s + 8 (l / 32) + 0 .. 7, i.e. 8 codes, k ascending, one byte each (int8,
 *   FLOAT8_E4M3FN): 2048-byte blocks.  int4 blocks are stored in pairs (2p, 2p + 1) as one
 *   2048-byte unit of the same order, each byte holding both blocks' codes at its lane's
 *   column and k, block 2p's in bits 0-3 (n is a multiple of 64).  Codes of k >= k (a final
 *   half block) are zero.
 * Every B fragment the kernels need is then one contiguous run of bytes.
 *
 * wq_prepack_weight_get_size: the packed size in bytes of x2 (WQ_I8, WQ_I4 or WQ_F8E4M3,
 * (k, n) with k in [1, 65535] and n in [1, 65535], the alignment rules of
 * wq_antiquant_matmul; row-major or transposed as there), written to *packed_bytes.
 * Touches no device.
 *
 * wq_prepack_weight: enqueue the relayout of x2 into `packed` on `stream`.  `packed` is a
 * descriptor with dtype x2->dtype | WQ_PACKED, shape (k, n), data a caller-owned device
 * buffer of at least the packed size, 16-byte aligned, not x2's.  The packed tensor can then
 * be passed as x2 to wq_antiquant_matmul_get_workspace_size, wq_antiquant_matmul and
 * wq_antiquant_matmul_noalloc (per-group scale and offset go with it row-major,
 * (ceil(k / g), n)), and, packed int8, to wq_quant_matmul_get_workspace_size and
 * wq_quant_matmul.  Returns WQ_OK, WQ_ERR_PARAM_NULLPTR, WQ_ERR_PARAM_INVALID or
 * WQ_ERR_RUNTIME.
 */
int wq_prepack_weight_get_size(const wq_tensor* x2, uint64_t* packed_bytes);
int wq_prepack_weight(const wq_tensor* x2, const wq_tensor* packed, void* stream);

/*
 * Workspace size of wq_quant_matmul (the W8A8 sibling).
 * Arguments (aclnnQuantMatmulAllReduceV2, "Parameters" table and "Constraints"):
 *   x1              required; WQ_I8; (m, k) or (b, s, k); m in [1, 2^31-1]; k in [1, 65535].
 *   x2              required; WQ_I8; (k, n); k and n multiples of 32.  Row-major with n in
 *                   [1, 65535], or transposed (strides (1, k): storage (n, k)) with n in
 *                   [1, 2^23] (Parameters table: only the last two axes may be swapped;
 *                   Constraints: n may exceed 65535 only when x2 is transposed), or
 *                   WQ_I8 | WQ_PACKED, the output of wq_prepack_weight, with n in [1, 65535].
 *   bias            optional; WQ_I32; (n).  Added to the int32 accumulator before scaling.
 *   x3              optional; the output's dtype and shape.
 *   dequant_scale   required; (1), (n) or (1, n).  With a WQ_F16 output: WQ_F32 (the
 *                   Constraints ask for FLOAT32 when a pertoken scale is given, and for the
 *                   packed INT64/UINT64 form without one, which FLOAT32 replaces here).
 *                   With a WQ_BF16 output: WQ_BF16 (the Constraints' type) or WQ_F32.
 *   pertoken_scale  optional; WQ_F32; (m) (m = b*s for 3-D x1).  Absent means 1.
 *   output          required; WQ_F16 or WQ_BF16; (m, n) or (b, s, n) following x1.
 *   acc_out         optional; WQ_I32; (m, n): receives x1 @ x2 + bias as int32 (two's
 *                   complement wrap on overflow), for exactness checks.
 * The pages' INT64/UINT64 packed dequant scale is not supported (WQ_ERR_PARAM_INVALID).
 */
int wq_quant_matmul_get_workspace_size(const wq_tensor* x1, const wq_tensor* x2,
                                       const wq_tensor* bias, const wq_tensor* x3,
                                       const wq_tensor* dequant_scale,
                                       const wq_tensor* pertoken_scale, const wq_tensor* output,
                                       const wq_tensor* acc_out, uint64_t* workspace_size);

/*
 * Enqueue the W8A8 matmul on `stream`.  Same conventions as wq_antiquant_matmul.  The
 * workspace (zero bytes unless the output tiles alone would leave compute units idle) holds
 * int32 split-k partial products until a finishing kernel of the same call adds them; the
 * sum wraps like the single-pass accumulator, so results do not depend on the split.
 */
int wq_quant_matmul(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                    const wq_tensor* x3, const wq_tensor* dequant_scale,
                    const wq_tensor* pertoken_scale, const wq_tensor* output,
                    const wq_tensor* acc_out, void* workspace, uint64_t workspace_size,
                    void* stream);

/* Profiling hook (not part of the pages' interface; for timing the device work of one
 * call).  `before` and `after` are hipEvent_t handles, created by the caller (with timing
 * enabled) and owned by it.  The next wq_antiquant_matmul or wq_quant_matmul call made on
 * the calling host thread that launches work records `before` on its stream immediately
 * before the launch of its main kernel (the one that carries the matmul) and `after`
 * immediately after it, then disarms the hook; hipEventElapsedTime(before, after) is then
 * that kernel's device time plus the dispatch gap in front of it.  Passing two nulls
 * disarms the hook.  Returns WQ_OK, or WQ_ERR_PARAM_NULLPTR if exactly one is null.  A
 * failing hipEventRecord makes the armed call return WQ_ERR_RUNTIME. */
int wq_profile_next_call(void* before, void* after);

/* Static text for a status code. */
const char* wq_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int wq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WQGEMM_H */

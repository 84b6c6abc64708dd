// Argument validation for the C ABI.  Pure host C++; no device is touched.
//
// Rules and their sources:
//  * order of checks: null pointers, dtypes, attributes, shapes -- guide
//    "CANN ops-transformer ... aclnnWeightQuantMatmulAllReduce 完全指南", section
//    返回值与错误码 (return codes);
//  * required inputs x1, x2, antiquantScale, output -- guide, 形状与范围约束 (shape
//    constraints); for W8A8 x1, x2, dequantScale, output -- aclnnQuantMatmulAllReduceV2,
//    Return Value table and Constraints;
//  * dtypes -- guide, 支持矩阵 (support matrix, Atlas A2 row) and the "same dtype" rule of
//    the shape constraints; W8A8 -- aclnnQuantMatmulAllReduceV2 Parameters table;
//  * group size -- guide, 关键属性的源码级说明 (attribute notes);
//  * shapes and ranges -- guide, 形状与范围约束 and 空 tensor 支持度 (empty tensors);
//    W8A8 -- aclnnQuantMatmulAllReduceV2, Constraints;
//  * alignment -- guide, 产品相关的格式与对齐约束 (950: int8 needs n, k multiples of 32,
//    int4 multiples of 64).  The text is silent on FLOAT8_E4M3FN; being one byte per
//    element like int8, it takes int8's multiple of 32;
//  * FLOAT8_E4M3FN weights -- guide, 支持矩阵 (950 row) and the note under the 950 dtype
//    table: per-channel only and no antiquantOffset;
//  * transposed x2 -- guide, 参数说明 (per-group: antiquantScale and antiquantOffset are
//    transposed together with x2) and its notes on CheckContiguous; W8A8 --
//    aclnnQuantMatmulAllReduceV2, Parameters table (x2: the last two axes may be transposed,
//    no other non-contiguous layout) and Constraints (n may exceed 65535 only then).
#include <climits>
#include <cstddef>
#include <cstdint>
#include <initializer_list>

#include "wq_problem.h"

namespace wq {
namespace {

constexpr int64_t kMaxM = INT32_MAX;   // m in [1, 2^31 - 1]
constexpr int64_t kMaxKN = 65535;      // k, n in [.., 65535]
// W8A8 with a transposed x2: n beyond 65535 (the pages give no bound; this library keeps
// n * 256 within int32 tile arithmetic)
constexpr int64_t kMaxNT = (int64_t)1 << 23;

int64_t numel(const wq_tensor* t) {
  int64_t e = 1;
  for (int i = 0; i < t->ndim; ++i) e *= t->shape[i];
  return e;
}

bool dims_ok(const wq_tensor* t) {
  if (t->ndim < 1 || t->ndim > 3) return false;
  for (int i = 0; i < t->ndim; ++i)
    if (t->shape[i] < 0) return false;
  return true;
}

bool contiguous(const wq_tensor* t) {
  if (numel(t) == 0) return true;  // strides of an empty tensor carry no layout
  int64_t expect = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] > 1 && t->stride[i] != expect) return false;
    expect *= t->shape[i];
  }
  return true;
}

// The transpose of a row-major (n, k) tensor, given with its logical shape (k, n): strides
// (1, k).  Both extents exceed 1 wherever this is asked (k and n are multiples of 32, and a
// per-group parameter tensor has at least two rows), so the test is unambiguous.
bool transposed2(const wq_tensor* t) {
  return t->ndim == 2 && t->shape[0] > 1 && t->shape[1] > 1 && t->stride[0] == 1 &&
         t->stride[1] == t->shape[0];
}

// data pointer may be NULL only for an empty tensor
bool data_ok(const wq_tensor* t) { return t->data != nullptr || (dims_ok(t) && numel(t) == 0); }

bool shape_is(const wq_tensor* t, int nd, int64_t a, int64_t b = 0, int64_t c = 0) {
  if (t->ndim != nd) return false;
  const int64_t s[3] = {a, b, c};
  for (int i = 0; i < nd; ++i)
    if (t->shape[i] != s[i]) return false;
  return true;
}

bool same_shape(const wq_tensor* a, const wq_tensor* b) {
  if (a->ndim != b->ndim) return false;
  for (int i = 0; i < a->ndim; ++i)
    if (a->shape[i] != b->shape[i]) return false;
  return true;
}

// The kernels move every tensor in 16-byte pieces from its first element on.
bool aligned16(const wq_tensor* t) { return t == nullptr || ((uintptr_t)t->data & 15u) == 0; }

bool aliases(const void* out, const wq_tensor* t) {
  return t != nullptr && t->data != nullptr && t->data == out;
}

}  // namespace

int validate_antiquant(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                       const wq_tensor* scale, const wq_tensor* offset, const wq_tensor* x3,
                       int64_t group_size, const wq_tensor* output, AntiquantProblem* p) {
  // 1. null pointers
  if (!x1 || !x2 || !scale || !output) return WQ_ERR_PARAM_NULLPTR;
  for (const wq_tensor* t : {x1, x2, scale, output, offset, bias, x3})
    if (t && !data_ok(t)) return WQ_ERR_PARAM_NULLPTR;

  // 2. dtypes (x2 may carry the packed-layout flag, wq_prepack_weight's output)
  const int32_t act = x1->dtype;
  if (act != WQ_F16 && act != WQ_BF16) return WQ_ERR_PARAM_INVALID;
  const bool x2p = (x2->dtype & WQ_PACKED) != 0;
  const int32_t wdt = x2->dtype & ~WQ_PACKED;
  if (wdt != WQ_I8 && wdt != WQ_I4 && wdt != WQ_F8E4M3) return WQ_ERR_PARAM_INVALID;
  for (const wq_tensor* t : {scale, output, offset, bias, x3})
    if (t && t->dtype != act) return WQ_ERR_PARAM_INVALID;
  const bool f8 = wdt == WQ_F8E4M3;
  if (f8 && offset) return WQ_ERR_PARAM_INVALID;  // fp8 weights take no offset

  // 3. attributes (the group size rule needs k, the last dimension of x1)
  for (const wq_tensor* t : {x1, x2, scale, output, offset, bias, x3})
    if (t && !dims_ok(t)) return WQ_ERR_PARAM_INVALID;
  if (x1->ndim < 2) return WQ_ERR_PARAM_INVALID;
  const int64_t k = x1->shape[x1->ndim - 1];
  if (k != 0 && group_size != 0) {
    const int64_t hi = (k - 1 < (int64_t)INT32_MAX) ? k - 1 : (int64_t)INT32_MAX;
    if (group_size % 32 != 0 || group_size < 32 || group_size > hi) return WQ_ERR_PARAM_INVALID;
  }
  if (group_size < 0) return WQ_ERR_PARAM_INVALID;
  if (f8 && group_size != 0) return WQ_ERR_PARAM_INVALID;  // fp8 weights: per-channel only

  // 4. shapes
  if (x1->ndim != 2 && x1->ndim != 3) return WQ_ERR_PARAM_INVALID;
  if (x2->ndim != 2) return WQ_ERR_PARAM_INVALID;
  if (x2->shape[0] != k) return WQ_ERR_PARAM_INVALID;
  const int64_t n = x2->shape[1];
  int64_t m = 1;
  for (int i = 0; i < x1->ndim - 1; ++i) {
    if (x1->shape[i] < 1) return WQ_ERR_PARAM_INVALID;  // bs / m == 0 is not supported
    m *= x1->shape[i];
    if (m > kMaxM) return WQ_ERR_PARAM_INVALID;
  }
  if (k < 0 || k > kMaxKN || n < 1 || n > kMaxKN) return WQ_ERR_PARAM_INVALID;
  const bool w4 = wdt == WQ_I4;
  const int64_t align = w4 ? 64 : 32;
  if (k % align != 0 || n % align != 0) return WQ_ERR_PARAM_INVALID;

  // output (and x3) shape follows x1: (m, n) or (b, s, n)
  if (output->ndim != x1->ndim) return WQ_ERR_PARAM_INVALID;
  for (int i = 0; i < x1->ndim - 1; ++i)
    if (output->shape[i] != x1->shape[i]) return WQ_ERR_PARAM_INVALID;
  if (output->shape[output->ndim - 1] != n) return WQ_ERR_PARAM_INVALID;
  if (x3 && !same_shape(x3, output)) return WQ_ERR_PARAM_INVALID;
  if (bias && !shape_is(bias, 1, n)) return WQ_ERR_PARAM_INVALID;

  // scale shape decides the mode; offset must match the scale
  QuantMode mode;
  int64_t groups = 1, group = k;
  if (group_size != 0 && k != 0) {
    groups = (k + group_size - 1) / group_size;
    if (!shape_is(scale, 2, groups, n)) return WQ_ERR_PARAM_INVALID;
    mode = QuantMode::kGroup;
    group = group_size;
  } else if (shape_is(scale, 1, 1)) {
    mode = QuantMode::kTensor;
  } else if (shape_is(scale, 1, n) || shape_is(scale, 2, 1, n)) {
    mode = QuantMode::kChannel;
  } else if (k == 0 && group_size != 0 && shape_is(scale, 2, 0, n)) {
    mode = QuantMode::kGroup;  // empty K: ceil(0 / g) = 0 parameter rows
    groups = 0;
    group = group_size;
  } else {
    return WQ_ERR_PARAM_INVALID;
  }
  if (offset && !same_shape(offset, scale)) return WQ_ERR_PARAM_INVALID;
  if (f8 && mode != QuantMode::kChannel) return WQ_ERR_PARAM_INVALID;

  // layout: row-major contiguous, except that x2 may be the transpose of a row-major (n, k)
  // tensor; per-group parameters then must be transposed with it (and only then).  No
  // output aliasing.
  // A packed x2 is an opaque buffer (its strides are not read); it is never transposed.
  const bool x2t = !x2p && k > 0 && transposed2(x2);
  if (!x2p && !x2t && !contiguous(x2)) return WQ_ERR_PARAM_INVALID;
  const bool pt = mode == QuantMode::kGroup && groups > 0 && x2t;
  for (const wq_tensor* t : {scale, offset}) {
    if (!t) continue;
    if (mode == QuantMode::kGroup && groups > 0) {
      if (pt ? !transposed2(t) : !contiguous(t)) return WQ_ERR_PARAM_INVALID;
    } else if (!contiguous(t)) {
      return WQ_ERR_PARAM_INVALID;
    }
  }
  for (const wq_tensor* t : {x1, output, bias, x3})
    if (t && !contiguous(t)) return WQ_ERR_PARAM_INVALID;
  for (const wq_tensor* t : {x1, x2, scale, offset, bias, x3})
    if (aliases(output->data, t)) return WQ_ERR_PARAM_INVALID;
  for (const wq_tensor* t : {x1, x2, scale, offset, bias, x3, output})
    if (!aligned16(t)) return WQ_ERR_PARAM_INVALID;

  if (p) {
    p->m = m; p->k = k; p->n = n; p->act = act; p->w4 = w4; p->f8 = f8; p->mode = mode;
    p->x2t = x2t; p->x2p = x2p; p->params_t = pt;
    p->group = group; p->groups = groups;
    p->x1 = x1->data; p->x2 = x2->data; p->scale = scale->data;
    p->offset = offset ? offset->data : nullptr;
    p->has_offset = offset != nullptr;
    p->bias = bias ? bias->data : nullptr;
    p->x3 = x3 ? x3->data : nullptr;
    p->out = output->data;
  }
  return WQ_OK;
}

int validate_quant(const wq_tensor* x1, const wq_tensor* x2, const wq_tensor* bias,
                   const wq_tensor* x3, const wq_tensor* dq, const wq_tensor* pt,
                   const wq_tensor* output, const wq_tensor* acc_out, QuantProblem* p) {
  if (!x1 || !x2 || !dq || !output) return WQ_ERR_PARAM_NULLPTR;
  for (const wq_tensor* t : {x1, x2, dq, output, bias, x3, pt, acc_out})
    if (t && !data_ok(t)) return WQ_ERR_PARAM_NULLPTR;

  // x2: int8, row-major, transposed, or in the packed layout (an opaque buffer whose strides
  // are not read; never transposed)
  const bool x2p = x2->dtype == (WQ_I8 | WQ_PACKED);
  if (x1->dtype != WQ_I8 || (x2->dtype != WQ_I8 && !x2p)) return WQ_ERR_PARAM_INVALID;
  if (bias && bias->dtype != WQ_I32) return WQ_ERR_PARAM_INVALID;
  if (output->dtype != WQ_F16 && output->dtype != WQ_BF16) return WQ_ERR_PARAM_INVALID;
  if (x3 && x3->dtype != output->dtype) return WQ_ERR_PARAM_INVALID;
  if (dq->dtype != WQ_F32 && dq->dtype != WQ_BF16) return WQ_ERR_PARAM_INVALID;
  // an FLOAT16 output takes an FLOAT32 dequant scale: with a pertoken scale the pages ask for
  // FLOAT32; without one they ask for the packed INT64/UINT64 form, which this library does
  // not take, and FLOAT32 stands in for it ("aclnnQuantMatmulAllReduceV2", Constraints)
  if (output->dtype == WQ_F16 && dq->dtype != WQ_F32) return WQ_ERR_PARAM_INVALID;
  if (pt && pt->dtype != WQ_F32) return WQ_ERR_PARAM_INVALID;
  if (acc_out && acc_out->dtype != WQ_I32) return WQ_ERR_PARAM_INVALID;

  for (const wq_tensor* t : {x1, x2, dq, output, bias, x3, pt, acc_out})
    if (t && !dims_ok(t)) return WQ_ERR_PARAM_INVALID;
  if (x1->ndim != 2 && x1->ndim != 3) return WQ_ERR_PARAM_INVALID;
  if (x2->ndim != 2) return WQ_ERR_PARAM_INVALID;
  const int64_t k = x1->shape[x1->ndim - 1];
  if (x2->shape[0] != k) return WQ_ERR_PARAM_INVALID;
  const int64_t n = x2->shape[1];
  int64_t m = 1;
  for (int i = 0; i < x1->ndim - 1; ++i) {
    if (x1->shape[i] < 1) return WQ_ERR_PARAM_INVALID;
    m *= x1->shape[i];
    if (m > kMaxM) return WQ_ERR_PARAM_INVALID;
  }
  // the W8A8 op supports no empty tensor (Constraints, "Empty tensor support"); n may exceed
  // 65535 only with a transposed x2 (Constraints)
  const bool x2t = !x2p && transposed2(x2);
  if (k < 1 || k > kMaxKN || n < 1 || n > (x2t ? kMaxNT : kMaxKN)) return WQ_ERR_PARAM_INVALID;
  if (k % 32 != 0 || n % 32 != 0) return WQ_ERR_PARAM_INVALID;

  if (output->ndim != x1->ndim) return WQ_ERR_PARAM_INVALID;
  for (int i = 0; i < x1->ndim - 1; ++i)
    if (output->shape[i] != x1->shape[i]) return WQ_ERR_PARAM_INVALID;
  if (output->shape[output->ndim - 1] != n) return WQ_ERR_PARAM_INVALID;
  if (x3 && !same_shape(x3, output)) return WQ_ERR_PARAM_INVALID;
  if (bias && !shape_is(bias, 1, n)) return WQ_ERR_PARAM_INVALID;
  bool dq_tensor;
  if (shape_is(dq, 1, 1)) dq_tensor = true;
  else if (shape_is(dq, 1, n) || shape_is(dq, 2, 1, n)) dq_tensor = false;
  else return WQ_ERR_PARAM_INVALID;
  if (pt && !shape_is(pt, 1, m)) return WQ_ERR_PARAM_INVALID;
  if (acc_out && !shape_is(acc_out, 2, m, n)) return WQ_ERR_PARAM_INVALID;

  if (!x2p && !x2t && !contiguous(x2)) return WQ_ERR_PARAM_INVALID;
  for (const wq_tensor* t : {x1, dq, output, bias, x3, pt, acc_out})
    if (t && !contiguous(t)) return WQ_ERR_PARAM_INVALID;
  for (const wq_tensor* t : {x1, x2, dq, bias, x3, pt, acc_out})
    if (aliases(output->data, t)) return WQ_ERR_PARAM_INVALID;
  for (const wq_tensor* t : {x1, x2, dq, bias, x3, pt, acc_out, output})
    if (!aligned16(t)) return WQ_ERR_PARAM_INVALID;
  if (acc_out)
    for (const wq_tensor* t : {x1, x2, dq, bias, x3, pt})
      if (aliases(acc_out->data, t)) return WQ_ERR_PARAM_INVALID;

  if (p) {
    p->m = m; p->k = k; p->n = n; p->out_dtype = output->dtype; p->dq_dtype = dq->dtype;
    p->dq_per_tensor = dq_tensor;
    p->x2t = x2t;
    p->x2p = x2p;
    p->x1 = x1->data; p->x2 = x2->data; p->bias = bias ? bias->data : nullptr;
    p->x3 = x3 ? x3->data : nullptr; p->dq = dq->data; p->pt = pt ? pt->data : nullptr;
    p->out = output->data; p->acc_out = acc_out ? acc_out->data : nullptr;
  }
  return WQ_OK;
}

int validate_prepack(const wq_tensor* x2, const wq_tensor* packed, PrepackProblem* p) {
  if (!x2) return WQ_ERR_PARAM_NULLPTR;
  if (!data_ok(x2)) return WQ_ERR_PARAM_NULLPTR;
  if (x2->dtype != WQ_I8 && x2->dtype != WQ_I4 && x2->dtype != WQ_F8E4M3) return WQ_ERR_PARAM_INVALID;
  if (!dims_ok(x2) || x2->ndim != 2) return WQ_ERR_PARAM_INVALID;
  const int64_t k = x2->shape[0], n = x2->shape[1];
  if (k < 1 || k > kMaxKN || n < 1 || n > kMaxKN) return WQ_ERR_PARAM_INVALID;
  const int64_t align = x2->dtype == WQ_I4 ? 64 : 32;
  if (k % align != 0 || n % align != 0) return WQ_ERR_PARAM_INVALID;
  const bool x2t = transposed2(x2);
  if (!x2t && !contiguous(x2)) return WQ_ERR_PARAM_INVALID;
  if (!aligned16(x2)) return WQ_ERR_PARAM_INVALID;
  if (packed) {
    if (!data_ok(packed)) return WQ_ERR_PARAM_NULLPTR;
    if (packed->dtype != (x2->dtype | WQ_PACKED)) return WQ_ERR_PARAM_INVALID;
    if (!dims_ok(packed) || !shape_is(packed, 2, k, n)) return WQ_ERR_PARAM_INVALID;
    if (!aligned16(packed) || aliases(packed->data, x2)) return WQ_ERR_PARAM_INVALID;
  }
  if (p) {
    p->k = k; p->n = n; p->w4 = x2->dtype == WQ_I4; p->x2t = x2t;
    p->x2 = x2->data;
    p->packed = packed ? packed->data : nullptr;
    p->bytes = packed_weight_bytes(k, n, p->w4);
  }
  return WQ_OK;
}

}  // namespace wq

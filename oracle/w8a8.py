"""Literal oracle of the W8A8 sibling.

Test infrastructure only (see the package docstring).

[qmmV2] "Function", case 2:
    output = dequantScale * pertokenScale * (x1_int8 @ x2_int8 + bias_int32) + x3
Case 1 of the same section is case 2 with no pertoken scale (treated as 1).  bias enters
inside the parentheses, in integer arithmetic, before any scaling.
"""
from __future__ import annotations

import numpy as np

from .storage import decode

INT32_MIN, INT32_MAX = -(2 ** 31), 2 ** 31 - 1


def ref_w8a8_acc(x1: np.ndarray, x2: np.ndarray, bias=None, x2_transposed: bool = False) -> np.ndarray:
    """int32 accumulator (x1 @ x2 + bias), shape (m, n).  With ``x2_transposed`` x2 is
    stored as its transpose, (n, k) ([qmmV2] Parameters: the last two axes of x2 may be
    transposed).

    The product is taken in fp64 BLAS: every partial sum is an integer of magnitude at
    most k * 2^14 <= 2^30 < 2^53, so it is exact.  The pages say nothing on overflow; the
    oracle refuses inputs whose accumulator leaves the int32 range."""
    assert x1.dtype == np.int8 and x2.dtype == np.int8
    k = x1.shape[-1]
    a = x1.reshape(-1, k).astype(np.float64)
    w = x2.T if x2_transposed else x2
    acc = a @ w.astype(np.float64)
    acc = np.rint(acc).astype(np.int64)
    if bias is not None:
        assert bias.dtype == np.int32
        acc = acc + bias.astype(np.int64).reshape(1, -1)
    if acc.size and (acc.min() < INT32_MIN or acc.max() > INT32_MAX):
        raise OverflowError("W8A8 accumulator leaves the int32 range")
    return acc


def ref_w8a8(x1, x2, dequant_scale, pertoken_scale=None, bias=None, x3=None, *,
             dequant_dtype: str = "fp32", out: str = "bf16", x2_transposed: bool = False):
    """(fp64 output in the output's shape, int64 accumulator (m, n))."""
    acc = ref_w8a8_acc(x1, x2, bias, x2_transposed)
    m, n = acc.shape
    dq = decode(dequant_scale, dequant_dtype).reshape(-1)
    dq = np.full(n, dq[0]) if dq.size == 1 else dq.reshape(n)
    y = acc.astype(np.float64) * dq.reshape(1, n)
    if pertoken_scale is not None:
        y = y * decode(pertoken_scale, "fp32").reshape(m, 1)
    if x3 is not None:
        y = y + decode(x3, out).reshape(m, n)
    return y.reshape(tuple(x1.shape[:-1]) + (n,)), acc

"""Literal fp64 oracle of the weight-anti-quant matmul.

Test infrastructure only (see the package docstring).

    output = x1 @ ((x2 + antiquantOffset) * antiquantScale) + bias + x3

[guide] "计算公式" (formula) and [npu_mm] "计算公式"; the AllReduce is the identity at
one rank.  Parameter granularity follows [guide] "关键属性的源码级说明" (attribute
notes: per-tensor (1), per-channel (n) or (1,n), per-group (ceil(k/g), n)) and
"约束说明 / 形状与范围约束" (shape constraints).  Per-group parameters are expanded
along k by repeating each row g times, as the guide's description of its golden
reference script states ("仓库中的验证与配套资源 / Golden 验证脚本").
"""
from __future__ import annotations

import numpy as np

from .storage import decode, decode_fp8e4m3, unpack_int4


def resolve_mode(scale_shape, group_size: int, n: int) -> str:
    """Quantisation mode from the scale's shape and the group size.

    [guide] attribute notes: group size 0 means "not per-group"; a non-zero group size
    selects per-group.  Otherwise a one-element scale is per-tensor and an (n) / (1, n)
    scale is per-channel."""
    numel = int(np.prod(scale_shape))
    if group_size != 0:
        return "group"
    if numel == 1 and tuple(scale_shape) == (1,):
        return "tensor"
    if tuple(scale_shape) in ((n,), (1, n)):
        return "channel"
    raise ValueError(f"scale shape {scale_shape} fits no mode for n={n}, g={group_size}")


def expand_params(p: np.ndarray, mode: str, k: int, n: int, group_size: int) -> np.ndarray:
    """Broadcast a decoded scale or offset to a full (k, n) matrix.

    per-tensor: every entry is the scalar; per-channel: the row vector repeated down k;
    per-group: row i of the result is parameter row floor(i / g), i.e. each parameter
    row repeated g times along k and cut to k rows (a partial last group keeps the last
    parameter row)."""
    if mode == "tensor":
        return np.full((k, n), p.reshape(-1)[0], dtype=np.float64)
    if mode == "channel":
        return np.broadcast_to(p.reshape(1, n), (k, n)).astype(np.float64)
    if mode == "group":
        groups = -(-k // group_size)
        assert p.shape == (groups, n), (p.shape, groups, n)
        return np.repeat(p, group_size, axis=0)[:k]
    raise ValueError(mode)


def ref_antiquant(x1, x2, scale, offset=None, bias=None, x3=None, group_size: int = 0, *,
                  act: str, weight: str, n: int | None = None,
                  x2_transposed: bool = False) -> np.ndarray:
    """fp64 result of the anti-quant matmul, unrounded, in the output's shape.

    Inputs are stored arrays: x1/scale/offset/bias/x3 in ``act`` ("fp16" -> float16,
    "bf16" -> uint16 bit patterns); x2 int8 (k, n), packed int4 uint8 (k, n/2), or
    FLOAT8_E4M3FN bit patterns uint8 (k, n) for weight="fp8e4m3".
    None means an absent optional input: offset 0, bias 0, x3 0 ([guide] shape
    constraints: those inputs may be empty).

    ``x2_transposed``: x2 is stored as the transpose, (n, k) (int4: (n, k/2) bytes, two
    nibbles per byte along k, the even k in the low nibble), and per-group scale and offset
    are stored transposed with it, (groups, n) -> (n, groups) ([guide] 参数说明: in the
    per-group case they are transposed together with x2).  The logical operands, and so
    the result, are those of the untransposed call."""
    x1f = decode(x1, act)
    lead = x1f.shape[:-1]
    k = x1f.shape[-1]
    m = int(np.prod(lead))
    a = x1f.reshape(m, k)
    if weight == "int4":
        # the packing runs along the storage's contiguous axis in either layout
        codes = unpack_int4(x2).astype(np.float64)
    elif weight == "fp8e4m3":
        # FLOAT8_E4M3FN weights ([guide] "支持矩阵", 950 series): the stored values enter
        # the same formula; the guide allows them per-channel only and without an offset
        codes = decode_fp8e4m3(x2)
    else:
        assert x2.dtype == np.int8
        codes = x2.astype(np.float64)
    if x2_transposed:
        codes = codes.T
    assert codes.shape[0] == k
    n_ = codes.shape[1]
    if n is not None:
        assert n == n_
    n = n_

    y = np.zeros((m, n), dtype=np.float64)
    if k > 0:
        sp, op = scale, offset
        if x2_transposed and group_size != 0:
            sp = scale.T
            op = None if offset is None else offset.T
        mode = resolve_mode(sp.shape, group_size, n)
        s_full = expand_params(decode(sp, act), mode, k, n, group_size)
        o_full = (np.zeros((k, n)) if op is None
                  else expand_params(decode(op, act), mode, k, n, group_size))
        w = (codes + o_full) * s_full          # add first, then multiply
        y = a @ w
    # k == 0: the product is empty and the output is bias + x3 ([guide] "空 tensor 支持度").
    if bias is not None:
        y = y + decode(bias, act).reshape(1, n)
    if x3 is not None:
        y = y + decode(x3, act).reshape(m, n)
    return y.reshape(lead + (n,))

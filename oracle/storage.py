"""Decoding of stored operands into exact fp64 / int64 values (oracle side).

Test infrastructure only (see the package docstring).

Every fp16, bf16 and fp8-e4m3 value is a dyadic rational exactly representable in fp64,
and every int8 / int4 code is an integer, so decoding is exact: the oracle always works on the
values *as stored* (for instance fp16(0.02) is 0.0200042724609375, not 0.02).
"""
from __future__ import annotations

import numpy as np


def decode_fp16(a: np.ndarray) -> np.ndarray:
    assert a.dtype == np.float16
    return a.astype(np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64: the pattern is the upper half of an fp32."""
    assert bits.dtype == np.uint16
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """(k, n/2) bytes -> (k, n) int64 codes.

    Layout (the pages leave the int4 packing open; this library fixes it): each byte
    holds two signed two's-complement nibbles along n; bits 0-3 are column 2j and bits
    4-7 are column 2j+1."""
    assert packed.dtype == np.uint8 and packed.ndim == 2
    b = packed.astype(np.int64)
    lo = b & 0xF
    hi = b >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    k, half = packed.shape
    out = np.empty((k, 2 * half), dtype=np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def decode_fp8e4m3(bits: np.ndarray) -> np.ndarray:
    """FLOAT8_E4M3FN codes (uint8) -> fp64.

    The 950-series weight dtype FLOAT8_E4M3FN ([guide] "支持矩阵") is the 8-bit float with
    a sign bit, a 4-bit exponent of bias 7 and a 3-bit mantissa, finite only ("FN"):
    exponent field 0 holds the subnormals m/8 * 2^-6; exponent fields 1..15 hold
    (1 + m/8) * 2^(e-7), except S.1111.111, the only NaN (so the largest value is 448)."""
    assert bits.dtype == np.uint8
    b = bits.astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = sign * mag
    out[(e == 15) & ((b & 7) == 7)] = np.nan
    return out


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored array of a named storage dtype -> exact fp64 values."""
    if dtype == "fp16":
        return decode_fp16(a)
    if dtype == "bf16":
        return decode_bf16(a)
    if dtype == "fp32":
        assert a.dtype == np.float32
        return a.astype(np.float64)
    if dtype in ("int8", "int32"):
        return a.astype(np.float64)
    if dtype == "int4":
        return unpack_int4(a).astype(np.float64)
    if dtype == "fp8e4m3":
        return decode_fp8e4m3(a)
    raise ValueError(dtype)

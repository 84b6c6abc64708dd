"""Seeded synthetic inputs for the weight-anti-quant matmul and its W8A8 sibling.

This module only draws random numbers and stores them in the storage formats the
operators consume (fp16, bf16 bit patterns, int8, packed int4, int32, fp32).  It holds
none of the method's arithmetic: no dequantisation, no matmul, no epilogue.  Both the
CPU oracle (through the tests and the benchmark's CPU leg) and the GPU path receive
exactly the arrays produced here.

Storage conventions
-------------------
* fp16  -> ``numpy.float16`` (round to nearest even from the fp64 draw).
* bf16  -> ``numpy.uint16`` bit patterns: the fp64 draw is rounded to fp32 (nearest
  even), then to bf16 by round-to-nearest-even on the low 16 bits.
* int4  -> ``numpy.uint8`` of shape (k, n/2): two signed two's-complement nibbles per
  byte along n, the even column in the low nibble.
* int8 / int32 / fp32 -> the matching numpy dtype.
* transposed weights (``x2_transposed``): x2 is stored as its transpose, (n, k) (int4:
  (n, k/2) bytes, two nibbles per byte along k, the even k in the low nibble), and per-group
  scale and offset as (n, groups).  The values drawn are the same as for the row-major case
  of the same seed.
* fp8e4m3 (FLOAT8_E4M3FN) -> ``numpy.uint8`` bit patterns.  Weight codes are drawn
  uniformly over the 254 finite patterns (every pattern except S.1111.111, the NaN), so a
  case covers zeros of both signs, subnormals and the largest magnitude 448.

Draw order (one ``numpy.random.Generator(PCG64(seed))`` per case):
anti-quant: x1, x2, antiquant_scale, antiquant_offset, bias, x3;
W8A8:       x1, x2, bias, dequant_scale, pertoken_scale, x3.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

ACT_DTYPES = ("fp16", "bf16")


# --------------------------------------------------------------------------- encoders
def encode_bf16(x: np.ndarray) -> np.ndarray:
    """fp64/fp32 values -> bf16 bit patterns (uint16), round to nearest even.

    Only finite inputs are produced by the generators below, so NaN handling is not
    needed here."""
    f32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = f32.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return np.asarray(x, dtype=np.float64).astype(np.float16)
    if dtype == "bf16":
        return encode_bf16(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def pack_int4(v: np.ndarray) -> np.ndarray:
    """(k, n) integers in [-8, 7] -> (k, n/2) uint8, even column in the low nibble."""
    v = np.asarray(v)
    assert v.ndim == 2 and v.shape[1] % 2 == 0
    assert v.min(initial=0) >= -8 and v.max(initial=0) <= 7
    u = (v.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


# --------------------------------------------------------------------------- cases
@dataclasses.dataclass
class AntiquantCase:
    """One anti-quant problem, every array in its storage format."""
    name: str
    act: str                      # "fp16" | "bf16"
    weight: str                   # "int8" | "int4" | "fp8e4m3"
    x1: np.ndarray                # (m, k) or (b, s, k)
    x2: np.ndarray                # int8 (k, n), packed uint8 (k, n/2) or fp8 bits uint8 (k, n)
    n: int
    scale: np.ndarray             # (1,), (n,), (1, n) or (ceil(k/g), n)
    offset: Optional[np.ndarray]
    bias: Optional[np.ndarray]    # (n,)
    x3: Optional[np.ndarray]      # output shape
    group_size: int
    x2_transposed: bool = False   # x2 (and per-group scale / offset) stored transposed

    @property
    def k(self) -> int:
        return self.x1.shape[-1]

    @property
    def m(self) -> int:
        return int(np.prod(self.x1.shape[:-1]))

    @property
    def out_shape(self):
        return tuple(self.x1.shape[:-1]) + (self.n,)

    def arrays(self):
        return {k: v for k, v in (("x1", self.x1), ("x2", self.x2), ("scale", self.scale),
                                  ("offset", self.offset), ("bias", self.bias), ("x3", self.x3))
                if v is not None}


@dataclasses.dataclass
class W8A8Case:
    name: str
    out: str                      # "fp16" | "bf16"
    x1: np.ndarray                # int8 (m, k) or (b, s, k)
    x2: np.ndarray                # int8 (k, n)
    bias: Optional[np.ndarray]    # int32 (n,)
    dequant_scale: np.ndarray     # fp32 (1,), (n,) or (1, n); or bf16 bits
    dequant_dtype: str            # "fp32" | "bf16"
    pertoken_scale: Optional[np.ndarray]  # fp32 (m,)
    x3: Optional[np.ndarray]      # out dtype, output shape
    x2_transposed: bool = False   # x2 stored as (n, k)

    @property
    def k(self) -> int:
        return self.x1.shape[-1]

    @property
    def n(self) -> int:
        return self.x2.shape[0] if self.x2_transposed else self.x2.shape[1]

    @property
    def m(self) -> int:
        return int(np.prod(self.x1.shape[:-1]))

    @property
    def out_shape(self):
        return tuple(self.x1.shape[:-1]) + (self.n,)

    def arrays(self):
        return {k: v for k, v in (("x1", self.x1), ("x2", self.x2), ("bias", self.bias),
                                  ("dequant_scale", self.dequant_scale),
                                  ("pertoken_scale", self.pertoken_scale), ("x3", self.x3))
                if v is not None}


def digest(case) -> dict:
    """SHA-256 (first 16 hex digits) of every stored buffer, for the record."""
    return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
            for k, v in case.arrays().items()}


def _dist(rng, spec, shape):
    kind = spec[0]
    if kind == "normal":
        return rng.normal(spec[1], spec[2], size=shape)
    if kind == "uniform":
        return rng.uniform(spec[1], spec[2], size=shape)
    if kind == "const":
        return np.full(shape, float(spec[1]))
    raise ValueError(spec)


def make_antiquant(*, seed: int, act: str, weight: str, x1_shape, n: int, mode: str,
                   group_size: int = 0, scale_dist=("uniform", 0.005, 0.02),
                   offset_dist=("uniform", -2.0, 2.0), with_offset=True,
                   bias_dist=("normal", 0.0, 0.1), with_bias=True,
                   x3_dist=("normal", 0.0, 0.1), with_x3=True,
                   x1_dist=("normal", 0.0, 1.0), channel_2d=False, x2_transposed=False,
                   name="") -> AntiquantCase:
    """Draw one anti-quant case.  ``mode`` is "tensor", "channel" or "group"."""
    assert act in ACT_DTYPES and weight in ("int8", "int4", "fp8e4m3")
    rng = np.random.Generator(np.random.PCG64(seed))
    x1_shape = tuple(int(d) for d in x1_shape)
    k = x1_shape[-1]
    x1 = encode(_dist(rng, x1_dist, x1_shape), act)
    if weight == "int8":
        x2 = rng.integers(-128, 127, size=(k, n), endpoint=True, dtype=np.int8)
    elif weight == "fp8e4m3":
        r = rng.integers(0, 253, size=(k, n), endpoint=True, dtype=np.int16)
        x2 = (r + (r >= 0x7F)).astype(np.uint8)   # 0..0x7E, 0x80..0xFE: no NaN pattern
    else:
        codes4 = rng.integers(-8, 7, size=(k, n), endpoint=True, dtype=np.int8)
        x2 = pack_int4(codes4.T if x2_transposed else codes4)
    if x2_transposed and weight != "int4":
        x2 = np.ascontiguousarray(x2.T)
    if mode == "tensor":
        pshape = (1,)
    elif mode == "channel":
        pshape = (1, n) if channel_2d else (n,)
    elif mode == "group":
        assert group_size > 0
        pshape = (-(-k // group_size), n)
    else:
        raise ValueError(mode)
    scale = encode(_dist(rng, scale_dist, pshape), act)
    offset = encode(_dist(rng, offset_dist, pshape), act) if with_offset else None
    if x2_transposed and mode == "group":
        scale = np.ascontiguousarray(scale.T)
        offset = None if offset is None else np.ascontiguousarray(offset.T)
    bias = encode(_dist(rng, bias_dist, (n,)), act) if with_bias else None
    out_shape = x1_shape[:-1] + (n,)
    x3 = encode(_dist(rng, x3_dist, out_shape), act) if with_x3 else None
    return AntiquantCase(name or f"aq_{act}_{weight}_{mode}", act, weight, x1, x2, n, scale,
                         offset, bias, x3, group_size if mode == "group" else 0, x2_transposed)


def make_w8a8(*, seed: int, out: str, x1_shape, n: int, dequant: str = "channel",
              dequant_dtype: str = "fp32", with_bias=True, with_pertoken=True, with_x3=True,
              bias_range=(-1000, 1000), dq_range=(1e-4, 1e-3), pt_range=(0.5, 2.0),
              x2_transposed=False, name="") -> W8A8Case:
    rng = np.random.Generator(np.random.PCG64(seed))
    x1_shape = tuple(int(d) for d in x1_shape)
    k = x1_shape[-1]
    m = int(np.prod(x1_shape[:-1]))
    x1 = rng.integers(-128, 127, size=x1_shape, endpoint=True, dtype=np.int8)
    x2 = rng.integers(-128, 127, size=(k, n), endpoint=True, dtype=np.int8)
    if x2_transposed:
        x2 = np.ascontiguousarray(x2.T)
    bias = (rng.integers(bias_range[0], bias_range[1], size=(n,), endpoint=True,
                         dtype=np.int64).astype(np.int32) if with_bias else None)
    dshape = (1,) if dequant == "tensor" else (n,)
    dq = encode(rng.uniform(dq_range[0], dq_range[1], size=dshape), dequant_dtype)
    pt = encode(rng.uniform(pt_range[0], pt_range[1], size=(m,)), "fp32") if with_pertoken else None
    x3 = encode(rng.normal(0.0, 0.1, size=x1_shape[:-1] + (n,)), out) if with_x3 else None
    return W8A8Case(name or f"w8a8_{out}", out, x1, x2, bias, dq, dequant_dtype, pt, x3, x2_transposed)


# --------------------------------------------------------------------------- named workloads
# The workloads the library is measured on, named by what they are.  The seed of the i-th
# (1-based) is 1000 + i.
WORKLOADS = {
    "tiny_pertensor_fp16_int8_16x256x256": dict(
        kind="antiquant", seed=1001, act="fp16", weight="int8", x1_shape=(16, 256), n=256,
        mode="tensor", scale_dist=("const", 0.02), offset_dist=("const", -1.0),
        bias_dist=("normal", 0.0, 0.1), x3_dist=("normal", 0.0, 0.1)),
    "perchannel_bf16_int8_4096x4096x4096": dict(
        kind="antiquant", seed=1002, act="bf16", weight="int8", x1_shape=(4096, 4096), n=4096,
        mode="channel", scale_dist=("uniform", 0.005, 0.02), offset_dist=("uniform", -2.0, 2.0),
        bias_dist=("normal", 0.0, 0.1), x3_dist=("normal", 0.0, 0.1)),
    "pergroup128_bf16_int4_4x2048x8192x2048": dict(
        kind="antiquant", seed=1003, act="bf16", weight="int4", x1_shape=(4, 2048, 8192), n=2048,
        mode="group", group_size=128, scale_dist=("uniform", 0.01, 0.05),
        offset_dist=("uniform", -1.0, 1.0), with_bias=False, x3_dist=("normal", 0.0, 0.1)),
    "smallm_pergroup64_fp16_int8_32x8192x8192": dict(
        kind="antiquant", seed=1004, act="fp16", weight="int8", x1_shape=(32, 8192), n=8192,
        mode="group", group_size=64, scale_dist=("uniform", 0.005, 0.02),
        offset_dist=("uniform", -4.0, 4.0), bias_dist=("normal", 0.0, 0.1), with_x3=False),
    "w8a8_bf16_8192x4096x8192": dict(
        kind="w8a8", seed=1005, out="bf16", x1_shape=(8192, 4096), n=8192, dequant="channel",
        dequant_dtype="fp32"),
    # FLOAT8_E4M3FN weights (per-channel, no offset) on the shapes of the second and the
    # fourth workload
    "perchannel_bf16_fp8e4m3_4096x4096x4096": dict(
        kind="antiquant", seed=1006, act="bf16", weight="fp8e4m3", x1_shape=(4096, 4096), n=4096,
        mode="channel", scale_dist=("uniform", 2e-4, 1e-3), with_offset=False,
        bias_dist=("normal", 0.0, 0.1), x3_dist=("normal", 0.0, 0.1)),
    "smallm_perchannel_bf16_fp8e4m3_32x8192x8192": dict(
        kind="antiquant", seed=1007, act="bf16", weight="fp8e4m3", x1_shape=(32, 8192), n=8192,
        mode="channel", scale_dist=("uniform", 2e-4, 1e-3), with_offset=False,
        bias_dist=("normal", 0.0, 0.1), with_x3=False),
    # a batch of 128 tokens on the fourth workload's weights (per-channel), and the W8A8
    # sibling at the same shape: few output tiles, so k is split
    "midm_perchannel_bf16_int8_128x8192x8192": dict(
        kind="antiquant", seed=1008, act="bf16", weight="int8", x1_shape=(128, 8192), n=8192,
        mode="channel", scale_dist=("uniform", 0.005, 0.02), offset_dist=("uniform", -2.0, 2.0),
        bias_dist=("normal", 0.0, 0.1), x3_dist=("normal", 0.0, 0.1)),
    "midm_w8a8_bf16_128x8192x8192": dict(
        kind="w8a8", seed=1009, out="bf16", x1_shape=(128, 8192), n=8192, dequant="channel",
        dequant_dtype="fp32"),
}


def make_workload(name: str, *, m_rows: Optional[int] = None):
    """Build one named workload.  ``m_rows`` keeps only the first rows of x1 (and x3,
    pertoken) after drawing the full case, so that a row sample of the full-size case
    has exactly the full case's values."""
    spec = dict(WORKLOADS[name])
    kind = spec.pop("kind")
    if kind == "antiquant":
        case = make_antiquant(name=name, **spec)
    else:
        case = make_w8a8(name=name, **spec)
    if m_rows is not None:
        case = take_rows(case, m_rows)
    return case


def take_rows(case, rows: int):
    """Restrict a case to its first ``rows`` flattened rows of x1 (views, no redraw)."""
    k = case.x1.shape[-1]
    x1 = case.x1.reshape(-1, k)[:rows]
    if isinstance(case, AntiquantCase):
        x3 = None if case.x3 is None else case.x3.reshape(-1, case.n)[:rows]
        return dataclasses.replace(case, x1=x1, x3=x3)
    x3 = None if case.x3 is None else case.x3.reshape(-1, case.n)[:rows]
    pt = None if case.pertoken_scale is None else case.pertoken_scale[:rows]
    return dataclasses.replace(case, x1=x1, x3=x3, pertoken_scale=pt)


def workload_flops(name: str) -> float:
    spec = WORKLOADS[name]
    shape = spec["x1_shape"]
    m = int(np.prod(shape[:-1]))
    return 2.0 * m * shape[-1] * spec["n"]

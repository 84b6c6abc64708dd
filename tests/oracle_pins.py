"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes the oracle entry point(s) as arguments and raises
AssertionError on a mismatch, so that the same pins can be run against deliberately
broken copies of the oracle (see test_oracle_mutants.py) to show that they bite.
"""
import json
import os
from fractions import Fraction

import numpy as np

import bruteforce
import workloads
from workloads import encode, pack_int4

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ exact tiny inputs
def dyadic(rng, shape, mant_bits, lo_exp, hi_exp):
    """Random values j * 2^e with |j| < 2^mant_bits: exact in the storage dtype."""
    j = rng.integers(-(2 ** mant_bits) + 1, 2 ** mant_bits, size=shape)
    e = rng.integers(lo_exp, hi_exp + 1, size=shape)
    return j.astype(np.float64) * np.exp2(e.astype(np.float64))


MANT = {"fp16": 11, "bf16": 8}


def tiny_antiquant_case(seed, act, weight, m_shape, k, n, mode, g=0, offset=True):
    rng = np.random.default_rng(seed)
    mb = MANT[act]
    x1v = dyadic(rng, tuple(m_shape) + (k,), mb, -6, 0)
    codes = rng.integers(-8, 8 if weight == "int4" else 128, size=(k, n))
    if weight == "int8":
        codes = rng.integers(-128, 128, size=(k, n))
    pshape = {"tensor": (1,), "channel": (n,), "group": (-(-k // g) if g else 0, n)}[mode]
    sv = dyadic(rng, pshape, mb, -8, -3)
    ov = dyadic(rng, pshape, mb, -4, 1) if offset else None
    bv = dyadic(rng, (n,), mb, -6, -2)
    x3v = dyadic(rng, tuple(m_shape) + (n,), mb, -6, -2)
    stored = dict(
        x1=encode(x1v, act),
        x2=pack_int4(codes.astype(np.int8)) if weight == "int4" else codes.astype(np.int8),
        scale=encode(sv, act), offset=None if ov is None else encode(ov, act),
        bias=encode(bv, act), x3=encode(x3v, act))
    F = lambda a: [[Fraction(float(v)) for v in row] for row in np.asarray(a).reshape(-1, a.shape[-1])]
    if mode == "group":
        sl, ol = F(sv), (F(ov) if ov is not None else None)
    else:
        sl = [Fraction(float(v)) for v in sv.reshape(-1)]
        ol = [Fraction(float(v)) for v in ov.reshape(-1)] if ov is not None else None
    logical = dict(x1=F(x1v), codes=[[int(c) for c in row] for row in codes],
                   scale=sl, offset=ol, bias=[Fraction(float(v)) for v in bv],
                   x3=F(x3v), mode=mode, g=g)
    return stored, logical


TINY_CASES = [
    # (seed, act, weight, lead shape, k, n, mode, g)
    (1, "fp16", "int8", (1,), 32, 2, "tensor", 0),
    (2, "bf16", "int8", (3,), 64, 4, "channel", 0),
    (3, "fp16", "int8", (3,), 64, 4, "group", 32),
    (4, "bf16", "int8", (2,), 96, 3, "group", 64),      # partial last group
    (5, "bf16", "int4", (2, 1), 64, 4, "group", 32),    # 3-D activations, int4
    (6, "fp16", "int4", (2,), 64, 6, "channel", 0),
    (7, "bf16", "int8", (2,), 160, 2, "group", 64),     # two full groups + one partial
]


def pin_bruteforce(ref_antiquant):
    for seed, act, weight, lead, k, n, mode, g in TINY_CASES:
        st, lg = tiny_antiquant_case(seed, act, weight, lead, k, n, mode, g)
        got = ref_antiquant(st["x1"], st["x2"], st["scale"], st["offset"], st["bias"], st["x3"],
                            g, act=act, weight=weight)
        want = bruteforce.antiquant(lg["x1"], lg["codes"], lg["scale"], lg["offset"], lg["bias"],
                                    lg["x3"], mode, g)
        want = np.array([[float(v) for v in row] for row in want]).reshape(got.shape)
        scale = np.maximum(1.0, np.abs(want))
        assert np.all(np.abs(got - want) <= 1e-12 * scale), (seed, np.abs(got - want).max())


def pin_bruteforce_w8a8(ref_w8a8):
    rng = np.random.default_rng(11)
    m, k, n = 3, 64, 5
    x1 = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    x2 = rng.integers(-128, 128, size=(k, n)).astype(np.int8)
    bias = rng.integers(-1000, 1001, size=(n,)).astype(np.int32)
    dqv = dyadic(rng, (n,), 20, -14, -10)
    ptv = dyadic(rng, (m,), 20, -2, 0)
    x3v = dyadic(rng, (m, n), 8, -6, -2)
    got, acc = ref_w8a8(x1, x2, dqv.astype(np.float32), ptv.astype(np.float32), bias,
                        encode(x3v, "bf16"), dequant_dtype="fp32", out="bf16")
    wacc, wout = bruteforce.w8a8(x1.tolist(), x2.tolist(), bias.tolist(),
                                 [Fraction(float(v)) for v in dqv],
                                 [Fraction(float(v)) for v in ptv],
                                 [[Fraction(float(v)) for v in r] for r in x3v])
    assert np.array_equal(acc, np.array(wacc, dtype=np.int64))
    want = np.array([[float(v) for v in r] for r in wout])
    assert np.all(np.abs(got - want) <= 1e-12 * np.maximum(1.0, np.abs(want)))


# ------------------------------------------------------------------ transposed x2
def transposed_storage(stored, logical, weight):
    """The same logical operands stored transposed: x2 as (n, k) (int4: (n, k/2) bytes,
    nibbles along k), per-group scale and offset as (n, groups)."""
    st = dict(stored)
    codes = np.array(logical["codes"], dtype=np.int64)
    if weight == "int4":
        st["x2"] = pack_int4(np.ascontiguousarray(codes.T).astype(np.int8))
    else:
        st["x2"] = np.ascontiguousarray(stored["x2"].T)
    if logical["mode"] == "group":
        st["scale"] = np.ascontiguousarray(stored["scale"].T)
        if stored["offset"] is not None:
            st["offset"] = np.ascontiguousarray(stored["offset"].T)
    return st


def pin_bruteforce_transposed(ref_antiquant):
    """Every tiny case again with x2 (and per-group parameters) stored transposed, against
    the same exact brute force on the logical values."""
    for seed, act, weight, lead, k, n, mode, g in TINY_CASES:
        st, lg = tiny_antiquant_case(seed, act, weight, lead, k, n, mode, g)
        tt = transposed_storage(st, lg, weight)
        got = ref_antiquant(tt["x1"], tt["x2"], tt["scale"], tt["offset"], tt["bias"], tt["x3"],
                            g, act=act, weight=weight, x2_transposed=True)
        want = bruteforce.antiquant(lg["x1"], lg["codes"], lg["scale"], lg["offset"], lg["bias"],
                                    lg["x3"], mode, g)
        want = np.array([[float(v) for v in row] for row in want]).reshape(got.shape)
        assert np.all(np.abs(got - want) <= 1e-12 * np.maximum(1.0, np.abs(want))), seed


def pin_int4_kpacked(ref_antiquant):
    """Transposed int4 storage written by hand: one column (n = 1) of k = 4 codes packed
    along k, bytes 0x21, 0xF8 -> codes 1, 2, -8, -1; with x1 = (1, 10, 100, 1000) and unit
    scale the output is 1 + 20 - 800 - 1000 = -1779."""
    x1 = np.array([[1, 10, 100, 1000]], dtype=np.float16)
    x2 = np.array([[0x21, 0xF8]], dtype=np.uint8)
    y = ref_antiquant(x1, x2, np.ones(1, np.float16), None, None, None, 0, act="fp16",
                      weight="int4", x2_transposed=True)
    assert y.tolist() == [[-1779.0]], y


def pin_bruteforce_w8a8_transposed(ref_w8a8):
    rng = np.random.default_rng(12)
    m, k, n = 4, 96, 3
    x1 = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    x2 = rng.integers(-128, 128, size=(k, n)).astype(np.int8)
    dqv = dyadic(rng, (1,), 20, -14, -10)
    got, acc = ref_w8a8(x1, np.ascontiguousarray(x2.T), dqv.astype(np.float32), None, None, None,
                        dequant_dtype="fp32", out="fp16", x2_transposed=True)
    wacc, wout = bruteforce.w8a8(x1.tolist(), x2.tolist(), None, [Fraction(float(dqv[0]))], None, None)
    assert np.array_equal(acc, np.array(wacc, dtype=np.int64))
    want = np.array([[float(v) for v in r] for r in wout])
    assert np.all(np.abs(got - want) <= 1e-12 * np.maximum(1.0, np.abs(want)))


# ------------------------------------------------------------------ FLOAT8_E4M3FN weights
# bit pattern -> value, worked by hand from the format (sign | 4-bit exponent, bias 7 |
# 3-bit mantissa; exponent 0 subnormal m/8 * 2^-6; S.1111.111 NaN)
FP8_HAND = [(0x00, 0.0), (0x80, -0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
            (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0xB8, -1.0), (0x7E, 448.0), (0xFE, -448.0),
            (0x77, 240.0), (0x30, 0.5)]


def torch_fp8_values(codes):
    """All codes through torch's CPU float8_e4m3fn conversion (a library routine, independent
    of the oracle's decoder)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def pin_fp8_decode(decode_fp8e4m3):
    for code, value in FP8_HAND:
        got = decode_fp8e4m3(np.array([code], dtype=np.uint8))[0]
        assert got == value and np.signbit(got) == np.signbit(value), (hex(code), got, value)
    for code in (0x7F, 0xFF):
        assert np.isnan(decode_fp8e4m3(np.array([code], dtype=np.uint8))[0])
    codes = np.arange(256, dtype=np.uint8)
    got, lib = decode_fp8e4m3(codes), torch_fp8_values(codes)
    assert np.array_equal(np.isnan(got), np.isnan(lib))
    fin = ~np.isnan(lib)
    assert np.array_equal(got[fin], lib[fin])


def fp8_codes(rng, shape):
    """Random finite FLOAT8_E4M3FN codes (every code except the two NaNs)."""
    c = rng.integers(0, 254, size=shape)
    return np.where(c >= 0x7F, c + 1, c).astype(np.uint8)  # skip 0x7F, and 0xFF at the top


def pin_bruteforce_fp8(ref_antiquant):
    """fp8 weights, per-channel scale, no offset: the oracle against exact rationals, with
    the weight values taken from torch's float8 conversion."""
    for seed, act, lead, k, n in [(21, "bf16", (3,), 64, 4), (22, "fp16", (2, 2), 96, 3)]:
        rng = np.random.default_rng(seed)
        mb = MANT[act]
        x1v = dyadic(rng, tuple(lead) + (k,), mb, -6, 0)
        codes = fp8_codes(rng, (k, n))
        sv = dyadic(rng, (n,), mb, -8, -3)
        bv = dyadic(rng, (n,), mb, -6, -2)
        x3v = dyadic(rng, tuple(lead) + (n,), mb, -6, -2)
        got = ref_antiquant(encode(x1v, act), codes, encode(sv, act), None, encode(bv, act),
                            encode(x3v, act), 0, act=act, weight="fp8e4m3")
        wvals = torch_fp8_values(codes)
        F = lambda a: [[Fraction(float(v)) for v in row] for row in np.asarray(a).reshape(-1, a.shape[-1])]
        want = bruteforce.antiquant(F(x1v), F(wvals), [Fraction(float(v)) for v in sv], None,
                                    [Fraction(float(v)) for v in bv], F(x3v), "channel", 0)
        want = np.array([[float(v) for v in row] for row in want]).reshape(got.shape)
        assert np.all(np.abs(got - want) <= 1e-12 * np.maximum(1.0, np.abs(want))), seed


# ------------------------------------------------------------------ page samples
def pin_page_sample_antiquant(ref_antiquant):
    gd = golden("page_sample_antiquant_all_ones.json")
    one = lambda shape: np.ones(shape, dtype=np.float16)
    x2 = np.ones(gd["x2_shape"], dtype=np.int8)
    y = ref_antiquant(one(gd["x1_shape"]), x2, one(gd["scale_shape"]), one(gd["offset_shape"]),
                      one(gd["bias_shape"]), one(gd["x3_shape"]), gd["group_size"],
                      act="fp16", weight="int8")
    assert y.shape == tuple(gd["x3_shape"])
    assert np.all(y == gd["expected_every_element"])


def pin_page_sample_w8a8(ref_w8a8):
    gd = golden("page_sample_w8a8_all_ones.json")
    y, acc = ref_w8a8(np.ones(gd["x1_shape"], np.int8), np.ones(gd["x2_shape"], np.int8),
                      np.ones(gd["dequant_shape"], np.float32),
                      np.ones(gd["pertoken_shape"], np.float32),
                      np.ones(gd["bias_shape"], np.int32),
                      np.ones(gd["x3_shape"], np.float16), dequant_dtype="fp32", out="fp16")
    assert np.all(acc == gd["expected_acc"])
    assert np.all(y == gd["expected_every_element"])


def pin_worked_onehot(ref_antiquant):
    gd = golden("worked_pergroup_onehot.json")
    k, n, i = gd["k"], gd["n"], gd["onehot_index"]
    x1 = np.zeros((1, k), np.float16)
    x1[0, i] = 1
    x2 = np.full((k, n), gd["x2_fill_elsewhere"], np.int8)
    x2[i] = gd["x2_row_at_index"]
    h = lambda v: np.array(v, np.float16)
    y = ref_antiquant(x1, x2, h(gd["scale"]), h(gd["offset"]), h(gd["bias"]), h(gd["x3"]),
                      gd["group_size"], act="fp16", weight="int8")
    assert np.array_equal(y, np.array(gd["expected"]))


# ------------------------------------------------------------------ decoding
def pin_decoding(decode_bf16, unpack_int4):
    # bf16 patterns written by hand: 0x3F80 = 1.0, 0xC000 = -2.0,
    # 0x3C23 = (1 + 35/128) * 2^-7, 0x0001 = the smallest subnormal 2^-133.
    bits = np.array([0x3F80, 0xC000, 0x3C23, 0x0001, 0x7F7F], dtype=np.uint16)
    want = [1.0, -2.0, (1 + 35 / 128) * 2.0 ** -7, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127]
    assert decode_bf16(bits).tolist() == want
    # int4 bytes written by hand: 0x8F -> (lo=-1, hi=-8); 0x70 -> (0, 7); 0x19 -> (-7, 1)
    got = unpack_int4(np.array([[0x8F, 0x70, 0x19]], dtype=np.uint8))
    assert got.tolist() == [[-1, -8, 0, 7, -7, 1]]
    # fp16(0.02) as stored is 1311/65536
    assert float(np.float16(0.02)) == 1311 / 65536


# ------------------------------------------------------------------ reductions
def pin_identity(ref_antiquant):
    """offset 0 (or absent) and scale 1 reduce to a plain matmul of the integer codes,
    compared here with exact integer arithmetic on integer-valued activations."""
    rng = np.random.default_rng(21)
    m, k, n = 5, 96, 8
    xi = rng.integers(-50, 51, size=(m, k))
    codes = rng.integers(-128, 128, size=(k, n))
    want = xi.astype(np.int64) @ codes.astype(np.int64)
    for act in ("fp16", "bf16"):
        x1 = encode(xi.astype(np.float64), act)
        for off in (None, encode(np.zeros(n), act)):
            y = ref_antiquant(x1, codes.astype(np.int8), encode(np.ones(n), act), off,
                              None, None, 0, act=act, weight="int8")
            assert np.array_equal(y, want.astype(np.float64))


def pin_granularity(ref_antiquant):
    """Per-group with every group row equal to one vector == per-channel with it;
    per-channel with a constant vector == per-tensor."""
    rng = np.random.default_rng(22)
    m, k, n, g = 4, 128, 6, 32
    act = "bf16"
    x1 = encode(rng.normal(size=(m, k)), act)
    x2 = rng.integers(-128, 128, size=(k, n)).astype(np.int8)
    s = encode(rng.uniform(0.01, 0.02, n), act)
    o = encode(rng.uniform(-2, 2, n), act)
    b = encode(rng.normal(0, .1, n), act)
    x3 = encode(rng.normal(0, .1, (m, n)), act)
    ch = ref_antiquant(x1, x2, s, o, b, x3, 0, act=act, weight="int8")
    gr = ref_antiquant(x1, x2, np.tile(s, (k // g, 1)), np.tile(o, (k // g, 1)), b, x3, g,
                       act=act, weight="int8")
    assert np.array_equal(ch, gr)
    ch2 = ref_antiquant(x1, x2, np.full(n, s[0]), np.full(n, o[0]), b, x3, 0, act=act, weight="int8")
    te = ref_antiquant(x1, x2, s[:1], o[:1], b, x3, 0, act=act, weight="int8")
    assert np.array_equal(ch2, te)
    ch3 = ref_antiquant(x1, x2, s.reshape(1, n), o.reshape(1, n), b, x3, 0, act=act, weight="int8")
    assert np.array_equal(ch, ch3)


def pin_empty_k(ref_antiquant):
    """k == 0: the output is bias + x3 ([guide] empty-tensor rule)."""
    m, n = 32, 128
    rng = np.random.default_rng(23)
    b = encode(rng.normal(size=n), "fp16")
    x3 = encode(rng.normal(size=(m, n)), "fp16")
    y = ref_antiquant(np.zeros((m, 0), np.float16), np.zeros((0, n), np.int8),
                      np.ones(n, np.float16), None, b, x3, 0, act="fp16", weight="int8")
    assert np.array_equal(y, b.astype(np.float64)[None, :] + x3.astype(np.float64))
    y0 = ref_antiquant(np.zeros((m, 0), np.float16), np.zeros((0, n), np.int8),
                       np.ones(n, np.float16), None, None, None, 0, act="fp16", weight="int8")
    assert np.array_equal(y0, np.zeros((m, n)))


def pin_w8a8_exact(ref_w8a8_acc):
    """fp64-BLAS accumulator == int64 product (a different arithmetic) on a slice of the
    full-size W8A8 workload, and the identity dq = pt = 1 with no x3 returns acc."""
    case = workloads.make_workload("w8a8_bf16_8192x4096x8192", m_rows=48)
    acc = ref_w8a8_acc(case.x1, case.x2, case.bias)
    want = case.x1.astype(np.int64) @ case.x2.astype(np.int64) + case.bias.astype(np.int64)
    assert np.array_equal(acc, want)


def pin_invariants(ref_antiquant):
    rng = np.random.default_rng(24)
    m, k, n, g = 3, 128, 4, 64
    act = "fp16"
    x1 = encode(rng.normal(size=(m, k)), act)
    x2 = rng.integers(-128, 128, size=(k, n)).astype(np.int8)
    s = encode(rng.uniform(0.01, 0.02, (k // g, n)), act)
    o = encode(rng.uniform(-2, 2, (k // g, n)), act)
    b = encode(rng.normal(0, .1, n), act)
    x3 = encode(rng.normal(0, .1, (m, n)), act)
    base = ref_antiquant(x1, x2, s, o, b, x3, g, act=act, weight="int8")
    core = ref_antiquant(x1, x2, s, o, None, None, g, act=act, weight="int8")
    # bias and x3 enter additively
    assert np.allclose(base - core, b.astype(np.float64)[None] + x3.astype(np.float64),
                       rtol=0, atol=1e-12)
    # scaling every scale by 2 doubles the product part (exact in binary)
    dbl = ref_antiquant(x1, x2, (s.astype(np.float64) * 2).astype(np.float16), o, None, None, g,
                        act=act, weight="int8")
    assert np.allclose(dbl, 2 * core, rtol=1e-13, atol=1e-12)
    # permuting k inside each group (x1 columns and x2 rows together) changes nothing
    perm = np.concatenate([rng.permutation(g) + j * g for j in range(k // g)])
    pm = ref_antiquant(x1[:, perm], x2[perm], s, o, None, None, g, act=act, weight="int8")
    assert np.allclose(pm, core, rtol=1e-12, atol=1e-10)
    # the sum over two group-aligned halves of k is the whole (split-k)
    h = k // 2
    lo = ref_antiquant(x1[:, :h], x2[:h], s[: h // g], o[: h // g], None, None, g, act=act, weight="int8")
    hi = ref_antiquant(x1[:, h:], x2[h:], s[h // g:], o[h // g:], None, None, g, act=act, weight="int8")
    assert np.allclose(lo + hi, core, rtol=1e-12, atol=1e-10)
    # swapping the scale of one column changes only that column
    s2 = s.copy()
    s2[:, 1] = s[:, 2]
    sw = ref_antiquant(x1, x2, s2, o, None, None, g, act=act, weight="int8")
    assert np.array_equal(sw[:, [0, 2, 3]], core[:, [0, 2, 3]])

"""Plant plausible mistakes in (copies of) the oracle and check that the pins catch each.

The mistakes are planted on the CPU, in the oracle's helpers, through monkeypatching;
the real oracle is untouched.
"""
import numpy as np
import pytest

import oracle
import oracle.antiquant as AQ
import oracle.storage as ST
import oracle.w8a8 as W8
import oracle_pins as P

AQ_PINS = [P.pin_bruteforce, P.pin_page_sample_antiquant, P.pin_worked_onehot, P.pin_identity,
           P.pin_granularity, P.pin_empty_k, P.pin_invariants]


def caught(pins, fn):
    for pin in pins:
        try:
            pin(fn)
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def _expand_tile(p, mode, k, n, g):            # np.tile instead of repeat along k
    if mode == "group":
        return np.tile(p, (-(-k // p.shape[0]), 1))[:k]
    return REAL_EXPAND(p, mode, k, n, g)


def _expand_shift(p, mode, k, n, g):           # off-by-one group index
    if mode == "group":
        idx = np.minimum((np.arange(k) + 1) // g, p.shape[0] - 1)
        return p[idx]
    return REAL_EXPAND(p, mode, k, n, g)


def _expand_truncate(p, mode, k, n, g):        # a partial last group takes the wrong row
    if mode == "group":
        idx = np.minimum(np.arange(k) // g, max(k // g - 1, 0))
        return p[idx]
    return REAL_EXPAND(p, mode, k, n, g)


REAL_EXPAND = AQ.expand_params


def _unpack_swapped(packed):                   # nibble order swapped
    b = packed.astype(np.int64)
    lo, hi = b >> 4, b & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((packed.shape[0], 2 * packed.shape[1]), np.int64)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out


def _decode_bf16_trunc(bits):                  # bf16 read as the low half of a word
    return (bits.astype(np.uint32)).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("name,target,attr,bad", [
    ("tile_not_repeat", AQ, "expand_params", _expand_tile),
    ("group_off_by_one", AQ, "expand_params", _expand_shift),
    ("partial_group_row", AQ, "expand_params", _expand_truncate),
    ("int4_nibbles_swapped", AQ, "unpack_int4", _unpack_swapped),
])
def test_antiquant_helper_mutants(monkeypatch, name, target, attr, bad):
    monkeypatch.setattr(target, attr, bad)
    assert caught(AQ_PINS, AQ.ref_antiquant), name


def test_bf16_decode_mutant(monkeypatch):
    monkeypatch.setattr(ST, "decode_bf16", _decode_bf16_trunc)
    assert caught([lambda f: P.pin_decoding(ST.decode_bf16, ST.unpack_int4)], None)
    assert caught(AQ_PINS, AQ.ref_antiquant)


def _mutant_formula(kind):
    def ref(x1, x2, scale, offset=None, bias=None, x3=None, group_size=0, *, act, weight, n=None):
        dec = ST.decode
        x1f = dec(x1, act)
        lead, k = x1f.shape[:-1], x1f.shape[-1]
        a = x1f.reshape(int(np.prod(lead)), k)
        codes = (ST.unpack_int4(x2) if weight == "int4" else x2).astype(np.float64)
        n = codes.shape[1]
        y = np.zeros((a.shape[0], n))
        if k:
            mode = AQ.resolve_mode(scale.shape, group_size, n)
            s = AQ.expand_params(dec(scale, act), mode, k, n, group_size)
            o = np.zeros((k, n)) if offset is None else AQ.expand_params(dec(offset, act), mode, k, n, group_size)
            if kind == "mul_then_add":
                w = codes * s + o
            elif kind == "sub_offset":
                w = (codes - o) * s
            elif kind == "transposed_scale":
                w = (codes + o) * s[::-1]
            else:
                w = (codes + o) * s
            y = a @ w
        if bias is not None and kind != "drop_bias":
            y = y + dec(bias, act)[None]
        if x3 is not None and kind != "drop_x3":
            y = y + dec(x3, act).reshape(y.shape)
        return y.reshape(lead + (n,))
    return ref


@pytest.mark.parametrize("kind", ["mul_then_add", "sub_offset", "transposed_scale",
                                  "drop_bias", "drop_x3"])
def test_formula_mutants(kind):
    assert caught(AQ_PINS, _mutant_formula(kind)), kind
    # the unmutated copy passes every pin (so the harness itself is sound)
    assert not caught(AQ_PINS[:3], _mutant_formula("none"))


def _w8a8_mutant(kind):
    def ref(x1, x2, dq, pt=None, bias=None, x3=None, *, dequant_dtype="fp32", out="bf16"):
        acc = x1.reshape(-1, x1.shape[-1]).astype(np.int64) @ x2.astype(np.int64)
        m, n = acc.shape
        d = ST.decode(dq, dequant_dtype).reshape(-1)
        d = np.full(n, d[0]) if d.size == 1 else d
        y = acc * d[None]
        if bias is not None:
            if kind == "bias_after_scale":
                y = y + bias[None]
            else:
                acc = acc + bias[None]
                y = acc * d[None]
        if pt is not None:
            y = y * (pt.astype(np.float64)[None, :n] if kind == "pertoken_on_columns" and pt.size >= n
                     else pt.astype(np.float64)[:, None] if kind != "drop_pertoken" else 1.0)
        if x3 is not None and kind != "drop_x3":
            y = y + ST.decode(x3, out).reshape(m, n)
        return y.reshape(x1.shape[:-1] + (n,)), acc
    return ref


@pytest.mark.parametrize("kind", ["bias_after_scale", "drop_pertoken", "drop_x3"])
def test_w8a8_mutants(kind):
    assert caught([P.pin_bruteforce_w8a8, P.pin_page_sample_w8a8], _w8a8_mutant(kind)), kind


def _fp8_mutant(kind):
    def dec(bits):
        b = bits.astype(np.int64)
        sign = np.where(b >> 7, -1.0, 1.0)
        e = (b >> 3) & 15
        m = (b & 7).astype(np.float64)
        bias = 8 if kind == "bias8" else 7
        sub = 2.0 ** (-7 if kind == "subnormal_scale" else -6)
        mag = np.where(e == 0, m / 8.0 * sub, (1.0 + m / 8.0) * np.exp2((e - bias).astype(np.float64)))
        out = mag if kind == "no_sign" else sign * mag
        out[(e == 15) & ((b & 7) == 7)] = np.nan
        return out
    return dec


@pytest.mark.parametrize("kind", ["bias8", "subnormal_scale", "no_sign"])
def test_fp8_decode_mutants(kind, monkeypatch):
    bad = _fp8_mutant(kind)
    assert caught([P.pin_fp8_decode], bad), kind
    # through the formula too: the brute-force pin sees the mutant via the oracle
    monkeypatch.setattr(AQ, "decode_fp8e4m3", bad)
    assert caught([P.pin_bruteforce_fp8], oracle.ref_antiquant), kind


# ---------------------------------------------------------------- transposed x2
def _transposed_mutant(kind):
    """An oracle that turns transposed storage into row-major storage the wrong way, then
    runs the real oracle on it."""
    from workloads import pack_int4

    def ref(x1, x2, scale, offset=None, bias=None, x3=None, group_size=0, *, act, weight, n=None,
            x2_transposed=False):
        if x2_transposed:
            k = x1.shape[-1]
            if weight == "int4":
                codes = ST.unpack_int4(x2)                       # (n, k)
                codes = codes.reshape(k, -1) if kind == "reshape" else codes.T
                x2 = pack_int4(np.ascontiguousarray(codes).astype(np.int8))
            else:
                x2 = x2.reshape(k, -1) if kind == "reshape" else np.ascontiguousarray(x2.T)
            if group_size:
                # "params_kept": the parameters are not transposed back, only re-viewed
                fix = (lambda p: p.reshape(-1, x2.shape[1] * (2 if weight == "int4" else 1))) \
                    if kind in ("reshape", "params_kept") else (lambda p: np.ascontiguousarray(p.T))
                scale = fix(scale)
                offset = None if offset is None else fix(offset)
        return AQ.ref_antiquant(x1, x2, scale, offset, bias, x3, group_size, act=act, weight=weight, n=n)
    return ref


@pytest.mark.parametrize("kind", ["reshape", "params_kept"])
def test_transposed_mutants(kind):
    bad = _transposed_mutant(kind)
    assert caught([P.pin_bruteforce_transposed, P.pin_int4_kpacked], bad), kind


def test_transposed_w8a8_mutant():
    def bad(x1, x2, dq, pt=None, bias=None, x3=None, *, dequant_dtype="fp32", out="bf16", x2_transposed=False):
        if x2_transposed:
            x2 = x2.reshape(x1.shape[-1], -1)                   # re-viewed, not transposed
        return W8.ref_w8a8(x1, x2, dq, pt, bias, x3, dequant_dtype=dequant_dtype, out=out)
    assert caught([P.pin_bruteforce_w8a8_transposed], bad)

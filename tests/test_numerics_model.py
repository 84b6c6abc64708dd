"""Why the GPU path keeps the integer codes exact (CPU only).

Two models of the GPU arithmetic are compared with the fp64 oracle at the full k of
each measured workload (the error per element depends on k, not on m and n, so m x n
is reduced):

* naive    -- restore W = (x2 + offset) * scale and round it to the activation dtype
              before the product (what a straight dequantise-then-GEMM would feed the
              matrix cores);
* factored -- feed the exact weight codes (integers, or FLOAT8_E4M3FN values, which are
              exact in fp16 and bf16 too), accumulate in fp32 per group, apply scale
              and offset in fp32: out = sum_g s_g * (P_g + off_g * S_g) + bias + x3,
              with P_g = x1_g @ codes_g and S_g the row sums of x1 over the group.

The factored form is the same formula by linearity (checked here in fp64 first).  Naive
rounding fails the output tolerance on a sizable fraction of elements; the factored
model passes every element.
"""
import numpy as np
import pytest

import oracle
import workloads
from workloads import encode


def _round_out(y, dt):
    return oracle.decode(encode(y, dt), dt)


def _factored_fp64(x1, codes, s, o, g):
    k = codes.shape[0]
    out = np.zeros((x1.shape[0], codes.shape[1]))
    for j in range(s.shape[0]):
        sl = slice(j * g, min(k, (j + 1) * g))
        P = x1[:, sl] @ codes[sl]
        S = x1[:, sl].sum(axis=1, keepdims=True)
        out += s[j][None] * (P + o[j][None] * S)
    return out


def _factored_fp32(x1, codes, s, o, g):
    x1 = x1.astype(np.float32)
    codes = codes.astype(np.float32)
    k = codes.shape[0]
    out = np.zeros((x1.shape[0], codes.shape[1]), np.float32)
    for j in range(s.shape[0]):
        sl = slice(j * g, min(k, (j + 1) * g))
        P = x1[:, sl] @ codes[sl]
        S = x1[:, sl].sum(axis=1, keepdims=True, dtype=np.float32)
        out += s[j][None].astype(np.float32) * (P + o[j][None].astype(np.float32) * S)
    return out


def _params(case):
    n, k = case.n, case.k
    mode = oracle.resolve_mode(case.scale.shape, case.group_size, n)
    s = oracle.decode(case.scale, case.act)
    o = oracle.decode(case.offset, case.act) if case.offset is not None else np.zeros_like(s)
    if mode == "group":
        return s, o, case.group_size
    return np.broadcast_to(s.reshape(1, -1), (1, n)), np.broadcast_to(o.reshape(1, -1), (1, n)), k


CASES = [
    ("tiny_pertensor_fp16_int8_16x256x256", 16, 256),
    ("perchannel_bf16_int8_4096x4096x4096", 128, 256),
    ("pergroup128_bf16_int4_4x2048x8192x2048", 128, 256),
    ("smallm_pergroup64_fp16_int8_32x8192x8192", 32, 512),
    ("perchannel_bf16_fp8e4m3_4096x4096x4096", 128, 256),
    ("smallm_perchannel_bf16_fp8e4m3_32x8192x8192", 32, 512),
]


def _reduced(name, m, n):
    spec = dict(workloads.WORKLOADS[name])
    spec.pop("kind")
    lead = spec["x1_shape"][:-1]
    spec["x1_shape"] = (m, spec["x1_shape"][-1])
    spec["n"] = n
    return workloads.make_antiquant(**spec)


@pytest.mark.parametrize("name,m,n", CASES)
def test_factored_identity_and_rounding(name, m, n):
    case = _reduced(name, m, n)
    ref = oracle.ref_antiquant(case.x1, case.x2, case.scale, case.offset, case.bias, case.x3,
                               case.group_size, act=case.act, weight=case.weight)
    ref = ref.reshape(m, n)
    x1 = oracle.decode(case.x1, case.act).reshape(m, -1)
    if case.weight == "fp8e4m3":
        codes = oracle.decode_fp8e4m3(case.x2)
    else:
        codes = (oracle.unpack_int4(case.x2) if case.weight == "int4" else case.x2).astype(np.float64)
    s, o, g = _params(case)
    extra = np.zeros((m, n))
    if case.bias is not None:
        extra += oracle.decode(case.bias, case.act)[None]
    if case.x3 is not None:
        extra += oracle.decode(case.x3, case.act).reshape(m, n)

    # linearity: the factored form equals the literal formula in fp64
    fac64 = _factored_fp64(x1, codes, s, o, g) + extra
    assert np.allclose(fac64, ref, rtol=1e-12, atol=1e-9)

    # factored model in fp32, output rounded once: every element within tolerance
    fac32 = _factored_fp32(x1, codes, s, o, g).astype(np.float64) + extra
    r = oracle.compare(_round_out(fac32, case.act), ref, case.act)
    assert r["ok"], r

    # naive model: dequantised weight rounded to the activation dtype first
    k = codes.shape[0]
    mode = "group" if s.shape[0] > 1 else "channel"
    S = oracle.expand_params(s, "group", k, n, g) if mode == "group" else np.broadcast_to(s, (k, n))
    O = oracle.expand_params(o, "group", k, n, g) if mode == "group" else np.broadcast_to(o, (k, n))
    w = oracle.decode(encode((codes + O) * S, case.act), case.act)
    naive = _round_out(x1 @ w + extra, case.act)
    rn = oracle.compare(naive, ref, case.act)
    assert rn["n_fail"] > 0.01 * rn["n"], rn

"""GPU: the offline weight prepack (wq_prepack_weight) and the anti-quant calls on packed
weights.

The packed bytes must equal the NumPy restatement of the layout (tests/packing.py) bit for
bit (byte work), from row-major and transposed weights of every code type, with a k tail.
Matmuls on the packed weight must match the fp64 oracle evaluated on the original logical
weight, to the usual tolerances (fp16 outputs 2e-3, bf16 1e-2, relative to max(1, |ref|)):
the small-m kernel on packed weights (with and without k splits) and the tiled kernels'
packed path (64-, 128- and 256-row tiles, split k), every mode and code type, and the
full-size small-m workload.  The W8A8 call on a packed int8 weight must give the oracle's
int32 accumulator bit for bit and its output to the same tolerances.  Seeded random sweeps
cover both calls on packed weights across dtypes, code types, modes, optional inputs,
ragged shapes and transposed sources.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
import weight_quantized_gemm_amd as W
from gpu_util import dev_tensor, ref_antiquant, ref_w8a8, run_w8a8, to_f64
from packing import logical_codes, pack_reference

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"[gpu-case] {name}", flush=True)


def _x2_dev(case):
    x2 = dev_tensor(case.x2, "raw")
    if case.weight == "fp8e4m3":
        x2 = x2.view(torch.float8_e4m3fn)
    return x2.t() if case.x2_transposed else x2


@pytest.mark.parametrize("weight,k,n,xt", [
    ("int8", 96, 64, False), ("int8", 256, 320, True), ("fp8e4m3", 160, 96, False),
    ("fp8e4m3", 64, 32, True), ("int4", 192, 128, False), ("int4", 128, 192, True),
], ids=lambda v: str(v))
def test_prepack_bytes(weight, k, n, xt):
    _announce(f"prepack_bytes_{weight}_{k}x{n}_{xt}")
    case = workloads.make_antiquant(seed=k * 31 + n, act="bf16", weight=weight, x1_shape=(1, k), n=n,
                                    mode="channel", with_offset=weight != "fp8e4m3", x2_transposed=xt)
    pw = W.prepack_weight(_x2_dev(case), x2_int4=weight == "int4")
    torch.cuda.synchronize()
    got = pw.data.cpu().numpy()
    want = pack_reference(logical_codes(case.x2, weight, xt), weight == "int4")
    assert got.size == want.size == W.packed_weight_bytes(_x2_dev(case), x2_int4=weight == "int4")
    assert np.array_equal(got, want)


def check_packed(case):
    _announce(f"packed:{case.name}")
    act = case.act
    pw = W.prepack_weight(_x2_dev(case), x2_int4=case.weight == "int4")
    scale, offset = case.scale, case.offset
    if case.x2_transposed and case.group_size:
        # packed weights take row-major per-group parameters
        scale = np.ascontiguousarray(scale.T)
        offset = None if offset is None else np.ascontiguousarray(offset.T)
    y = W.antiquant_matmul(dev_tensor(case.x1, act), pw, dev_tensor(scale, act), dev_tensor(offset, act),
                           dev_tensor(case.bias, act), dev_tensor(case.x3, act), case.group_size)
    got = to_f64(y).reshape(case.out_shape)
    r = oracle.compare(got, ref_antiquant(case), act)
    assert r["ok"], (case.name, r)


PACKED_CASES = [
    # small m (m <= 32): the column-block kernel; n < 4096 splits k
    ("pk_sm_m1_perchannel_bf16_i8", dict(act="bf16", weight="int8", x1_shape=(1, 2048), n=256, mode="channel")),
    ("pk_sm_m7_pertensor_fp16_i8_ktail", dict(act="fp16", weight="int8", x1_shape=(7, 1056), n=96, mode="tensor")),
    ("pk_sm_m32_pergroup64_fp16_i8", dict(act="fp16", weight="int8", x1_shape=(32, 4096), n=512, mode="group",
                                          group_size=64, offset_dist=("uniform", -4, 4), with_x3=False)),
    ("pk_sm_m17_pergroup96_bf16_i8_partial", dict(act="bf16", weight="int8", x1_shape=(17, 1120), n=192,
                                                  mode="group", group_size=96)),
    ("pk_sm_m3_pergroup128_bf16_i4_3d", dict(act="bf16", weight="int4", x1_shape=(3, 1, 2048), n=256, mode="group",
                                             group_size=128)),
    ("pk_sm_m24_perchannel_fp16_i4_xt", dict(act="fp16", weight="int4", x1_shape=(24, 1024), n=384, mode="channel",
                                             x2_transposed=True)),
    ("pk_sm_m16_perchannel_bf16_f8", dict(act="bf16", weight="fp8e4m3", x1_shape=(16, 2048), n=320, mode="channel",
                                          with_offset=False, scale_dist=("uniform", 2e-4, 1e-3))),
    ("pk_sm_m32_pergroup64_fp16_i8_xt_wide", dict(act="fp16", weight="int8", x1_shape=(32, 2048), n=8192,
                                                  mode="group", group_size=64, x2_transposed=True)),
    # n >= 8192 with k > 1024: split k, a k tail, n not a multiple of the slab
    ("pk_wide_m32_pergroup128_bf16_i4", dict(act="bf16", weight="int4", x1_shape=(32, 2048), n=8192, mode="group",
                                           group_size=128, offset_dist=("uniform", -1, 1))),
    ("pk_wide_m9_perchannel_fp16_i8_ktail", dict(act="fp16", weight="int8", x1_shape=(9, 1056), n=8192,
                                               mode="channel")),
    ("pk_wide_m2_pertensor_bf16_i4_nooff", dict(act="bf16", weight="int4", x1_shape=(2, 1152), n=8256, mode="tensor",
                                              with_offset=False)),
    ("pk_sm_m5_pergroup32_bf16_i8_k96", dict(act="bf16", weight="int8", x1_shape=(5, 96), n=64, mode="group",
                                             group_size=32)),
    # large m: the tiled kernels' packed path (64-, 128-, 256-row tiles; split k; n edge; k tail)
    ("pk_tl_m40_perchannel_bf16_i8_split", dict(act="bf16", weight="int8", x1_shape=(40, 2048), n=320,
                                                mode="channel")),
    ("pk_tl_m100_pergroup96_fp16_i8_split", dict(act="fp16", weight="int8", x1_shape=(100, 2304), n=384,
                                                 mode="group", group_size=96, offset_dist=("uniform", -4, 4))),
    ("pk_tl_m300_pertensor_bf16_i4", dict(act="bf16", weight="int4", x1_shape=(300, 1024), n=320, mode="tensor")),
    ("pk_tl_m600_perchannel_bf16_i8_ktail", dict(act="bf16", weight="int8", x1_shape=(600, 288), n=544,
                                                 mode="channel")),
    ("pk_tl_m1100_pergroup128_bf16_i4_3d", dict(act="bf16", weight="int4", x1_shape=(2, 550, 512), n=320,
                                                mode="group", group_size=128, with_bias=False)),
    ("pk_tl_m257_perchannel_fp16_f8_xt", dict(act="fp16", weight="fp8e4m3", x1_shape=(257, 320), n=288,
                                              mode="channel", with_offset=False, scale_dist=("uniform", 2e-4, 1e-3),
                                              x2_transposed=True)),
    ("pk_tl_m200_pergroup64_bf16_i8_xt", dict(act="bf16", weight="int8", x1_shape=(200, 2048), n=256, mode="group",
                                              group_size=64, x2_transposed=True)),
    ("pk_tl_m1024_perchannel_fp16_i4", dict(act="fp16", weight="int4", x1_shape=(1024, 1024), n=1024,
                                            mode="channel")),
]


@pytest.mark.parametrize("name,spec", PACKED_CASES, ids=[c[0] for c in PACKED_CASES])
def test_packed_parity(name, spec):
    case = workloads.make_antiquant(seed=zlib.crc32(name.encode()) % 10000, name=name, **spec)
    check_packed(case)


@pytest.mark.parametrize("name", ["smallm_pergroup64_fp16_int8_32x8192x8192", "perchannel_bf16_int8_4096x4096x4096",
                                  "pergroup128_bf16_int4_4x2048x8192x2048",
                                  "smallm_perchannel_bf16_fp8e4m3_32x8192x8192"])
def test_full_size_packed(name):
    """Measured workloads with their weights prepacked: every output element."""
    check_packed(workloads.make_workload(name))


def test_packed_noalloc_and_graph():
    """The packed small-m call through the no-allocation entry point equals the ordinary call
    bit for bit, and replays from a HIP graph."""
    import ctypes
    _announce("packed_noalloc_graph")
    case = workloads.make_antiquant(seed=77, name="pk_graph", act="fp16", weight="int8", x1_shape=(16, 2048),
                                    n=256, mode="group", group_size=64)
    act = case.act
    pw = W.prepack_weight(_x2_dev(case))
    t = [dev_tensor(case.x1, act), pw, dev_tensor(case.scale, act), dev_tensor(case.offset, act),
         dev_tensor(case.bias, act), dev_tensor(case.x3, act)]
    call = W.AntiquantMatmul(*t, case.group_size)
    ref = call().clone()
    out = torch.empty_like(ref)
    r = lambda d: ctypes.byref(d) if d is not None else None
    descs = [W._desc(t[0]), pw.desc(), W._desc(t[4]), W._desc(t[2]), W._desc(t[3]), W._desc(t[5])]
    st = W.lib().wq_antiquant_matmul_noalloc(*map(r, descs), case.group_size, r(W._desc(out)),
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == W.WQ_OK
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        call.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.out.view(torch.int16), ref.view(torch.int16))
    res = oracle.compare(to_f64(ref).reshape(case.out_shape), ref_antiquant(case), act)
    assert res["ok"], res


# W8A8 on packed int8 weights: 256-, 128- and 64-row tiles, split k with a k tail, n not a
# multiple of the tile, 3-D x1, packed from a transposed weight, and the full-size workload
W8A8_PACKED_CASES = [
    ("pk_w8a8_ragged_bf16", dict(out="bf16", x1_shape=(600, 288), n=544)),
    ("pk_w8a8_fp16_tensor_nopt_3d", dict(out="fp16", x1_shape=(2, 130, 256), n=96, dequant="tensor",
                                         with_pertoken=False, with_bias=False)),
    ("pk_w8a8_m1", dict(out="bf16", x1_shape=(1, 128), n=64)),
    ("pk_w8a8_splitk_m300_tail_xt", dict(out="fp16", x1_shape=(300, 2080), n=320, x2_transposed=True)),
    ("pk_w8a8_rows64_m100_bf16dq", dict(out="bf16", x1_shape=(100, 2048), n=512, dequant_dtype="bf16")),
    ("pk_w8a8_rows128_m200", dict(out="bf16", x1_shape=(200, 4096), n=1024)),
]


@pytest.mark.parametrize("name,spec", W8A8_PACKED_CASES, ids=[c[0] for c in W8A8_PACKED_CASES])
def test_w8a8_packed_parity(name, spec):
    _announce(f"packed:{name}")
    case = workloads.make_w8a8(seed=zlib.crc32(name.encode()) % 10000, name=name, **spec)
    y, acc = run_w8a8(case, packed=True)
    ref, racc = ref_w8a8(case)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), racc)
    r = oracle.compare(to_f64(y).reshape(ref.shape), ref, case.out)
    assert r["ok"], (name, r)


def test_w8a8_full_size_packed():
    """The measured W8A8 workload with its weight prepacked: every output element, and the
    int32 accumulator bit for bit."""
    case = workloads.make_workload("w8a8_bf16_8192x4096x8192")
    _announce("packed:w8a8 full size")
    y, acc = run_w8a8(case, packed=True)
    ref, racc = ref_w8a8(case)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), racc)
    r = oracle.compare(to_f64(y).reshape(ref.shape), ref, case.out)
    assert r["ok"], r


# ---------------------------------------------------------------- seeded sweeps, packed
def _sweep_packed(count, seed, ms, kmax, prefix):
    """Random combinations of dtype, code type, mode, optional inputs, ragged shapes and a
    transposed source weight, all prepacked (small-m and tiled paths), from fixed seeds."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        act = str(rng.choice(["fp16", "bf16"]))
        weight = str(rng.choice(["int8", "int4", "fp8e4m3"], p=[0.45, 0.35, 0.2]))
        align = 64 if weight == "int4" else 32
        k = int(align * rng.integers(1, kmax + 1))
        n = int(align * rng.integers(1, 13))
        m = int(rng.choice(list(ms)))
        mode = "channel" if weight == "fp8e4m3" else str(rng.choice(["tensor", "channel", "group"]))
        g = 0
        if mode == "group":
            gs = list(range(32, k, 32))
            if gs:
                g = int(rng.choice(gs))
            else:
                mode = "channel"
        spec = dict(act=act, weight=weight, x1_shape=(m, k), n=n, mode=mode, group_size=g,
                    with_offset=weight != "fp8e4m3" and bool(rng.random() < 0.7),
                    with_bias=bool(rng.random() < 0.6), with_x3=bool(rng.random() < 0.6),
                    x2_transposed=bool(rng.random() < 0.3))
        if weight == "fp8e4m3":
            spec["scale_dist"] = ("uniform", 2e-4, 1e-3)
        out.append((f"{prefix}{i}_{act}_{weight}_{mode}{g or ''}_m{m}k{k}n{n}"
                    f"{'_xt' if spec['x2_transposed'] else ''}", spec))
    return out


PACKED_SWEEP = (_sweep_packed(24, 5151, (1, 3, 16, 31, 32), 40, "pksw")
                + _sweep_packed(24, 5252, (33, 64, 100, 129, 257, 600), 64, "pkswt"))


@pytest.mark.parametrize("name,spec", PACKED_SWEEP, ids=[c[0] for c in PACKED_SWEEP])
def test_packed_sweep(name, spec):
    check_packed(workloads.make_antiquant(seed=zlib.crc32(name.encode()) % 10000, name=name, **spec))


def _sweep_w8a8_packed(count=12, seed=5353):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        k = int(32 * rng.integers(1, 65))
        n = int(32 * rng.integers(1, 17))
        m = int(rng.choice([1, 5, 32, 77, 256, 300, 640]))
        out_dt = str(rng.choice(["fp16", "bf16"]))
        spec = dict(out=out_dt, x1_shape=(m, k), n=n, dequant=str(rng.choice(["tensor", "channel"])),
                    dequant_dtype=str(rng.choice(["fp32", "bf16"])) if out_dt == "bf16" else "fp32",
                    with_bias=bool(rng.random() < 0.7), with_pertoken=bool(rng.random() < 0.7),
                    with_x3=bool(rng.random() < 0.6), x2_transposed=bool(rng.random() < 0.4))
        out.append((f"pksw8_{i}_m{m}k{k}n{n}{'_xt' if spec['x2_transposed'] else ''}", spec))
    return out


W8A8_PACKED_SWEEP = _sweep_w8a8_packed()


@pytest.mark.parametrize("name,spec", W8A8_PACKED_SWEEP, ids=[c[0] for c in W8A8_PACKED_SWEEP])
def test_w8a8_packed_sweep(name, spec):
    _announce(f"packed:{name}")
    case = workloads.make_w8a8(seed=zlib.crc32(name.encode()) % 10000, name=name, **spec)
    y, acc = run_w8a8(case, packed=True)
    ref, racc = ref_w8a8(case)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), racc)
    r = oracle.compare(to_f64(y).reshape(ref.shape), ref, case.out)
    assert r["ok"], (name, r)

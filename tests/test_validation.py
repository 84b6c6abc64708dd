"""Argument validation through the C ABI's size queries (CPU; no device is touched).

Named rows follow the unit-test CSV rows the aclnnWeightQuantMatmulAllReduce guide lists
(section 单元测试); the other cases follow the rules of its constraint sections and of the
aclnnQuantMatmulAllReduceV2 page (Parameters, Constraints, Return Value).  Data pointers
are fake non-null addresses: the size query reads only the descriptors.
"""
import ctypes
import json
import os

import pytest

import weight_quantized_gemm_amd as W
from weight_quantized_gemm_amd import make_desc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FAKE = 0x10000
DT = {"fp16": W.WQ_F16, "bf16": W.WQ_BF16, "int8": W.WQ_I8, "int4": W.WQ_I4,
      "fp8e4m3": W.WQ_F8E4M3}
OK, NULLPTR, INVALID = W.WQ_OK, W.WQ_ERR_PARAM_NULLPTR, W.WQ_ERR_PARAM_INVALID


_next = [FAKE + 0x1000000]


def D(shape, dt, ptr=None, strides=None):
    """Descriptor with a fresh fake address unless one is given (0 = null data)."""
    if ptr is None:
        _next[0] += 0x100000
        ptr = _next[0]
    return make_desc(shape, dt, ptr, strides)


def aq(wqlib, x1, x2, scale, out, offset=None, bias=None, x3=None, g=0, ws=True):
    r = lambda d: ctypes.byref(d) if d is not None else None
    size = ctypes.c_uint64(0)
    return wqlib.wq_antiquant_matmul_get_workspace_size(
        r(x1), r(x2), r(bias), r(scale), r(offset), r(x3), g, r(out),
        ctypes.byref(size) if ws else None)


def base(act="fp16", w="int8", m=32, k=64, n=128, scale=None, g=0):
    a, wd = DT[act], DT[w]
    x1 = D([m, k], a, FAKE + 0x100000)
    x2 = D([k, n], wd, FAKE + 0x200000)
    sc = D(scale if scale is not None else [n], a, FAKE + 0x300000)
    out = D([m, n], a, FAKE + 0x400000)
    return x1, x2, sc, out


@pytest.mark.parametrize("row", json.load(open(os.path.join(GOLDEN, "ut_named_rows.json")))["rows"],
                         ids=lambda r: r["name"])
def test_named_ut_rows(wqlib, row):
    st = json.load(open(os.path.join(GOLDEN, "ut_named_rows.json")))["status"]
    a, wd = DT[row["act"]], DT[row["weight"]]
    x1 = D(row["x1"], a, FAKE + 0x100000)
    x2 = D(row["x2"], wd, FAKE + 0x200000)
    sc = D(row["scale"], a, FAKE + 0x300000)
    out = D(row["out"], a, FAKE + 0x400000)
    assert aq(wqlib, x1, x2, sc, out, g=row["group_size"]) == st[row["expect"]]


def test_null_required(wqlib):
    x1, x2, sc, out = base()
    assert aq(wqlib, None, x2, sc, out) == NULLPTR
    assert aq(wqlib, x1, None, sc, out) == NULLPTR
    assert aq(wqlib, x1, x2, None, out) == NULLPTR
    assert aq(wqlib, x1, x2, sc, None) == NULLPTR
    assert aq(wqlib, x1, x2, sc, out, ws=False) == NULLPTR
    x1n = D([32, 64], W.WQ_F16, 0)
    assert aq(wqlib, x1n, x2, sc, out) == NULLPTR
    # null checks come before dtype checks (the pages' order)
    bad = D([32, 64], W.WQ_F32, 0)
    assert aq(wqlib, bad, x2, sc, out) == NULLPTR


def test_dtypes(wqlib):
    x1, x2, sc, out = base()
    assert aq(wqlib, x1, x2, sc, out) == OK
    assert aq(wqlib, D([32, 64], W.WQ_F32), x2, sc, out) == INVALID
    assert aq(wqlib, x1, D([64, 128], W.WQ_F16), sc, out) == INVALID
    assert aq(wqlib, x1, x2, D([128], W.WQ_BF16), out) == INVALID           # scale != x1 dtype
    assert aq(wqlib, x1, x2, sc, out, x3=D([32, 128], W.WQ_BF16)) == INVALID  # illegal x3 dtype
    assert aq(wqlib, x1, x2, sc, out, bias=D([128], W.WQ_F32)) == INVALID
    assert aq(wqlib, x1, x2, sc, D([32, 128], W.WQ_BF16)) == INVALID
    assert aq(wqlib, x1, x2, sc, out, offset=D([128], W.WQ_BF16)) == INVALID


def test_group_size_rule(wqlib):
    # g = 0, or a multiple of 32 in [32, min(k-1, INT32_MAX)]
    for g, k, expect in [(32, 64, OK), (64, 128, OK), (96, 256, OK), (224, 256, OK),
                         (256, 256, INVALID), (16, 64, INVALID), (24, 64, INVALID),
                         (33, 128, INVALID), (-32, 128, INVALID), (64, 64, INVALID)]:
        groups = max(1, -(-k // g)) if g > 0 else 1
        x1, x2, sc, out = base(k=k, scale=[groups, 128])
        assert aq(wqlib, x1, x2, sc, out, g=g) == expect, (g, k)
    # partial last group: k = 96, g = 64 -> scale (2, n)
    x1, x2, sc, out = base(k=96, scale=[2, 128])
    assert aq(wqlib, x1, x2, sc, out, g=64) == OK
    x1, x2, sc, out = base(k=96, scale=[1, 128])
    assert aq(wqlib, x1, x2, sc, out, g=64) == INVALID


def test_scale_shapes(wqlib):
    for shape, expect in [([1], OK), ([128], OK), ([1, 128], OK), ([2, 128], INVALID),
                          ([127], INVALID), ([1, 1], INVALID), ([128, 1], INVALID)]:
        x1, x2, sc, out = base(scale=shape)
        assert aq(wqlib, x1, x2, sc, out) == expect, shape
    x1, x2, sc, out = base()
    assert aq(wqlib, x1, x2, sc, out, offset=D([1, 128], W.WQ_F16)) == INVALID  # offset != scale shape
    assert aq(wqlib, x1, x2, sc, out, offset=D([128], W.WQ_F16)) == OK


def test_shapes_and_ranges(wqlib):
    f16 = W.WQ_F16
    x1, x2, sc, out = base()
    assert aq(wqlib, D([32, 96], f16), x2, sc, out) == INVALID                # k mismatch
    assert aq(wqlib, x1, x2, sc, out, bias=D([64], f16)) == INVALID
    assert aq(wqlib, x1, x2, sc, out, x3=D([32, 64], f16)) == INVALID
    assert aq(wqlib, x1, x2, sc, D([31, 128], f16)) == INVALID
    assert aq(wqlib, D([32], f16), x2, sc, out) == INVALID                    # 1-D x1
    # 3-D activations: output follows x1
    x13 = D([2, 16, 64], f16)
    assert aq(wqlib, x13, x2, sc, D([2, 16, 128], f16)) == OK
    assert aq(wqlib, x13, x2, sc, D([32, 128], f16)) == INVALID
    assert aq(wqlib, D([2, 0, 64], f16, 0), x2, sc, D([2, 0, 128], f16, 0)) == INVALID
    # n == 0, k > 65535, alignment
    assert aq(wqlib, x1, D([64, 0], W.WQ_I8, 0), D([1], f16), D([32, 0], f16, 0)) == INVALID
    assert aq(wqlib, D([32, 65536], f16), D([65536, 128], W.WQ_I8), sc, out) == INVALID
    assert aq(wqlib, D([32, 48], f16), D([48, 128], W.WQ_I8), sc, out) == INVALID   # k % 32
    assert aq(wqlib, x1, D([64, 112], W.WQ_I8), D([112], f16), D([32, 112], f16)) == INVALID
    # int4 needs k, n multiples of 64
    assert aq(wqlib, x1, D([64, 128], W.WQ_I4), sc, out) == OK
    assert aq(wqlib, x1, D([64, 96], W.WQ_I4), D([96], f16), D([32, 96], f16)) == INVALID
    assert aq(wqlib, D([32, 96], f16), D([96, 128], W.WQ_I4), sc, out) == INVALID


def test_fp8_weight_rules(wqlib):
    """FLOAT8_E4M3FN weights (guide, support matrix 950 row and the note under the 950
    dtype table): per-channel scale only, no offset; one byte per element, so k and n
    are multiples of 32 as for int8."""
    for act in ("fp16", "bf16"):
        a = DT[act]
        x1, x2, sc, out = base(act=act, w="fp8e4m3")
        assert aq(wqlib, x1, x2, sc, out) == OK                                     # (n)
        assert aq(wqlib, x1, x2, D([1, 128], a), out, bias=D([128], a), x3=D([32, 128], a)) == OK
        assert aq(wqlib, x1, x2, D([1], a), out) == INVALID                         # per-tensor
        assert aq(wqlib, x1, x2, D([2, 128], a), out, g=32) == INVALID              # per-group
        assert aq(wqlib, x1, x2, sc, out, offset=D([128], a)) == INVALID            # offset
        # the same shapes with int8 weights are all accepted
        x2i = D([64, 128], W.WQ_I8)
        assert aq(wqlib, x1, x2i, D([1], a), out) == OK
        assert aq(wqlib, x1, x2i, D([2, 128], a), out, g=32) == OK
        assert aq(wqlib, x1, x2i, sc, out, offset=D([128], a)) == OK
    f16 = W.WQ_F16
    x1, x2, sc, out = base(w="fp8e4m3")
    assert aq(wqlib, D([32, 96], f16), D([96, 128], W.WQ_F8E4M3), sc, out) == OK   # k % 32
    assert aq(wqlib, D([32, 48], f16), D([48, 128], W.WQ_F8E4M3), sc, out) == INVALID
    assert aq(wqlib, x1, D([64, 112], W.WQ_F8E4M3), D([112], f16), D([32, 112], f16)) == INVALID
    # an offset with fp8 weights is refused whatever its shape; a null data pointer in it is
    # still a null-pointer error, as those are checked first
    assert aq(wqlib, x1, x2, sc, out, offset=D([7], f16)) == INVALID
    assert aq(wqlib, x1, x2, sc, out, offset=D([128], f16, 0)) == NULLPTR
    # empty K keeps the per-channel rule
    x1e, x2e = D([32, 0], f16, 0), D([0, 128], W.WQ_F8E4M3, 0)
    assert aq(wqlib, x1e, x2e, D([128], f16), D([32, 128], f16)) == OK
    assert aq(wqlib, x1e, x2e, D([0, 128], f16, 0), D([32, 128], f16), g=64) == INVALID


def test_transposed_x2(wqlib):
    """x2 may be the transpose of a row-major (n, k) tensor; per-group scale and offset go
    with it (guide, 参数说明); W8A8 likewise (Parameters table), and only then may n exceed
    65535 (Constraints)."""
    f16, bf16 = W.WQ_F16, W.WQ_BF16
    k, n = 64, 128
    x1 = D([32, k], f16, FAKE + 0x100000)
    out = D([32, n], f16, FAKE + 0x400000)
    for wd in (W.WQ_I8, W.WQ_I4, W.WQ_F8E4M3):
        xt = D([k, n], wd, None, [1, k])
        assert aq(wqlib, x1, xt, D([n], f16), out) == OK
        assert aq(wqlib, x1, xt, D([1, n], f16), out) == OK
    xt = D([k, n], W.WQ_I8, None, [1, k])
    assert aq(wqlib, x1, xt, D([1], f16), out, offset=D([1], f16)) == OK          # per-tensor
    # per-group: parameters transposed with x2, and only then
    gt, gr = D([2, n], f16, None, [1, 2]), D([2, n], f16)
    assert aq(wqlib, x1, xt, gt, out, offset=D([2, n], f16, None, [1, 2]), g=32) == OK
    assert aq(wqlib, x1, xt, gr, out, g=32) == INVALID
    assert aq(wqlib, x1, xt, gt, out, offset=D([2, n], f16), g=32) == INVALID
    xr = D([k, n], W.WQ_I8)
    assert aq(wqlib, x1, xr, gt, out, g=32) == INVALID
    assert aq(wqlib, x1, xr, gr, out, g=32) == OK
    # other strided layouts stay invalid
    assert aq(wqlib, x1, D([k, n], W.WQ_I8, None, [2 * n, 1]), D([n], f16), out) == INVALID
    assert aq(wqlib, x1, D([k, n], W.WQ_I8, None, [1, 2 * k]), D([n], f16), out) == INVALID
    # alignment still applies to the logical (k, n)
    assert aq(wqlib, x1, D([k, 96], W.WQ_I4, None, [1, k]), D([96], f16), D([32, 96], f16)) == INVALID
    # W8A8
    i8 = W.WQ_I8
    q1 = D([16, k], i8, FAKE + 0x100000)
    assert qm(wqlib, q1, D([k, n], i8, None, [1, k]), D([n], W.WQ_F32), D([16, n], bf16)) == OK
    big = 70016
    assert qm(wqlib, q1, D([k, big], i8, None, [1, k]), D([1], W.WQ_F32), D([16, big], bf16)) == OK
    assert qm(wqlib, q1, D([k, big], i8), D([1], W.WQ_F32), D([16, big], bf16)) == INVALID
    assert qm(wqlib, q1, D([k, n], i8, None, [2 * n, 1]), D([n], W.WQ_F32), D([16, n], bf16)) == INVALID


def test_empty_k(wqlib):
    f16 = W.WQ_F16
    x1, x2 = D([32, 0], f16, 0), D([0, 128], W.WQ_I8, 0)
    for scale, g in [([128], 0), ([1], 0), ([0, 128], 64), ([128], 16)]:
        assert aq(wqlib, x1, x2, D(scale, f16, FAKE if scale[0] else 0), D([32, 128], f16), g=g) == OK


def test_layout_and_alias(wqlib):
    f16 = W.WQ_F16
    x1, x2, sc, out = base()
    # a padded (non-contiguous) x2 is not accepted; its transpose is (test_transposed_x2)
    assert aq(wqlib, x1, D([64, 128], W.WQ_I8, None, [256, 1]), sc, out) == INVALID
    # the output may not alias an input
    assert aq(wqlib, x1, x2, sc, D([32, 128], f16, FAKE + 0x100000)) == INVALID
    # every tensor starts 16-byte aligned (the kernels move 16-byte pieces)
    assert aq(wqlib, D([32, 64], f16, FAKE + 0x900002), x2, sc, out) == INVALID
    assert aq(wqlib, x1, x2, sc, out, bias=D([128], f16, FAKE + 0x900008)) == INVALID
    assert aq(wqlib, x1, x2, sc, out, bias=D([128], f16, FAKE + 0x900010)) == OK
    assert qm(wqlib, D([16, 64], W.WQ_I8, FAKE + 0x900004), D([64, 128], W.WQ_I8), D([128], W.WQ_F32),
              D([16, 128], W.WQ_BF16)) == INVALID


def test_workspace_sizes(wqlib):
    import ctypes as C
    x1, x2, sc, out = base(m=32, k=8192, n=8192, scale=[128, 8192])
    size = C.c_uint64(0)
    r = C.byref
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(x2), None, r(sc), None, None, 64,
                                                        r(out), r(size)) == OK
    assert size.value > 0
    # a workspace smaller than required is refused before anything is launched
    st = wqlib.wq_antiquant_matmul(r(x1), r(x2), None, r(sc), None, None, 64, r(out),
                                   C.c_void_p(FAKE), C.c_uint64(size.value - 1), None)
    assert st == INVALID
    # a workspace that is not 256-byte aligned is refused too, before any launch
    st = wqlib.wq_antiquant_matmul(r(x1), r(x2), None, r(sc), None, None, 64, r(out),
                                   C.c_void_p(FAKE + 16), C.c_uint64(size.value), None)
    assert st == INVALID
    # large m, per-group with an offset: room for the row sums of x1 per group, (groups, m)
    # fp32, which feed the offset term s * (off - C) * S_g ...
    x1, x2, sc, out = base(m=300, k=1024, n=256, scale=[8, 256])
    off = D([8, 256], W.WQ_F16, FAKE + 0x500000)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(x2), None, r(sc), r(off), None, 128,
                                                        r(out), r(size)) == OK
    assert size.value >= 8 * 300 * 4
    # ... none without an offset when the images are exact (C = 0) ...
    size_no = C.c_uint64(0)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(x2), None, r(sc), None, None, 128,
                                                        r(out), r(size_no)) == OK
    assert size.value - size_no.value == 9728              # (8, 300) fp32 padded to 256
    # ... but bf16 images of int4 codes carry C = 136, so the row sums stay
    x1b, x2b, scb, outb = base(act="bf16", w="int4", m=300, k=1024, n=256, scale=[8, 256])
    size_b = C.c_uint64(0)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1b), r(x2b), None, r(scb), None, None, 128,
                                                        r(outb), r(size_b)) == OK
    size_b_off = C.c_uint64(0)
    offb = D([8, 256], W.WQ_BF16, FAKE + 0x500000)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1b), r(x2b), None, r(scb), r(offb), None, 128,
                                                        r(outb), r(size_b_off)) == OK
    assert size_b.value == size_b_off.value and size_b.value >= 9728
    # ... and transposed per-group parameters add two row-major copies
    xt = D([1024, 256], W.WQ_I8, None, [1, 1024])
    st_ = D([8, 256], W.WQ_F16, None, [1, 8])
    size_t = C.c_uint64(0)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(xt), None, r(st_),
                                                        r(D([8, 256], W.WQ_F16, FAKE + 0x500000, [1, 8])),
                                                        None, 128, r(out), r(size_t)) == OK
    assert size_t.value >= size.value + 2 * 8 * 256 * 2
    # per-channel large m: none while the tiles fill the 256 CUs (16 x 16 tiles of 256)...
    x1, x2, sc, out = base(m=4096, k=4096, n=4096)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(x2), None, r(sc), None, None, 0,
                                                        r(out), r(size)) == OK
    assert size.value == 0
    # ... else fp32 split-k partials and row sums: 256-row tiles would split k = 1024 into
    # chunks of 256, so the tiles are 128 rows (3 x 1 want 85 splits), but a split keeps at
    # least 256 k, so k = 1024 gives 4 splits
    x1, x2, sc, out = base(m=300, k=1024, n=256)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(x2), None, r(sc), None, None, 0,
                                                        r(out), r(size)) == OK
    assert size.value == 4 * 300 * 256 * 4 + 4864          # partials, then row sums padded to 256
    # per-group splits hold whole groups: g = 96 gives units of 192 and splits of at least
    # 384; 3 tiles of 128 rows want 85 splits, k = 2304 takes 6; then the row sums per group
    x1, x2, sc, out = base(m=300, k=2304, n=256, scale=[24, 256])
    off = D([24, 256], W.WQ_F16, FAKE + 0x500000)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(x2), None, r(sc), r(off), None, 96,
                                                        r(out), r(size)) == OK
    assert size.value == 6 * 300 * 256 * 4 + 28928          # partials, (24, 300) fp32 padded
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(x2), None, r(sc), None, None, 96,
                                                        r(out), r(size)) == OK
    assert size.value == 6 * 300 * 256 * 4                  # no offset, exact images: partials only
    # m <= 64 counts tiles of 64 rows: one tile, k = 1024 split in four
    x1, x2, sc, out = base(m=64, k=1024, n=256)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(x2), None, r(sc), None, None, 0,
                                                        r(out), r(size)) == OK
    assert size.value == 4 * 64 * 256 * 4 + 1024
    # beyond m = 128 the 256-row tiles stay where their split chunks would be over 512 long:
    # 256 x 16384 x 4096 has 16 such tiles, chunks of 1024, 16 splits (128-row tiles would
    # have taken 8); 512 x 4096 x 4096 would split 32 tiles into chunks of 512, so it takes
    # 64 tiles of 128 rows, chunks of 1024, 4 splits (256-row tiles would have taken 8)
    # and at 64 < m <= 128 the 64-row tiles likewise: 96 x 4096 x 4096 would split one row of
    # 16 tiles of 128 rows into chunks of 256, so it takes 2 x 16 tiles of 64 rows, 8 splits;
    # 128 x 8192 x 8192 keeps 128 rows (chunks of 1024, 8 splits; 64 rows would take 4)
    for (m, k, n), splits in (((256, 16384, 4096), 16), ((512, 4096, 4096), 4),
                              ((96, 4096, 4096), 8), ((128, 8192, 8192), 8)):
        x1, x2, sc, out = base(m=m, k=k, n=n)
        assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(x2), None, r(sc), None, None, 0,
                                                            r(out), r(size)) == OK
        assert size.value == splits * m * n * 4 + splits * m * 4, (m, k, n, size.value)
    # per-group too: 96 x 8192 x 2048 with g = 128 would split 8 tiles of 128 rows into chunks
    # of 256 (32 splits), so it takes 16 tiles of 64 rows, chunks of 512, 16 splits; then the
    # row sums per group, (64, 96) fp32
    x1, x2, sc, out = base(m=96, k=8192, n=2048, scale=[64, 2048])
    off = D([64, 2048], W.WQ_F16, FAKE + 0x500000)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(x2), None, r(sc), r(off), None, 128,
                                                        r(out), r(size)) == OK
    assert size.value == 16 * 96 * 2048 * 4 + 64 * 96 * 4
    # W8A8: int32 partials under the same rules (tiles of 256, 128 or 64 rows)
    i8 = W.WQ_I8
    for (m, k, n), want in (((4096, 4096, 4096), 0), ((32, 8192, 8192), 8 * 32 * 8192 * 4),
                            ((300, 1024, 256), 4 * 300 * 256 * 4),
                            ((256, 16384, 4096), 16 * 256 * 4096 * 4),
                            ((512, 4096, 4096), 4 * 512 * 4096 * 4),
                            ((96, 4096, 4096), 8 * 96 * 4096 * 4)):
        assert wqlib.wq_quant_matmul_get_workspace_size(
            r(D([m, k], i8)), r(D([k, n], i8)), None, None, r(D([n], W.WQ_F32)), None,
            r(D([m, n], W.WQ_BF16)), None, r(size)) == OK
        assert size.value == want, (m, k, n, size.value)


def qm(wqlib, x1, x2, dq, out, bias=None, x3=None, pt=None, acc=None):
    r = lambda d: ctypes.byref(d) if d is not None else None
    size = ctypes.c_uint64(0)
    return wqlib.wq_quant_matmul_get_workspace_size(r(x1), r(x2), r(bias), r(x3), r(dq), r(pt),
                                                    r(out), r(acc), ctypes.byref(size))


def test_w8a8_rules(wqlib):
    i8, i32, f32, bf, f16 = W.WQ_I8, W.WQ_I32, W.WQ_F32, W.WQ_BF16, W.WQ_F16
    x1, x2 = D([32, 64], i8, FAKE + 0x10000), D([64, 128], i8, FAKE + 0x20000)
    dq, out = D([128], f32, FAKE + 0x30000), D([32, 128], bf, FAKE + 0x40000)
    assert qm(wqlib, x1, x2, dq, out) == OK
    assert qm(wqlib, x1, x2, dq, out, bias=D([128], i32), x3=D([32, 128], bf),
              pt=D([32], f32), acc=D([32, 128], i32)) == OK
    assert qm(wqlib, None, x2, dq, out) == NULLPTR
    assert qm(wqlib, x1, x2, None, out) == NULLPTR
    assert qm(wqlib, x1, x2, dq, None) == NULLPTR
    assert qm(wqlib, D([32, 64], f16), x2, dq, out) == INVALID
    assert qm(wqlib, x1, x2, dq, out, bias=D([128], f32)) == INVALID
    assert qm(wqlib, x1, x2, D([128], W.WQ_I32), out) == INVALID          # packed int64 scale: no
    assert qm(wqlib, x1, x2, dq, D([32, 128], f32)) == INVALID
    assert qm(wqlib, x1, x2, dq, out, x3=D([32, 128], f16)) == INVALID     # x3 dtype != output
    assert qm(wqlib, x1, x2, dq, out, pt=D([31], f32)) == INVALID
    assert qm(wqlib, x1, x2, D([1], f32), out) == OK
    assert qm(wqlib, x1, x2, D([1, 128], bf), out) == OK
    assert qm(wqlib, x1, x2, D([2, 128], f32), out) == INVALID
    assert qm(wqlib, D([32, 0], i8, 0), D([0, 128], i8, 0), dq, out) == INVALID  # no empty tensors
    assert qm(wqlib, D([2, 16, 64], i8), x2, dq, D([2, 16, 128], bf), pt=D([32], f32)) == OK


@pytest.mark.parametrize("out_dt,dq_dt,with_pt,want", [
    # FLOAT16 output: FLOAT32 with a pertoken scale; without one the pages' packed
    # INT64/UINT64 form, which FLOAT32 replaces here; never BFLOAT16
    ("fp16", "fp32", True, "ok"), ("fp16", "fp32", False, "ok"),
    ("fp16", "bf16", True, "invalid"), ("fp16", "bf16", False, "invalid"),
    ("fp16", "fp16", True, "invalid"), ("fp16", "i32", False, "invalid"),
    # BFLOAT16 output: BFLOAT16 (the pages' type) or FLOAT32 (the W8A8 workload's)
    ("bf16", "bf16", True, "ok"), ("bf16", "bf16", False, "ok"),
    ("bf16", "fp32", True, "ok"), ("bf16", "fp32", False, "ok"),
    ("bf16", "fp16", False, "invalid"), ("bf16", "i32", True, "invalid"),
])
def test_w8a8_dequant_dtype_rule(wqlib, out_dt, dq_dt, with_pt, want):
    """aclnnQuantMatmulAllReduceV2, Constraints: the dequant scale's dtype follows the output
    dtype and the presence of a pertoken scale."""
    code = {"fp16": W.WQ_F16, "bf16": W.WQ_BF16, "fp32": W.WQ_F32, "i32": W.WQ_I32}
    i8 = W.WQ_I8
    x1, x2 = D([32, 64], i8, FAKE + 0x10000), D([64, 128], i8, FAKE + 0x20000)
    for dq_shape in ([1], [128], [1, 128]):
        st = qm(wqlib, x1, x2, D(dq_shape, code[dq_dt], FAKE + 0x30000), D([32, 128], code[out_dt], FAKE + 0x40000),
                pt=D([32], W.WQ_F32, FAKE + 0x50000) if with_pt else None)
        assert st == (OK if want == "ok" else INVALID), (out_dt, dq_dt, with_pt, dq_shape, st)

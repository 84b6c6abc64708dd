"""The NumPy restatement of the packed weight layout (tests/packing.py) and the prepack's size
query and argument rules through the C ABI (CPU; no device is touched)."""
import ctypes

import numpy as np
import pytest

import weight_quantized_gemm_amd as W
from packing import pack_reference, unpack_reference, logical_codes


@pytest.mark.parametrize("int4,k,n", [(False, 64, 32), (False, 96, 64), (False, 192, 96), (True, 64, 64),
                                        (True, 128, 192)])
def test_pack_roundtrip(int4, k, n):
    rng = np.random.default_rng(k * 7 + n)
    codes = rng.integers(-8, 8, size=(k, n)) if int4 else rng.integers(-128, 128, size=(k, n))
    packed = pack_reference(codes, int4)
    assert packed.size == -(-k // 64) * (n // 32) * (1024 if int4 else 2048)
    got = unpack_reference(packed, k, n, int4)
    if not int4:
        got = got.astype(np.uint8).astype(np.int8)
    assert np.array_equal(got, codes)


def test_pack_hand_positions():
    """Positions worked out by hand from the layout's definition: codes[k, c] = k + 2 c
    (mod 128) for a 96 x 64 int8 weight (two k blocks, two column blocks; the second k block
    is half padding)."""
    k, n = 96, 64
    kk, cc = np.meshgrid(np.arange(k), np.arange(n), indexing="ij")
    codes = (kk + 2 * cc) % 128
    p = pack_reference(codes, False)
    # block (k block 0, column block 0), step 0, lane 0 (column 0, k 0..7): 0, 1, .., 7
    assert list(p[0:8]) == [0, 1, 2, 3, 4, 5, 6, 7]
    # lane 33 (column 1, k 8..15): 10, 11, .., 17
    assert list(p[33 * 8:33 * 8 + 8]) == [10, 11, 12, 13, 14, 15, 16, 17]
    # step 2, lane 5 (column 5, k 32..39): 42 .. 49
    off = (2 * 64 + 5) * 8
    assert list(p[off:off + 8]) == [42, 43, 44, 45, 46, 47, 48, 49]
    # block (k block 0, column block 1) starts at 2048: step 0, lane 0 = column 32: 64 .. 71
    assert list(p[2048:2056]) == [64, 65, 66, 67, 68, 69, 70, 71]
    # block (k block 1, column block 0) at 4096: step 1, lane 40 (column 8, k 64+16+8 = 88):
    # 88 + 16 = 104 .. 111; step 2 is padding (k 96..) -> zeros
    off = 4096 + (1 * 64 + 40) * 8
    assert list(p[off:off + 8]) == [104, 105, 106, 107, 108, 109, 110, 111]
    off = 4096 + (2 * 64 + 3) * 8
    assert list(p[off:off + 8]) == [0] * 8


def test_pack_int4_nibble_order():
    """int4: a byte holds one k of a lane's column in both blocks of a pair, the even block's
    code in bits 0-3; one byte per k, k ascending (positions worked out by hand)."""
    codes = np.zeros((64, 128), dtype=np.int64)
    codes[0, 0], codes[0, 32], codes[1, 0] = 3, -2, 7     # lane 0, step 0: e = 0 (both blocks), e = 1
    codes[8, 1], codes[8, 33] = 5, -8                     # lane 33 (column 1, k 8..15), e = 0
    codes[63, 31] = -1                                    # step 3, lane 63 (column 31, k 56..63), e = 7
    codes[0, 64], codes[2, 96] = 6, 1                     # the second pair (columns 64..127) at 2048
    p = pack_reference(codes, True)
    assert p.size == 4096
    assert p[0] == (3 | ((-2 & 0xF) << 4))
    assert p[1] == 7
    assert p[33 * 8] == (5 | (8 << 4))
    assert p[(3 * 64 + 63) * 8 + 7] == 0xF
    assert p[2048] == 6 and p[2048 + 2] == (1 << 4)
    assert int(np.count_nonzero(p)) == 6                   # columns 0 and 32 share byte 0


def test_logical_codes_int4_layouts():
    """Row-major int4 storage packs along n, transposed storage along k: both decode to the
    same logical (k, n) codes."""
    rng = np.random.default_rng(5)
    v = rng.integers(-8, 8, size=(64, 128))
    u = (v & 0xF).astype(np.uint8)
    row = u[:, 0::2] | (u[:, 1::2] << 4)
    vt = v.T
    ut = (vt & 0xF).astype(np.uint8)
    tr = ut[:, 0::2] | (ut[:, 1::2] << 4)
    assert np.array_equal(logical_codes(row, "int4"), v)
    assert np.array_equal(logical_codes(tr, "int4", transposed=True), v)


def _size(wqlib, d):
    s = ctypes.c_uint64(0)
    st = wqlib.wq_prepack_weight_get_size(ctypes.byref(d), ctypes.byref(s))
    return st, s.value


def test_prepack_size_and_rules(wqlib):
    D = W.make_desc
    i8, i4, f8 = W.WQ_I8, W.WQ_I4, W.WQ_F8E4M3
    assert _size(wqlib, D([8192, 8192], i8, 0x1000)) == (W.WQ_OK, 128 * 256 * 2048)
    assert _size(wqlib, D([96, 64], f8, 0x1000)) == (W.WQ_OK, 2 * 2 * 2048)
    assert _size(wqlib, D([128, 128], i4, 0x1000)) == (W.WQ_OK, 2 * 4 * 1024)
    # transposed storage: same size
    assert _size(wqlib, D([4096, 256], i8, 0x1000, [1, 4096])) == (W.WQ_OK, 64 * 8 * 2048)
    assert _size(wqlib, D([96, 64], i4, 0x1000))[0] == W.WQ_ERR_PARAM_INVALID      # int4: k % 64
    assert _size(wqlib, D([64, 48], i8, 0x1000))[0] == W.WQ_ERR_PARAM_INVALID      # n % 32
    assert _size(wqlib, D([0, 64], i8, 0x1000))[0] == W.WQ_ERR_PARAM_INVALID       # k >= 1
    assert _size(wqlib, D([64, 64], W.WQ_BF16, 0x1000))[0] == W.WQ_ERR_PARAM_INVALID
    assert _size(wqlib, D([64, 64], i8, 0x1000, [1, 1]))[0] == W.WQ_ERR_PARAM_INVALID  # not a layout
    assert _size(wqlib, D([64, 64], i8, 0))[0] == W.WQ_ERR_PARAM_NULLPTR
    assert wqlib.wq_prepack_weight_get_size(None, None) == W.WQ_ERR_PARAM_NULLPTR
    # the run call checks its output descriptor before touching a device
    x2 = D([64, 64], i8, 0x100000)
    fn = wqlib.wq_prepack_weight
    assert fn(ctypes.byref(x2), None, None) == W.WQ_ERR_PARAM_NULLPTR
    for bad in (D([64, 64], i8, 0x200000),                      # dtype without the flag
                D([64, 64], i4 | W.WQ_PACKED, 0x200000),        # another code type
                D([64, 32], i8 | W.WQ_PACKED, 0x200000),        # another shape
                D([64, 64], i8 | W.WQ_PACKED, 0x100000),        # x2's own buffer
                D([64, 64], i8 | W.WQ_PACKED, 0x200008)):       # not 16-byte aligned
        assert fn(ctypes.byref(x2), ctypes.byref(bad), None) == W.WQ_ERR_PARAM_INVALID


def test_packed_weight_in_the_size_query(wqlib):
    """A packed x2 is accepted by the anti-quant size query (the same workspace as the ND
    weight: the same kernels' splits) and, int8 only, by the W8A8 one; the anti-quant call
    takes row-major per-group parameters only with it."""
    D, r = W.make_desc, ctypes.byref
    f16, i8 = W.WQ_F16, W.WQ_I8
    size = ctypes.c_uint64(0)
    x1 = D([32, 8192], f16, 0x100000)
    pk = D([8192, 8192], i8 | W.WQ_PACKED, 0x200000, [0, 0])
    sc, of = D([128, 8192], f16, 0x300000), D([128, 8192], f16, 0x400000)
    out = D([32, 8192], f16, 0x500000)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(pk), None, r(sc), r(of), None, 64, r(out),
                                                        r(size)) == W.WQ_OK
    packed_ws = size.value
    nd = D([8192, 8192], i8, 0x200000)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(nd), None, r(sc), r(of), None, 64, r(out),
                                                        r(size)) == W.WQ_OK
    assert size.value == packed_ws > 0
    sct = D([128, 8192], f16, 0x300000, [1, 128])
    oft = D([128, 8192], f16, 0x400000, [1, 128])
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(pk), None, r(sct), r(oft), None, 64, r(out),
                                                        r(size)) == W.WQ_ERR_PARAM_INVALID
    # W8A8 takes a packed int8 weight, and no other packed code type
    q1, q2 = D([32, 64], i8, 0x100000), D([64, 128], i8 | W.WQ_PACKED, 0x200000, [0, 0])
    dq, qo = D([128], W.WQ_F32, 0x300000), D([32, 128], W.WQ_BF16, 0x400000)
    assert wqlib.wq_quant_matmul_get_workspace_size(r(q1), r(q2), None, None, r(dq), None, r(qo), None,
                                                    r(size)) == W.WQ_OK
    for bad in (W.WQ_I4 | W.WQ_PACKED, W.WQ_F8E4M3 | W.WQ_PACKED):
        q2b = D([64, 128], bad, 0x200000, [0, 0])
        assert wqlib.wq_quant_matmul_get_workspace_size(r(q1), r(q2b), None, None, r(dq), None, r(qo), None,
                                                        r(size)) == W.WQ_ERR_PARAM_INVALID

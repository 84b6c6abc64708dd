"""The C-ABI library loads and exports every function include/wqgemm.h declares (CPU)."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "wqgemm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(wq_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_api():
    names = declared_functions()
    assert names == sorted(["wq_antiquant_matmul_get_workspace_size", "wq_antiquant_matmul",
                            "wq_antiquant_matmul_noalloc", "wq_prepack_weight_get_size", "wq_prepack_weight",
                            "wq_quant_matmul_get_workspace_size", "wq_quant_matmul",
                            "wq_profile_next_call", "wq_status_string", "wq_version"])


def test_library_exports_every_declared_symbol(wqlib):
    for name in declared_functions():
        assert hasattr(wqlib, name), name


def test_binding_names_match_header():
    import weight_quantized_gemm_amd as W
    assert sorted(W.EXPORTS) == declared_functions()


def test_status_strings(wqlib):
    import weight_quantized_gemm_amd as W
    assert wqlib.wq_status_string(W.WQ_OK) == b"WQ_OK"
    assert b"NULLPTR" in wqlib.wq_status_string(161001)
    assert b"INVALID" in wqlib.wq_status_string(161002)
    assert b"SCRATCH" in wqlib.wq_status_string(W.WQ_ERR_SCRATCH_LIMIT)
    assert wqlib.wq_version() >= 100


def test_profile_hook_arguments(wqlib):
    """The hook takes both events or neither; arming and disarming touch no device."""
    import ctypes
    import weight_quantized_gemm_amd as W
    fn = wqlib.wq_profile_next_call
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert fn(None, None) == W.WQ_OK
    assert fn(ctypes.c_void_p(0x10), None) == W.WQ_ERR_PARAM_NULLPTR
    assert fn(None, ctypes.c_void_p(0x10)) == W.WQ_ERR_PARAM_NULLPTR


def test_noalloc_refuses_calls_beyond_its_scratch(wqlib):
    """The no-allocation entry point checks the arguments and the workspace the call needs
    before anything else: invalid arguments return the size query's status, and a call that
    needs more than WQ_NOALLOC_SCRATCH_BYTES returns WQ_ERR_SCRATCH_LIMIT.  Neither touches a
    device (fake data pointers)."""
    import ctypes
    import weight_quantized_gemm_amd as W
    D, bf, i8 = W.make_desc, W.WQ_BF16, W.WQ_I8
    r = ctypes.byref
    # 256 x 16384 x 16384 per-channel: 64 tiles, so k splits four ways: 64 MiB of partials
    m, k, n = 256, 16384, 16384
    x1, x2 = D([m, k], bf, 0x100000), D([k, n], i8, 0x200000)
    sc, out = D([n], bf, 0x300000), D([m, n], bf, 0x400000)
    size = ctypes.c_uint64(0)
    assert wqlib.wq_antiquant_matmul_get_workspace_size(r(x1), r(x2), None, r(sc), None, None, 0, r(out),
                                                        r(size)) == W.WQ_OK
    assert size.value > W.WQ_NOALLOC_SCRATCH_BYTES
    fn = wqlib.wq_antiquant_matmul_noalloc
    assert fn(r(x1), r(x2), None, r(sc), None, None, 0, r(out), None) == W.WQ_ERR_SCRATCH_LIMIT
    assert fn(None, r(x2), None, r(sc), None, None, 0, r(out), None) == W.WQ_ERR_PARAM_NULLPTR
    bad = D([m, n + 32], bf, 0x400000)
    assert fn(r(x1), r(x2), None, r(sc), None, None, 0, r(bad), None) == W.WQ_ERR_PARAM_INVALID

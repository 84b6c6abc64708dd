"""The oracle against its pins (CPU only)."""
import oracle_pins as P
import oracle


def test_bruteforce_antiquant():
    P.pin_bruteforce(oracle.ref_antiquant)


def test_bruteforce_w8a8():
    P.pin_bruteforce_w8a8(oracle.ref_w8a8)


def test_page_sample_antiquant():
    P.pin_page_sample_antiquant(oracle.ref_antiquant)


def test_page_sample_w8a8():
    P.pin_page_sample_w8a8(oracle.ref_w8a8)


def test_worked_onehot():
    P.pin_worked_onehot(oracle.ref_antiquant)


def test_decoding():
    P.pin_decoding(oracle.decode_bf16, oracle.unpack_int4)


def test_identity():
    P.pin_identity(oracle.ref_antiquant)


def test_granularity():
    P.pin_granularity(oracle.ref_antiquant)


def test_empty_k():
    P.pin_empty_k(oracle.ref_antiquant)


def test_w8a8_exact():
    P.pin_w8a8_exact(oracle.ref_w8a8_acc)


def test_invariants():
    P.pin_invariants(oracle.ref_antiquant)


def test_compare_tolerance():
    import numpy as np
    ref = np.array([0.0, 0.5, 100.0, -300.0])
    ok = ref + np.array([1.9e-3, -1.9e-3, 0.19, -0.59])
    assert oracle.compare(ok, ref, "fp16")["ok"]
    bad = ref + np.array([0, 0, 0.21, 0])
    r = oracle.compare(bad, ref, "fp16")
    assert not r["ok"] and r["n_fail"] == 1 and r["worst_index"] == (2,)
    assert not oracle.compare(np.array([np.nan]), np.array([0.0]), "bf16")["ok"]


def test_fp8_decode():
    P.pin_fp8_decode(oracle.decode_fp8e4m3)


def test_bruteforce_fp8():
    P.pin_bruteforce_fp8(oracle.ref_antiquant)


def test_bruteforce_transposed():
    P.pin_bruteforce_transposed(oracle.ref_antiquant)


def test_int4_kpacked():
    P.pin_int4_kpacked(oracle.ref_antiquant)


def test_bruteforce_w8a8_transposed():
    P.pin_bruteforce_w8a8_transposed(oracle.ref_w8a8)

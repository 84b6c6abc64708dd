"""Host-side checks of the benchmark (no GPU): the algorithmic bytes and flops it divides by
are the ones the measured configurations define, every workload names its dominant kernel
and bound, the HBM-traffic figure is withheld once the kernel sources change, and a
request for more than one GPU is refused."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402

# Each input read once at its stored width plus the 16-bit output written once, and 2MNK:
# the per-configuration totals of the measured shapes (x1, x2, scale / dequant, offset /
# pertoken, bias, x3, output).
EXPECTED = {
    "tiny_pertensor_fp16_int8_16x256x256": (90_628, 2.097152e6),
    "perchannel_bf16_int8_4096x4096x4096": (117_465_088, 137.438953472e9),
    "pergroup128_bf16_int4_4x2048x8192x2048": (210_239_488, 274.877906944e9),
    "smallm_pergroup64_fp16_int8_32x8192x8192": (72_368_128, 4.294967296e9),
    "w8a8_bf16_8192x4096x8192": (335_642_624, 549.755813888e9),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_algorithmic_work(name):
    case = workloads.make_workload(name)
    nbytes, flops = EXPECTED[name]
    assert bench.algorithmic_bytes(case) == nbytes
    assert workloads.workload_flops(name) == pytest.approx(flops, rel=1e-12)
    assert 2.0 * case.m * case.k * case.n == pytest.approx(flops, rel=1e-12)


def test_every_workload_has_a_dominant_kernel():
    assert set(bench.DOMINANT) == set(workloads.WORKLOADS)
    for kernel, bound in bench.DOMINANT.values():
        assert kernel in ("aq_gemm_kernel", "aq_smallm_kernel", "qm_gemm_kernel")
        assert bound in ("mfma", "hbm")


def test_traffic_withheld_for_other_sources(monkeypatch):
    name = bench.HEADLINE
    kernel = bench.DOMINANT[name][0]
    monkeypatch.setattr(bench, "source_digest", lambda: "not-the-profiled-sources")
    assert bench.traffic_for(kernel, name) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_roofline_from_kernel_durations():
    """The roofline divides the algorithmic work by the kernel's average duration; an event
    average above the mean step (which must contain the kernel) is replaced by the step."""
    r = bench.make_roofline("mfma", "bf16", 137.438953472e9, 117_465_088, [0.100, 0.110, 0.105], 0.112)
    assert r["launch_us_avg"] == pytest.approx(105.0) and r["kernel_time"] == "kernel events"
    assert r["achieved"] == pytest.approx(137.438953472e9 / 105e-6 / 1e12, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0, rel=1e-3)
    h = bench.make_roofline("hbm", "fp16", 4.29e9, 72_368_128, [0.020, 0.022], 0.025)
    assert h["unit"] == "GB/s" and h["achieved"] == pytest.approx(72_368_128 / 21e-6 / 1e9, rel=1e-3)
    b = bench.make_roofline("mfma", "bf16", 1e9, 1, [0.168, 0.167], 0.162)
    assert b["launch_us_avg"] == pytest.approx(162.0) and b["events_us_avg"] == pytest.approx(167.5)
    assert b["kernel_time"].startswith("mean step")
    assert b["launch_us_avg"] <= 162.0


def test_hooked_steps():
    """Which timed steps carry the kernel events: every fifth by default, at least one."""
    assert bench.hooked_steps("sampled", 50, 5) == [4, 9, 14, 19, 24, 29, 34, 39, 44, 49]
    assert bench.hooked_steps("sampled", 3, 5) == [2]
    assert bench.hooked_steps("sampled", 7, 1) == list(range(7))
    assert bench.hooked_steps("timed", 4, 5) == [0, 1, 2, 3]
    assert bench.hooked_steps("after", 4, 5) == []

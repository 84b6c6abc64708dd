#!/usr/bin/env python3
"""Benchmark of the weight-anti-quant matmul (and its W8A8 sibling) on one MI355X.

A step is one call of the library on one batch of resident synthetic inputs: for the
anti-quant workloads x1 @ ((x2 + offset) * scale) + bias + x3, for the W8A8 workload
dequant_scale * pertoken_scale * (x1 @ x2 + bias) + x3.  Inputs are drawn by the seeded
generators in ``workloads`` and copied to HBM before timing.  Several input sets are
rotated so that the footprint of consecutive steps exceeds the 256 MB Infinity Cache: the
timed steps read their operands from HBM, not from a warm cache.

Each input set gets a prepared call (descriptors and workspace settled once), so the host
enqueues steps faster than the device runs them.  The timed region covers exactly the
timed steps, bracketed by device synchronisation.  In every fifth timed step the
library's profiling hook passes a pair of HIP events with the launch of the step's main
kernel (hipExtLaunchKernel), so that they take that kernel's own start and end on its
launch stream; their average is the kernel duration of the roofline.  The events are
created without a system-scope fence; a hooked launch still costs the stream a few
microseconds, which is why only a sample of the steps carries them.

Output: one JSON line (the headline workload), with the roofline of the dominant kernel
and the CPU oracle's rate on the host as a baseline.  ``--all`` prints one line per
workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "TFLOP/s and HBM GB/s (% of MI355X peak) for anti-quant GEMM+bias+x3"
HEADLINE = "perchannel_bf16_int8_4096x4096x4096"
# MI355X published peaks: dense MFMA bf16/fp16 2.5 PFLOP/s, int8 5.0 POP/s; HBM3E 8 TB/s.
PEAK = {"bf16": 2500.0, "fp16": 2500.0, "int8": 5000.0}   # TFLOP/s (TOP/s)
PEAK_HBM = 8000.0                                          # GB/s
# the kernel that dominates each workload's step, and what bounds it
DOMINANT = {
    "tiny_pertensor_fp16_int8_16x256x256": ("aq_smallm_kernel", "hbm"),
    "perchannel_bf16_int8_4096x4096x4096": ("aq_gemm_kernel", "mfma"),
    "pergroup128_bf16_int4_4x2048x8192x2048": ("aq_gemm_kernel", "mfma"),
    "smallm_pergroup64_fp16_int8_32x8192x8192": ("aq_smallm_kernel", "hbm"),
    "w8a8_bf16_8192x4096x8192": ("qm_gemm_kernel", "mfma"),
    "perchannel_bf16_fp8e4m3_4096x4096x4096": ("aq_gemm_kernel", "mfma"),
    "smallm_perchannel_bf16_fp8e4m3_32x8192x8192": ("aq_smallm_kernel", "hbm"),
    "midm_perchannel_bf16_int8_128x8192x8192": ("aq_gemm_kernel", "hbm"),
    "midm_w8a8_bf16_128x8192x8192": ("qm_gemm_kernel", "hbm"),
}
CACHE_BYTES = 256 << 20


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_quantized_gemm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(case) -> int:
    total = sum(int(a.nbytes) for a in case.arrays().values())
    out_elems = int(np.prod(case.out_shape))
    return total + 2 * out_elems          # fp16 / bf16 output written once


def to_dev(a, kind, torch, dev):
    if a is None:
        return None
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def make_runner(case, torch, dev, sets, packed=False):
    """Device-resident input sets and one prepared call per set.  With `packed`, each set's
    weight is converted once to the packed layout (wq_prepack_weight) before any timing, as
    an offline weight conversion would be."""
    import weight_quantized_gemm_amd as W
    calls, bufs = [], []
    if isinstance(case, workloads.AntiquantCase):
        act = case.act
        int4 = case.weight == "int4"
        ws = None
        for s in range(sets):
            # extra sets are copies of the same values at other addresses
            x2 = to_dev(case.x2, "raw", torch, dev)
            if case.weight == "fp8e4m3":
                x2 = x2.view(torch.float8_e4m3fn)
            if packed:
                x2 = W.prepack_weight(x2, x2_int4=int4)
            b = dict(x1=to_dev(case.x1, act, torch, dev), x2=x2,
                     scale=to_dev(case.scale, act, torch, dev), offset=to_dev(case.offset, act, torch, dev),
                     bias=to_dev(case.bias, act, torch, dev), x3=to_dev(case.x3, act, torch, dev))
            b["out"] = torch.empty(case.out_shape, dtype=b["x1"].dtype, device=dev)
            c = W.AntiquantMatmul(b["x1"], b["x2"], b["scale"], b["offset"], b["bias"], b["x3"],
                                  case.group_size, x2_int4=int4, out=b["out"], workspace=ws)
            ws = c.workspace  # one workspace serves every set (the steps run in stream order)
            calls.append(c)
            bufs.append(b)
        return calls, bufs
    odt = torch.bfloat16 if case.out == "bf16" else torch.float16
    for s in range(sets):
        x2 = to_dev(case.x2, "raw", torch, dev)
        if packed:
            x2 = W.prepack_weight(x2)
        b = dict(x1=to_dev(case.x1, "raw", torch, dev), x2=x2,
                 dq=to_dev(case.dequant_scale, case.dequant_dtype, torch, dev),
                 pt=to_dev(case.pertoken_scale, "fp32", torch, dev), bias=to_dev(case.bias, "raw", torch, dev),
                 x3=to_dev(case.x3, case.out, torch, dev))
        b["out"] = torch.empty(case.out_shape, dtype=odt, device=dev)
        calls.append(W.QuantMatmul(b["x1"], b["x2"], b["dq"], b["pt"], b["bias"], b["x3"], out=b["out"]))
        bufs.append(b)
    return calls, bufs


def cpu_baseline(case, name, budget_s=10.0, max_runs=20):
    """The oracle as it stands, on the host cores: the whole workload, repeated until about
    budget_s seconds of CPU work (at most max_runs runs); the rate is from the mean run."""
    import oracle
    blas = []
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([d.get("num_threads", 1) for d in info] or [1])
        blas = [f"{d.get('internal_api')} {d.get('version')} ({d.get('num_threads')} threads)" for d in info]
    except Exception:  # threadpoolctl missing: report the visible cores
        threads = os.cpu_count() or 1
    times = []
    while not times or (sum(times) < budget_s and len(times) < max_runs):
        t0 = time.perf_counter()
        if isinstance(case, workloads.AntiquantCase):
            oracle.ref_antiquant(case.x1, case.x2, case.scale, case.offset, case.bias, case.x3,
                                 case.group_size, act=case.act, weight=case.weight)
        else:
            oracle.ref_w8a8(case.x1, case.x2, case.dequant_scale, case.pertoken_scale, case.bias, case.x3,
                            dequant_dtype=case.dequant_dtype, out=case.out)
        times.append(time.perf_counter() - t0)
    dt = sum(times) / len(times)
    flops = 2.0 * case.m * case.k * case.n
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the whole workload, {len(times)} runs ({sum(times):.1f} s of CPU work), fp64 NumPy/BLAS",
            "seconds_per_run": round(dt, 3),
            "host": {"os_cpu_count": os.cpu_count(), "cpu_model": cpu_model(), "blas": blas}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None



def traffic_for(kernel, name):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(name)
    if not rec or rec.get("source_digest") != source_digest() or rec.get("kernel") != kernel:
        return None
    return rec.get("hbm_bytes_per_launch")


def make_roofline(bound, dtype, flops, abytes, launch_ms, ms_per_step):
    """The roofline entry of the dominant kernel from its per-launch durations (ms, one per
    hooked step).  Each step launches that kernel once, so the kernel cannot take longer
    than the mean step of a back-to-back stream; an event average above it (the events'
    own overhead, e.g. under a tracing profiler) is replaced by the mean step, an upper
    bound on the kernel's duration, and the entry says so.  The events' own figures are
    kept under events_us_*."""
    per = sorted(launch_ms)
    ev_ms = sum(per) / len(per)
    bounded = ev_ms > ms_per_step
    avg_ms = ms_per_step if bounded else ev_ms
    avg_s = avg_ms / 1e3
    if bound == "mfma":
        achieved = flops / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK[dtype], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK[dtype], 4)}
    else:
        achieved = abytes / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM, 4)}
    roof["launch_us_avg"] = round(avg_ms * 1e3, 2)
    roof["kernel_time"] = "mean step (events above it)" if bounded else "kernel events"
    roof["events_us_avg"] = round(ev_ms * 1e3, 2)
    roof["events_us_median"] = round(per[len(per) // 2] * 1e3, 2)
    roof["events_us_min"] = round(per[0] * 1e3, 2)
    roof["events_us_max"] = round(per[-1] * 1e3, 2)
    return roof


def hooked_steps(mode, steps, every):
    """The timed steps that carry the profiling hook's events: every `every`-th one
    (`sampled`, at least the last), all (`timed`), or none (`after`: the events go to as many
    steps after the timed ones)."""
    if mode == "timed":
        return list(range(steps))
    if mode == "after" or steps < 1:
        return []
    every = max(1, every)
    return [i for i in range(steps) if i % every == every - 1] or [steps - 1]


def _hip_runtime():
    """The HIP runtime this process already uses (torch's, which the library shares)."""
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1]
            if "libamdhip64" in os.path.basename(path):
                return ctypes.CDLL(path)
    return ctypes.CDLL("libamdhip64.so")


class KernelEvents:
    """Pairs of HIP timing events for the profiling hook, created without the system-scope
    fence that a default event's record performs (hipEventDisableSystemFence): the hook
    records a pair at every timed step, and fenced records would add several microseconds of
    stream time to each step, more than a small call takes."""

    NO_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        rt = _hip_runtime()
        rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        for f in (rt.hipEventCreateWithFlags, rt.hipEventElapsedTime, rt.hipEventDestroy):
            f.restype = ctypes.c_int
        self.rt = rt
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            for e in (a, b):
                st = rt.hipEventCreateWithFlags(ctypes.byref(e), self.NO_SYSTEM_FENCE)
                if st != 0:
                    raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")
            self.pairs.append((a.value, b.value))

    def elapsed_ms(self, i):
        ms = ctypes.c_float(0.0)
        st = self.rt.hipEventElapsedTime(ctypes.byref(ms), *self.pairs[i])
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def close(self):
        for a, b in self.pairs:
            self.rt.hipEventDestroy(a)
            self.rt.hipEventDestroy(b)
        self.pairs = []


def bench_one(name, args, torch, dev):
    import weight_quantized_gemm_amd as W
    case = workloads.make_workload(name)
    abytes = algorithmic_bytes(case)
    sets = max(1, min(8, -(-2 * CACHE_BYTES // max(abytes, 1))))
    packed = bool(getattr(args, "packed", False))
    calls, bufs = make_runner(case, torch, dev, sets, packed=packed)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    for i in range(args.warmup):
        calls[i % sets](sh)
    # The timed steps.  A hooked step arms the library's profiling hook, which hands a pair
    # of events to the launch of the step's main kernel (hipExtLaunchKernel): they take that
    # kernel's own start and end on its launch stream.  A hooked launch costs the stream a
    # few microseconds, and the idle gap lets the clock recover, so that the hooked kernel
    # itself runs faster than in a back-to-back stream (C2: 141-155 us against 160 us, by
    # rocprofv3 kernel traces).  By default every fifth timed step is hooked
    # (--kernel-events sampled), which keeps the stream close to back-to-back; `timed`
    # hooks every timed step, `after` as many steps after the timed ones.
    mode = args.kernel_events
    every = max(1, args.kernel_sample_every) if mode == "sampled" else 1
    hooked = hooked_steps(mode, args.steps, every)
    evs = KernelEvents(len(hooked) if mode != "after" else args.steps)
    slot = {i: n for n, i in enumerate(hooked)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i in slot:
            W.profile_next_call(*evs.pairs[slot[i]])
        calls[(args.warmup + i) % sets](sh)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if mode == "after":
        for i in range(args.steps):
            W.profile_next_call(*evs.pairs[i])
            calls[(args.warmup + args.steps + i) % sets](sh)
        torch.cuda.synchronize()
    launch_ms = [evs.elapsed_ms(i) for i in range(len(evs.pairs))]  # ms, main kernel per hooked step
    evs.close()
    ms_per_step = wall * 1e3 / args.steps
    flops = 2.0 * case.m * case.k * case.n
    kernel, bound = DOMINANT[name]
    dtype = "int8" if isinstance(case, workloads.W8A8Case) else case.act
    roof = make_roofline(bound, dtype, flops, abytes, launch_ms, ms_per_step)
    roof["traffic"] = traffic_for(kernel, name + (".packed" if packed else ""))
    roof["kernel"] = kernel
    roof["kernel_events"] = {"sampled": f"every {every}th timed step ({len(launch_ms)} launches)",
                             "timed": "every timed step",
                             "after": "steps after the timed ones"}[mode]
    value = flops / (ms_per_step / 1e3) / 1e12
    spec = workloads.WORKLOADS[name]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if dtype == "int8" else dtype,
        "data": "synthetic (seeded generators; inputs resident in HBM, rotated over "
                f"{sets} sets to defeat the Infinity Cache)",
        "config": {"workload": name, "m": case.m, "k": case.k, "n": case.n,
                   "weight_layout": "packed (wq_prepack_weight, outside the timed steps)" if packed else "ND",
                   "x1_shape": list(case.x1.shape), "seed": spec["seed"],
                   "algorithmic_bytes": abytes, "flops": flops,
                   "hbm_gbps": round(abytes / (ms_per_step / 1e3) / 1e9, 1),
                   "hbm_frac": round(abytes / (ms_per_step / 1e3) / 1e9 / PEAK_HBM, 4),
                   "inputs_sha256": workloads.digest(case)},
        "roofline": roof,
        "cpu_baseline": cpu_baseline(case, name) if args.cpu else None,
    }
    del calls, bufs
    torch.cuda.empty_cache()
    return line


def copy_calibration(args, torch, dev):
    """A plain copy of known size: it reads and writes copy_mib MiB per launch."""
    nbytes = args.copy_mib << 20
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "us_per_copy": round(dt * 1e6, 2),
            "gbps_read_plus_write": round(2 * nbytes / dt / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--all", action="store_true", help="one line per workload")
    ap.add_argument("--no-cpu", dest="cpu", action="store_false", help="skip the CPU oracle leg")
    ap.add_argument("--packed", action="store_true",
                    help="weights prepacked once before timing (wq_prepack_weight)")
    ap.add_argument("--kernel-events", choices=("sampled", "timed", "after"), default="sampled",
                    help="which steps carry the main kernel's event pairs: every Nth timed step "
                         "(default; N = --kernel-sample-every), every timed step, or as many steps "
                         "after the timed ones")
    ap.add_argument("--kernel-sample-every", type=int, default=5,
                    help="with --kernel-events sampled: hook every Nth timed step")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the matmul, time a plain device-to-device copy of this many MiB "
                         "(the reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU path is "
              "not part of this library", file=sys.stderr)
        sys.exit(2)
    import torch
    import weight_quantized_gemm_amd as W
    W.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.copy_mib > 0:
        print(json.dumps(copy_calibration(args, torch, dev)), flush=True)
        return
    names = sorted(workloads.WORKLOADS) if args.all else [args.workload]
    for name in names:
        print(json.dumps(bench_one(name, args, torch, dev)), flush=True)


if __name__ == "__main__":
    main()

"""Element-wise comparison of a GPU result with the oracle.

Test infrastructure only (see the package docstring).

An element passes when |gpu - ref| <= tol * max(1, |ref|), with tol = 2e-3 for fp16
outputs and 1e-2 for bf16 outputs.  Integer results are compared for equality.
"""
from __future__ import annotations

import numpy as np

TOLERANCE = {"fp16": 2e-3, "bf16": 1e-2}


def compare(gpu: np.ndarray, ref: np.ndarray, out_dtype: str) -> dict:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    tol = TOLERANCE[out_dtype]
    limit = tol * np.maximum(1.0, np.abs(ref))
    err = np.abs(gpu - ref)
    bad = ~(err <= limit)                     # NaN counts as a failure
    ratio = np.where(np.isfinite(err), err / limit, np.inf)
    worst = int(np.argmax(ratio)) if ratio.size else 0
    return {
        "n": int(ref.size),
        "n_fail": int(bad.sum()),
        "max_ratio": float(ratio.reshape(-1)[worst]) if ratio.size else 0.0,
        "worst_index": tuple(int(i) for i in np.unravel_index(worst, ref.shape)) if ratio.size else (),
        "ok": bool(not bad.any()),
    }

"""The no-allocation entry point, wq_antiquant_matmul_noalloc, against wq_antiquant_matmul.

Both are called through the C ABI on the same device buffers; the no-allocation call takes
its workspace from the library's scratch area instead of the caller's.  Three calls in a
row, each smaller than the one before and using the workspace differently (split-k partials
of the small-m path; split-k partials and row sums of the tiled path; transposed per-group
parameters and per-group row sums), must give the existing entry point's output bit for bit
and pass the oracle comparison.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
import weight_quantized_gemm_amd as W
from gpu_util import dev_tensor, ref_antiquant, to_f64

pytestmark = pytest.mark.gpu

CASES = [
    ("smallm_pergroup64_fp16_i8_32x8192x8192",
     dict(act="fp16", weight="int8", x1_shape=(32, 8192), n=8192, mode="group", group_size=64,
          offset_dist=("uniform", -4, 4), with_x3=False)),
    ("splitk_perchannel_bf16_i8_96x4096x1024",
     dict(act="bf16", weight="int8", x1_shape=(96, 4096), n=1024, mode="channel")),
    ("xt_pergroup128_fp16_i4_300x1024x256",
     dict(act="fp16", weight="int4", x1_shape=(300, 1024), n=256, mode="group", group_size=128,
          x2_transposed=True)),
]


def _tensors(case):
    act = case.act
    x1 = dev_tensor(case.x1, act)
    x2 = dev_tensor(case.x2, "raw")
    scale = dev_tensor(case.scale, act)
    offset = dev_tensor(case.offset, act)
    if case.x2_transposed:
        x2 = x2.t()
        if case.group_size:
            scale = scale.t()
            offset = None if offset is None else offset.t()
    return x1, x2, scale, offset, dev_tensor(case.bias, act), dev_tensor(case.x3, act)


def test_noalloc_matches_workspace_entry_point():
    L = W.lib()
    stream = torch.cuda.current_stream().cuda_stream
    for i, (name, spec) in enumerate(CASES):
        print(f"[gpu-case] noalloc:{name}", flush=True)
        case = workloads.make_antiquant(seed=3100 + i, name=name, **spec)
        x1, x2, scale, offset, bias, x3 = _tensors(case)
        int4 = case.weight == "int4"
        ref_call = W.AntiquantMatmul(x1, x2, scale, offset, bias, x3, case.group_size, x2_int4=int4)
        assert 0 < ref_call.workspace_size <= W.WQ_NOALLOC_SCRATCH_BYTES, (name, ref_call.workspace_size)
        ref = ref_call()
        out = torch.empty_like(ref)
        descs = [W._desc(x1), W._desc(x2, int4), W._desc(bias), W._desc(scale), W._desc(offset), W._desc(x3)]
        od = W._desc(out)
        r = lambda d: ctypes.byref(d) if d is not None else None
        st = L.wq_antiquant_matmul_noalloc(*map(r, descs), int(case.group_size), r(od), ctypes.c_void_p(stream))
        assert st == W.WQ_OK, (name, st)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), name
        res = oracle.compare(to_f64(out).reshape(case.out_shape), ref_antiquant(case), case.act)
        assert res["ok"], (name, res)

"""Helpers for the GPU tests: move a stored case to the device, run it through the binding,
read results back as fp64, and evaluate the oracle on all or on sampled rows."""
import numpy as np

import oracle
import workloads


def torch_mod():
    import torch
    return torch


def dev_tensor(a, dtype_name, device="cuda:0"):
    torch = torch_mod()
    if a is None:
        return None
    if dtype_name == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_antiquant(case, device="cuda:0", out=None, stream=None, keep=None):
    """The one-shot call on `case`.  With `stream`, the call runs there after waiting for the
    current stream (which made the inputs); `keep` (a list) then receives the input tensors,
    which the caller holds until it has synchronised `stream`."""
    import weight_quantized_gemm_amd as W
    act = case.act
    x1 = dev_tensor(case.x1, act, device)
    x2 = dev_tensor(case.x2, "raw", device)
    if case.weight == "fp8e4m3":
        x2 = x2.view(torch_mod().float8_e4m3fn)
    scale = dev_tensor(case.scale, act, device)
    offset = dev_tensor(case.offset, act, device)
    if case.x2_transposed:
        # transposed storage is handed over as the (k, n) transpose view, as a caller would
        x2 = x2.t()
        if case.group_size:
            scale = scale.t()
            offset = None if offset is None else offset.t()
    args = dict(antiquant_offset=offset,
                bias=dev_tensor(case.bias, act, device), x3=dev_tensor(case.x3, act, device),
                antiquant_group_size=case.group_size, x2_int4=case.weight == "int4", out=out)
    if stream is not None:
        stream.wait_stream(torch_mod().cuda.current_stream(device))
        if keep is not None:
            keep.extend([x1, x2, scale, args["antiquant_offset"], args["bias"], args["x3"]])
    return W.antiquant_matmul(x1, x2, scale, **args, stream=stream)


def ref_antiquant(case, rows=None):
    if rows is None:
        c = case
    else:
        c = sample_rows(case, rows)
    return oracle.ref_antiquant(c.x1, c.x2, c.scale, c.offset, c.bias, c.x3, c.group_size,
                                act=c.act, weight=c.weight, x2_transposed=c.x2_transposed)


def sample_rows(case, rows):
    import dataclasses
    k = case.x1.shape[-1]
    x1 = case.x1.reshape(-1, k)[rows]
    if isinstance(case, workloads.AntiquantCase):
        x3 = None if case.x3 is None else case.x3.reshape(-1, case.n)[rows]
        return dataclasses.replace(case, x1=x1, x3=x3)
    x3 = None if case.x3 is None else case.x3.reshape(-1, case.n)[rows]
    pt = None if case.pertoken_scale is None else case.pertoken_scale[rows]
    return dataclasses.replace(case, x1=x1, x3=x3, pertoken_scale=pt)


def run_w8a8(case, device="cuda:0", with_acc=True, stream=None, keep=None, packed=False):
    """The one-shot W8A8 call; `stream` and `keep` as for run_antiquant; with `packed` the
    weight goes through wq_prepack_weight first."""
    import weight_quantized_gemm_amd as W
    torch = torch_mod()
    x1 = dev_tensor(case.x1, "raw", device)
    x2 = dev_tensor(case.x2, "raw", device)
    if case.x2_transposed:
        x2 = x2.t()
    if packed:
        x2 = W.prepack_weight(x2)
    dq = dev_tensor(case.dequant_scale, case.dequant_dtype, device)
    pt = dev_tensor(case.pertoken_scale, "fp32", device)
    bias = dev_tensor(case.bias, "raw", device)
    x3 = dev_tensor(case.x3, case.out, device)
    acc = torch.empty((case.m, case.n), dtype=torch.int32, device=device) if with_acc else None
    out_dtype = torch.bfloat16 if case.out == "bf16" else torch.float16
    if stream is not None:
        stream.wait_stream(torch.cuda.current_stream(device))
        if keep is not None:
            keep.extend([x1, x2, dq, pt, bias, x3, acc])
    y = W.quant_matmul(x1, x2, dq, pt, bias, x3, out_dtype=out_dtype, acc_out=acc, stream=stream)
    return y, acc


def ref_w8a8(case, rows=None):
    c = case if rows is None else sample_rows(case, rows)
    return oracle.ref_w8a8(c.x1, c.x2, c.dequant_scale, c.pertoken_scale, c.bias, c.x3,
                           dequant_dtype=c.dequant_dtype, out=c.out, x2_transposed=c.x2_transposed)


def sampled_rows(m, count=48, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, m // 2, m - 2, m - 1]
    extra = rng.choice(m, size=min(m, count), replace=False).tolist()
    return np.array(sorted(set(r for r in fixed + extra if 0 <= r < m)))

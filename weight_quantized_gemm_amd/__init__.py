"""weight_quantized_gemm_amd -- weight-anti-quant matmul and its W8A8 sibling on MI355X.

Thin Python binding over the C ABI of ``libwqgemm.so`` (declared in ``include/wqgemm.h``).
It only marshals arguments: tensors become ``wq_tensor`` descriptors (device pointer,
dtype, shape, strides), the output and workspace are allocated with torch on the
inputs' device, and the call is enqueued on torch's current HIP stream.  Every step of
the computation runs in the library's HIP kernels; there is no fallback path.

``AntiquantMatmul`` / ``QuantMatmul`` are prepared calls, the counterpart of the
executor of the pages' two-phase interface: descriptors, workspace size and workspace
are settled once, and each call only enqueues the kernels (for tight loops).

    antiquant_matmul:  out = x1 @ ((x2 + offset) * scale) + bias + x3
    quant_matmul:      out = dequant_scale * pertoken_scale * (x1 @ x2 + bias) + x3

(the formulas of the aclnnWeightQuantMatmulAllReduce guide, section 计算公式, and of the
aclnnQuantMatmulAllReduceV2 page, section Function, at one rank).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = ["WQ_F16", "WQ_BF16", "WQ_F32", "WQ_I8", "WQ_I4", "WQ_I32", "WQ_F8E4M3", "WQ_OK",
           "WQ_ERR_PARAM_NULLPTR", "WQ_ERR_PARAM_INVALID", "WQ_ERR_RUNTIME", "WQ_ERR_SCRATCH_LIMIT",
           "WQ_NOALLOC_SCRATCH_BYTES", "WQ_PACKED", "WqTensor", "PackedWeight", "prepack_weight",
           "packed_weight_bytes",
           "WqError", "lib", "library_path", "make_desc", "antiquant_matmul",
           "antiquant_workspace_size", "quant_matmul", "quant_workspace_size", "AntiquantMatmul",
           "QuantMatmul", "profile_next_call", "EXPORTS"]

WQ_F16, WQ_BF16, WQ_F32, WQ_I8, WQ_I4, WQ_I32, WQ_F8E4M3 = 1, 2, 3, 4, 5, 6, 7
WQ_OK, WQ_ERR_PARAM_NULLPTR, WQ_ERR_PARAM_INVALID, WQ_ERR_RUNTIME = 0, 161001, 161002, 561001
WQ_ERR_SCRATCH_LIMIT = 561002
WQ_PACKED = 0x100
WQ_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("wq_antiquant_matmul_get_workspace_size", "wq_antiquant_matmul", "wq_antiquant_matmul_noalloc",
           "wq_prepack_weight_get_size", "wq_prepack_weight",
           "wq_quant_matmul_get_workspace_size", "wq_quant_matmul", "wq_profile_next_call",
           "wq_status_string", "wq_version")

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libwqgemm.so")


class WqTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 3), ("stride", ctypes.c_int64 * 3)]


class WqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def declare(L):
    """Set the argument and result types of the C-ABI functions a loaded library exports
    (all of them for the full library; a host-only build of the validation and planning
    code exports the size queries, the status strings and the version)."""
    P = ctypes.POINTER(WqTensor)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    sigs = {
        "wq_antiquant_matmul_get_workspace_size": ([P, P, P, P, P, P, ctypes.c_int64, P, u64p], ctypes.c_int),
        "wq_antiquant_matmul": ([P, P, P, P, P, P, ctypes.c_int64, P, ctypes.c_void_p, ctypes.c_uint64,
                                 ctypes.c_void_p], ctypes.c_int),
        "wq_antiquant_matmul_noalloc": ([P, P, P, P, P, P, ctypes.c_int64, P, ctypes.c_void_p], ctypes.c_int),
        "wq_quant_matmul_get_workspace_size": ([P, P, P, P, P, P, P, P, u64p], ctypes.c_int),
        "wq_quant_matmul": ([P, P, P, P, P, P, P, P, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p],
                            ctypes.c_int),
        "wq_prepack_weight_get_size": ([P, u64p], ctypes.c_int),
        "wq_prepack_weight": ([P, P, ctypes.c_void_p], ctypes.c_int),
        "wq_profile_next_call": ([ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
        "wq_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "wq_version": ([], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        if hasattr(L, name):
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
    return L


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is missing: build it with "
                              "`python -m weight_quantized_gemm_amd.build`")
        _lib = declare(ctypes.CDLL(library_path))
    return _lib


def _check(status: int):
    if status == WQ_OK:
        return
    msg = lib().wq_status_string(status).decode()
    if status in (WQ_ERR_PARAM_NULLPTR, WQ_ERR_PARAM_INVALID):
        raise ValueError(f"{msg} (status {status})")
    raise WqError(status, msg)


def make_desc(shape: Sequence[int], dtype: int, data: int, strides: Optional[Sequence[int]] = None):
    """A descriptor from plain values (strides default to row-major contiguous)."""
    d = WqTensor()
    d.data = data or None
    d.dtype = dtype
    d.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= int(s)
    for i in range(3):
        d.shape[i] = int(shape[i]) if i < len(shape) else 0
        d.stride[i] = int(strides[i]) if i < len(shape) else 0
    return d


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float16: WQ_F16, torch.bfloat16: WQ_BF16, torch.float32: WQ_F32,
         torch.int8: WQ_I8, torch.int32: WQ_I32, torch.float8_e4m3fn: WQ_F8E4M3}
    if t.dtype not in m:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


class PackedWeight:
    """A weight in the packed layout written by :func:`prepack_weight` (64 k x 32 column
    blocks in MFMA B-fragment order, see include/wqgemm.h).  ``data`` is the uint8 device
    tensor; ``k``, ``n`` the logical shape; ``dtype`` the WQ_* code of the codes (WQ_I8, WQ_I4
    or WQ_F8E4M3).  Pass it as x2 to the anti-quant calls."""

    def __init__(self, data, k: int, n: int, dtype: int):
        self.data, self.k, self.n, self.dtype = data, int(k), int(n), int(dtype)

    @property
    def shape(self):
        return (self.k, self.n)

    def desc(self):
        return make_desc([self.k, self.n], self.dtype | WQ_PACKED, self.data.data_ptr(), [0, 0])


def packed_weight_bytes(x2, *, x2_int4: bool = False) -> int:
    """Bytes of the packed layout of x2 (wq_prepack_weight_get_size)."""
    size = ctypes.c_uint64(0)
    _check(lib().wq_prepack_weight_get_size(ctypes.byref(_desc(x2, x2_int4)), ctypes.byref(size)))
    return size.value


def prepack_weight(x2, *, x2_int4: bool = False, out=None, stream=None) -> PackedWeight:
    """Relayout a weight (int8 (k, n), packed int4 (k, n/2) bytes, or float8_e4m3fn (k, n);
    row-major or the transpose view of a row-major (n, k) tensor) into the packed layout, on
    `stream` (default torch's current stream).  Returns a :class:`PackedWeight`; `out`, if
    given, is a uint8 device tensor of at least packed_weight_bytes(x2) bytes."""
    torch = _torch()
    d = _desc(x2, x2_int4)
    size = packed_weight_bytes(x2, x2_int4=x2_int4)
    with _alloc_on(stream, x2.device) as s:
        if out is None:
            out = torch.empty(max(size, 1), dtype=torch.uint8, device=x2.device)
        elif out.numel() < size or out.dtype != torch.uint8:
            raise ValueError(f"the packed weight needs a uint8 tensor of at least {size} bytes")
        pw = PackedWeight(out, d.shape[0], d.shape[1], d.dtype)
        _check(lib().wq_prepack_weight(ctypes.byref(d), ctypes.byref(pw.desc()), _stream_handle(s, x2.device)))
    return pw


def _desc(t, int4: bool = False):
    if t is None:
        return None
    if isinstance(t, PackedWeight):
        return t.desc()
    if int4:
        torch = _torch()
        if t.dtype not in (torch.uint8, torch.int8) or t.dim() != 2:
            raise ValueError("packed int4 weights are a 2-D uint8/int8 tensor: (k, n/2) bytes, or "
                             "the (k/2, n) transpose view of an (n, k/2) tensor")
        a, b = t.shape
        if t.stride(0) == 1 and t.stride(1) == a and a > 1 and b > 1:
            # transpose view of row-major (n, k/2) storage: logical (k, n), nibbles along k
            return make_desc([2 * a, b], WQ_I4, t.data_ptr(), [1, 2 * a])
        # row-major (k, n/2) storage (strides in logical elements; the library checks them)
        return make_desc([a, 2 * b], WQ_I4, t.data_ptr(), [t.stride(0) * 2, t.stride(1)])
    return make_desc(list(t.shape), _dtype_code(t), t.data_ptr(), list(t.stride()))


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _stream_handle(stream, device) -> ctypes.c_void_p:
    """A raw stream handle: `stream` may be None (torch's current stream on `device`), a
    torch stream, or an integer handle."""
    if stream is None:
        stream = _torch().cuda.current_stream(device)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


class _alloc_on:
    """Context for a one-shot call: torch's current stream is the call's stream while the
    call allocates and enqueues, so that its output and workspace belong to that stream (a
    raw integer handle is wrapped as an external stream).  Yields the torch stream."""

    def __init__(self, stream, device):
        torch = _torch()
        if stream is None:
            stream = torch.cuda.current_stream(device)
        elif isinstance(stream, int):
            stream = torch.cuda.ExternalStream(stream, device=device)
        self.stream = stream
        self._ctx = torch.cuda.stream(stream)

    def __enter__(self):
        self._ctx.__enter__()
        return self.stream

    def __exit__(self, *exc):
        return self._ctx.__exit__(*exc)


def profile_next_call(before, after):
    """Arm the library's profiling hook: the next call on this thread records the events
    `before` / `after` around the launch of its main kernel.  Each is a raw hipEvent_t handle
    (an int) or a torch event (created with enable_timing=True and recorded once before, so
    that its HIP event exists)."""
    def handle(e):
        if e is None:
            return 0
        return e if isinstance(e, int) else e.cuda_event
    b, a = handle(before), handle(after)
    if (before is not None and not b) or (after is not None and not a):
        raise ValueError("record the events once before arming the hook")
    _check(lib().wq_profile_next_call(ctypes.c_void_p(b or None), ctypes.c_void_p(a or None)))


def antiquant_workspace_size(x1, x2, antiquant_scale, antiquant_offset=None, bias=None, x3=None,
                             antiquant_group_size: int = 0, *, x2_int4: bool = False, out=None) -> int:
    d = [_desc(x1), _desc(x2, x2_int4), _desc(bias), _desc(antiquant_scale),
         _desc(antiquant_offset), _desc(x3)]
    od = _desc(out) if out is not None else _out_desc_like(x1, x2, x2_int4)
    ws = ctypes.c_uint64(0)
    _check(lib().wq_antiquant_matmul_get_workspace_size(*map(_ref, d), int(antiquant_group_size),
                                                        _ref(od), ctypes.byref(ws)))
    return ws.value


def _is_t_view(t) -> bool:
    """The transpose view of a row-major 2-D tensor (strides (1, rows))."""
    return t.dim() == 2 and t.shape[0] > 1 and t.shape[1] > 1 and t.stride(0) == 1 and t.stride(1) == t.shape[0]


def _weight_n(x2, x2_int4: bool) -> int:
    """Output columns n of a weight tensor (row-major int4 storage packs two columns a byte)."""
    if isinstance(x2, PackedWeight):
        return x2.n
    return x2.shape[1] * (2 if x2_int4 and not _is_t_view(x2) else 1)


def _out_desc_like(x1, x2, x2_int4):
    n = _weight_n(x2, x2_int4)
    return make_desc(list(x1.shape[:-1]) + [n], _dtype_code(x1), 0x1)


class AntiquantMatmul:
    """Prepared anti-quant call: out = x1 @ ((x2 + offset) * scale) + bias + x3.

    Arguments as for :func:`antiquant_matmul`.  The descriptors are validated and the
    workspace is sized (and allocated unless given) once; ``call(stream=None)`` enqueues
    the kernels on `stream` (default: torch's current stream) and returns ``out``.  The
    prepared call holds references to its tensors; their storage must not change."""

    def __init__(self, x1, x2, antiquant_scale, antiquant_offset=None, bias=None, x3=None,
                 antiquant_group_size: int = 0, *, x2_int4: bool = False, out=None, workspace=None):
        torch = _torch()
        n = _weight_n(x2, x2_int4)
        if out is None:
            out = torch.empty(tuple(x1.shape[:-1]) + (n,), dtype=x1.dtype, device=x1.device)
        self._descs = [_desc(x1), _desc(x2, x2_int4), _desc(bias), _desc(antiquant_scale),
                       _desc(antiquant_offset), _desc(x3)]
        od = _desc(out)
        L = lib()
        ws = ctypes.c_uint64(0)
        g = int(antiquant_group_size)
        _check(L.wq_antiquant_matmul_get_workspace_size(*map(_ref, self._descs), g, _ref(od),
                                                        ctypes.byref(ws)))
        if workspace is None or workspace.numel() < ws.value:
            workspace = torch.empty(max(int(ws.value), 1), dtype=torch.uint8, device=x1.device)
        self.workspace_size = int(ws.value)
        self.out, self.workspace, self.device = out, workspace, x1.device
        self._keep = (x1, x2, antiquant_scale, antiquant_offset, bias, x3, od)
        self._fn = L.wq_antiquant_matmul
        self._args = (*map(_ref, self._descs), g, _ref(od), ctypes.c_void_p(workspace.data_ptr()),
                      ctypes.c_uint64(workspace.numel()))

    def __call__(self, stream=None):
        _check(self._fn(*self._args, _stream_handle(stream, self.device)))
        return self.out


def antiquant_matmul(x1, x2, antiquant_scale, antiquant_offset=None, bias=None, x3=None,
                     antiquant_group_size: int = 0, *, x2_int4: bool = False, out=None,
                     workspace=None, stream=None):
    """out = x1 @ ((x2 + antiquant_offset) * antiquant_scale) + bias + x3 on x1's device.

    x1: fp16/bf16 (m, k) or (b, s, k); x2: int8 (k, n), or with ``x2_int4`` a uint8 (k, n/2)
    tensor of packed signed nibbles (even column in the low nibble), or float8_e4m3fn (k, n)
    with a per-channel scale and no offset; scale/offset: (1), (n), (1, n) or (ceil(k/g), n)
    for group size g.  x2 may also be the transpose view ``w.t()`` of a row-major (n, k)
    tensor (int4: of an (n, k/2) tensor packed along k); per-group scale and offset are then
    transpose views too.  x2 may also be a :class:`PackedWeight` (prepack_weight), with
    row-major per-group parameters.  The output and the workspace (unless given) are allocated on the
    stream the call runs on (`stream`, default torch's current stream), so that torch's
    allocator does not hand their memory to other work while the call's kernels may still
    use it.  Returns the output tensor."""
    with _alloc_on(stream, x1.device) as s:
        return AntiquantMatmul(x1, x2, antiquant_scale, antiquant_offset, bias, x3, antiquant_group_size,
                               x2_int4=x2_int4, out=out, workspace=workspace)(s)


def quant_workspace_size(x1, x2, dequant_scale, pertoken_scale=None, bias=None, x3=None, *,
                         out=None, acc_out=None) -> int:
    d = [_desc(x1), _desc(x2), _desc(bias), _desc(x3), _desc(dequant_scale), _desc(pertoken_scale),
         _desc(out), _desc(acc_out)]
    ws = ctypes.c_uint64(0)
    _check(lib().wq_quant_matmul_get_workspace_size(*map(_ref, d), ctypes.byref(ws)))
    return ws.value


class QuantMatmul:
    """Prepared W8A8 call: out = dequant_scale * pertoken_scale * (x1 @ x2 + bias) + x3.

    Arguments as for :func:`quant_matmul`; ``call(stream=None)`` enqueues the kernel and
    returns ``out``."""

    def __init__(self, x1, x2, dequant_scale, pertoken_scale=None, bias=None, x3=None, *,
                 out_dtype=None, out=None, acc_out=None):
        torch = _torch()
        if out is None:
            dt = out_dtype if out_dtype is not None else (x3.dtype if x3 is not None else torch.bfloat16)
            out = torch.empty(tuple(x1.shape[:-1]) + (x2.shape[1],), dtype=dt, device=x1.device)
        self._descs = [_desc(x1), _desc(x2), _desc(bias), _desc(x3), _desc(dequant_scale),
                       _desc(pertoken_scale), _desc(out), _desc(acc_out)]
        L = lib()
        ws = ctypes.c_uint64(0)
        _check(L.wq_quant_matmul_get_workspace_size(*map(_ref, self._descs), ctypes.byref(ws)))
        workspace = torch.empty(max(int(ws.value), 1), dtype=torch.uint8, device=x1.device)
        self.workspace_size = int(ws.value)
        self.out, self.acc_out, self.workspace, self.device = out, acc_out, workspace, x1.device
        self._keep = (x1, x2, dequant_scale, pertoken_scale, bias, x3)
        self._fn = L.wq_quant_matmul
        self._args = (*map(_ref, self._descs), ctypes.c_void_p(workspace.data_ptr()),
                      ctypes.c_uint64(workspace.numel()))

    def __call__(self, stream=None):
        _check(self._fn(*self._args, _stream_handle(stream, self.device)))
        return self.out


def quant_matmul(x1, x2, dequant_scale, pertoken_scale=None, bias=None, x3=None, *,
                 out_dtype=None, out=None, acc_out=None, stream=None):
    """out = dequant_scale * pertoken_scale * (x1 @ x2 + bias) + x3 on x1's device.

    x1, x2 int8; bias int32 (n); dequant_scale (1), (n) or (1, n), fp32 (fp16 output) or
    bf16/fp32 (bf16 output); pertoken_scale fp32 (m); x3 and the output fp16/bf16.
    ``acc_out`` (int32, (m, n)) receives x1 @ x2 + bias.  The output and the workspace are
    allocated on the stream the call runs on (`stream`, default torch's current stream)."""
    with _alloc_on(stream, x1.device) as s:
        return QuantMatmul(x1, x2, dequant_scale, pertoken_scale, bias, x3, out_dtype=out_dtype, out=out,
                           acc_out=acc_out)(s)

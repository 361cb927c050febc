"""Python binding of librib.so: RIB window attention on MI355X (gfx950).

Thin ctypes marshalling over the C ABI in include/rib.h. torch supplies device
memory and the current stream; every step of the computation runs in the HIP
kernels of librib.so. There is no fallback: if the library is missing or no
GPU is present, the compute entry points raise.

Entry points (same names as the C ABI, without the ``rib_`` prefix):
  posgen, posgen_bwd, window_partition, window_unpartition, window_attn_fwd,
  window_attn_bwd, fwd_workspace_size, bwd_workspace_size,
  rpb_window_attn_fwd, rpb_fwd_workspace_size (the relative-position-bias
  comparison kernel), cla_gate, window_attn_fwd_gated (the CLA gating map and
  the forward with O' = O * G fused into its output stage)
plus ``FwdPlan`` / ``BwdPlan`` / ``RpbFwdPlan``, which preallocate workspace
and outputs so a call can be repeated without allocating.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "RIB_OK", "RIB_ERR_INVALID_ARG", "RIB_ERR_UNSUPPORTED", "RIB_ERR_WORKSPACE", "RIB_ERR_HIP",
    "RIB_F32", "RIB_BF16", "RibError", "lib", "lib_path", "exported_symbols",
    "posgen", "posgen_bwd", "window_partition", "window_unpartition", "window_attn_fwd", "window_attn_bwd",
    "fwd_workspace_size", "bwd_workspace_size", "FwdPlan", "BwdPlan", "Shape",
    "rpb_window_attn_fwd", "rpb_fwd_workspace_size", "RpbFwdPlan",
    "cla_gate", "window_attn_fwd_gated", "window_attn_fwd_noalloc", "NOALLOC_WORKSPACE_BYTES",
    "KERNEL_GROUPS", "kernel_timing_enable", "kernel_timing_select", "kernel_timing_read",
]

RIB_OK, RIB_ERR_INVALID_ARG, RIB_ERR_UNSUPPORTED, RIB_ERR_WORKSPACE, RIB_ERR_HIP = range(5)
RIB_F32, RIB_BF16 = 0, 1

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG_DIR, "librib.so")


class RibError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("d_c", ctypes.c_int32), ("w", ctypes.c_int32),
                ("r", ctypes.c_int32)]


class _Mlp(ctypes.Structure):
    _fields_ = [("n_freq", ctypes.c_int32), ("hidden", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p)]


_LIB = None
_vp, _sz, _i32, _f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
_SIGS = {
    "rib_posgen": (_i32, [_i32, ctypes.POINTER(_Mlp), _i32, _vp, _vp, _vp]),
    "rib_posgen_bwd_workspace_size": (_sz, [_i32, ctypes.POINTER(_Mlp)]),
    "rib_posgen_bwd": (_i32, [_i32, ctypes.POINTER(_Mlp)] + [_vp] * 6 + [_vp, _sz, _vp]),
    "rib_window_partition": (_i32, [ctypes.POINTER(Shape), _i32, _vp, _vp, _vp]),
    "rib_window_unpartition": (_i32, [ctypes.POINTER(Shape), _i32, _vp, _vp, _vp]),
    "rib_fwd_workspace_size": (_sz, [ctypes.POINTER(Shape), _i32]),
    "rib_bwd_workspace_size": (_sz, [ctypes.POINTER(Shape), _i32]),
    "rib_window_attn_fwd": (_i32, [ctypes.POINTER(Shape), _i32, _f32] + [_vp] * 7 + [_vp, _sz, _vp]),
    "rib_window_attn_bwd": (_i32, [ctypes.POINTER(Shape), _i32, _f32] + [_vp] * 13 + [_vp, _sz, _vp]),
    "rib_rpb_fwd_workspace_size": (_sz, [ctypes.POINTER(Shape), _i32]),
    "rib_cla_gate": (_i32, [ctypes.POINTER(Shape), _i32] + [_vp] * 6 + [_vp]),
    "rib_window_attn_fwd_gated": (_i32, [ctypes.POINTER(Shape), _i32, _f32] + [_vp] * 8 + [_vp, _sz, _vp]),
    "rib_window_attn_fwd_noalloc": (_i32, [ctypes.POINTER(Shape), _i32, _f32] + [_vp] * 7 + [_vp]),
    "rib_rpb_window_attn_fwd": (_i32, [ctypes.POINTER(Shape), _i32, _f32] + [_vp] * 6 + [_vp, _sz, _vp]),
    "rib_kernel_timing_enable": (_i32, [_i32]),
    "rib_kernel_timing_select": (_i32, [ctypes.c_uint32]),
    "rib_kernel_timing_read": (_i32, [_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    "rib_status_string": (ctypes.c_char_p, [_i32]),
    "rib_last_error": (ctypes.c_char_p, []),
}
exported_symbols = tuple(_SIGS)


def lib():
    """Loads librib.so once (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is missing: build it with "
                               "`python -m windowed_attention_implicit_amd.build`")
        L = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _status_name(status: int) -> str:
    try:
        return lib().rib_status_string(status).decode()
    except Exception:  # noqa: BLE001 - naming an error must never raise
        return f"status {status}"


def _check(status: int):
    if status != RIB_OK:
        raise RibError(status, lib().rib_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return RIB_BF16
    if t == torch.float32:
        return RIB_F32
    raise TypeError(f"unsupported dtype {t}: use torch.bfloat16 or torch.float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_gpu(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous GPU tensors")


def _shape_of(x: torch.Tensor, w: int, r: int) -> Shape:
    if x.dim() != 5:
        raise ValueError("feature maps are [B, H, W, heads, d_c]")
    B, H, W, heads, d_c = x.shape
    return Shape(B, H, W, heads, d_c, w, r)


def fwd_workspace_size(shape: Shape, dtype: torch.dtype) -> int:
    return int(lib().rib_fwd_workspace_size(ctypes.byref(shape), _dtype_code(dtype)))


def bwd_workspace_size(shape: Shape, dtype: torch.dtype) -> int:
    return int(lib().rib_bwd_workspace_size(ctypes.byref(shape), _dtype_code(dtype)))


def _run_stream(stream, device, tensors):
    """The stream handle of a plan's run(): the current stream, or the raw hipStream_t `stream`. For
    a raw stream the plan's tensors are recorded on it, so the caching allocator does not hand
    their memory to other work before the kernels queued there have finished with it (the plan
    may be dropped first)."""
    if stream is None:
        return _stream(device)
    ext = torch.cuda.ExternalStream(stream, device=device)
    for t in tensors:
        if t is not None:
            t.record_stream(ext)
    return ctypes.c_void_p(stream)


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte (or better) aligned blocks
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- posgen

def posgen(w: int, w1: torch.Tensor, b1, w2: torch.Tensor, b2, rank: int, n_freq: int = 16,
           out_dtype: torch.dtype = torch.bfloat16):
    """Positional tokens (Q_p, K_p) of window size w, each [w*w, rank] in out_dtype."""
    _require_gpu(w1, b1, w2, b2)
    for t in (w1, b1, w2, b2):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("MLP weights are float32")
    hidden = w1.shape[0]
    mlp = _Mlp(n_freq, hidden, rank, w1.data_ptr(), b1.data_ptr() if b1 is not None else None,
               w2.data_ptr(), b2.data_ptr() if b2 is not None else None)
    qp = torch.empty((w * w, rank), dtype=out_dtype, device=w1.device)
    kp = torch.empty_like(qp)
    _check(lib().rib_posgen(w, ctypes.byref(mlp), _dtype_code(out_dtype), _ptr(qp), _ptr(kp), _stream(w1.device)))
    return qp, kp


def posgen_bwd(w: int, w1: torch.Tensor, b1, w2: torch.Tensor, b2, rank: int, dq_p: torch.Tensor,
               dk_p: torch.Tensor, n_freq: int = 16):
    """Position-MLP weight gradients (dW1, db1, dW2, db2), float32, from dQ_p, dK_p (float32 [w*w, rank])."""
    _require_gpu(w1, b1, w2, b2, dq_p, dk_p)
    for t in (w1, b1, w2, b2, dq_p, dk_p):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise TypeError("weights and positional gradients are contiguous float32")
    if dq_p.shape != (w * w, rank) or dk_p.shape != (w * w, rank):
        raise ValueError("dq_p and dk_p must be [w*w, rank]")
    hidden = w1.shape[0]
    mlp = _Mlp(n_freq, hidden, rank, w1.data_ptr(), b1.data_ptr() if b1 is not None else None,
               w2.data_ptr(), b2.data_ptr() if b2 is not None else None)
    nbytes = lib().rib_posgen_bwd_workspace_size(w, ctypes.byref(mlp))
    if nbytes == 0:
        _check(lib().rib_posgen_bwd(w, ctypes.byref(mlp), None, None, None, None, None, None, None, 0, None))
    ws = _workspace(nbytes, w1.device)
    dw1 = torch.empty((hidden, 4 * n_freq), dtype=torch.float32, device=w1.device)
    db1 = torch.empty((hidden,), dtype=torch.float32, device=w1.device)
    dw2 = torch.empty((2 * rank, hidden), dtype=torch.float32, device=w1.device)
    db2 = torch.empty((2 * rank,), dtype=torch.float32, device=w1.device)
    _check(lib().rib_posgen_bwd(w, ctypes.byref(mlp), _ptr(dq_p), _ptr(dk_p), _ptr(dw1), _ptr(db1), _ptr(dw2),
                                _ptr(db2), _ptr(ws), nbytes, _stream(w1.device)))
    return dw1, db1, dw2, db2


# ---------------------------------------------------------------- partition

def window_partition(x: torch.Tensor, w: int) -> torch.Tensor:
    """[B, H, W, heads, d] -> [B*(H/w)*(W/w), heads, w*w, d]."""
    _require_gpu(x)
    s = _shape_of(x, w, 1)
    out = torch.empty((s.B * (s.H // w) * (s.W // w), s.heads, w * w, s.d_c), dtype=x.dtype, device=x.device)
    _check(lib().rib_window_partition(ctypes.byref(s), _dtype_code(x.dtype), _ptr(x), _ptr(out), _stream(x.device)))
    return out


def window_unpartition(xw: torch.Tensor, B: int, H: int, W: int, w: int) -> torch.Tensor:
    """Inverse of ``window_partition``."""
    _require_gpu(xw)
    heads, d = xw.shape[1], xw.shape[3]
    s = Shape(B, H, W, heads, d, w, 1)
    out = torch.empty((B, H, W, heads, d), dtype=xw.dtype, device=xw.device)
    _check(lib().rib_window_unpartition(ctypes.byref(s), _dtype_code(xw.dtype), _ptr(xw), _ptr(out),
                                        _stream(xw.device)))
    return out


# ---------------------------------------------------------------- attention

class FwdPlan:
    """Preallocated forward call: workspace, O and LSE for one shape."""

    def __init__(self, q_c, k_c, v, q_p, k_p, w: int, scale: float | None = None, want_lse: bool = True):
        _require_gpu(q_c, k_c, v, q_p, k_p)
        self.shape = _shape_of(q_c, w, q_p.shape[1])
        self.dtype = _dtype_code(q_c.dtype)
        for t in (k_c, v, q_p, k_p):
            if t.dtype != q_c.dtype:
                raise TypeError("all activations and Q_p, K_p must share one dtype")
        self.inputs = (q_c, k_c, v, q_p, k_p)
        self.scale = 0.0 if scale is None else float(scale)
        self.o = torch.empty_like(q_c)
        s = self.shape
        self.lse = torch.empty((s.B, s.H, s.W, s.heads), dtype=torch.float32, device=q_c.device) if want_lse else None
        self.ws_bytes = fwd_workspace_size(self.shape, q_c.dtype)
        self.ws = _workspace(self.ws_bytes, q_c.device)

    def run(self, stream=None):
        """Enqueues the call on the current stream, or on `stream` (a raw hipStream_t handle)."""
        q_c, k_c, v, q_p, k_p = self.inputs
        st = _run_stream(stream, q_c.device, (*self.inputs, self.o, self.lse, self.ws))
        _check(lib().rib_window_attn_fwd(ctypes.byref(self.shape), self.dtype, self.scale, _ptr(q_c), _ptr(k_c),
                                         _ptr(v), _ptr(q_p), _ptr(k_p), _ptr(self.o), _ptr(self.lse),
                                         _ptr(self.ws), self.ws_bytes, st))
        return self.o, self.lse


def window_attn_fwd(q_c, k_c, v, q_p, k_p, w: int, scale: float | None = None, want_lse: bool = True):
    """O = softmax(scale [Q_c|Q_p][K_c|K_p]^T) V per window and head; returns (O, LSE or None)."""
    return FwdPlan(q_c, k_c, v, q_p, k_p, w, scale, want_lse).run()


def window_attn_fwd_gated(q_c, k_c, v, q_p, k_p, gate, w: int, scale: float | None = None,
                          want_lse: bool = True):
    """O' = O * G with O the RIB attention output; ``gate`` [B, H, W, heads, d_c] (or [B, H, W, C]) in the
    activations' dtype, e.g. from ``cla_gate``. Returns (O', LSE of the ungated attention or None)."""
    plan = FwdPlan(q_c, k_c, v, q_p, k_p, w, scale, want_lse)
    _require_gpu(gate)
    if gate.dtype != q_c.dtype or gate.numel() != q_c.numel():
        raise ValueError("gate must match the feature map's dtype and size")
    _check(lib().rib_window_attn_fwd_gated(ctypes.byref(plan.shape), plan.dtype, plan.scale, _ptr(q_c), _ptr(k_c),
                                           _ptr(v), _ptr(q_p), _ptr(k_p), _ptr(gate), _ptr(plan.o), _ptr(plan.lse),
                                           _ptr(plan.ws), plan.ws_bytes, _stream(q_c.device)))
    return plan.o, plan.lse


NOALLOC_WORKSPACE_BYTES = 64 << 20


def window_attn_fwd_noalloc(q_c, k_c, v, q_p, k_p, w: int, o=None, lse=None, scale: float | None = None):
    """The forward through the allocation-free entry point (its workspace is the library's own
    per-GPU array of NOALLOC_WORKSPACE_BYTES). Writes into `o` / `lse` when given (`lse` may be
    None), else allocates them here in Python; returns (O, LSE or None)."""
    _require_gpu(q_c, k_c, v, q_p, k_p, o, lse)
    shape = _shape_of(q_c, w, q_p.shape[1])
    o = torch.empty_like(q_c) if o is None else o
    _check(lib().rib_window_attn_fwd_noalloc(ctypes.byref(shape), _dtype_code(q_c.dtype),
                                             0.0 if scale is None else float(scale), _ptr(q_c), _ptr(k_c), _ptr(v),
                                             _ptr(q_p), _ptr(k_p), _ptr(o), _ptr(lse), _stream(q_c.device)))
    return o, lse


def cla_gate(x: torch.Tensor, w_dw: torch.Tensor, b_dw, w_pw: torch.Tensor, b_pw, heads: int,
             out: torch.Tensor | None = None) -> torch.Tensor:
    """CLA gating map G = sigmoid(PW_1x1(DW_3x3(X))) of a [B, H, W, C] map (C = heads * d_c); returns G
    [B, H, W, C] in x's dtype (written into ``out`` when given). Weights float32: w_dw [C, 3, 3],
    b_dw [C] or None, w_pw [C, C], b_pw [C] or None."""
    _require_gpu(x, w_dw, b_dw, w_pw, b_pw, out)
    if x.dim() != 4:
        raise ValueError("x is [B, H, W, C]")
    B, H, W, C = x.shape
    if C % heads:
        raise ValueError("C must be a multiple of heads")
    for t in (w_dw, b_dw, w_pw, b_pw):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("CLA weights are float32")
    if w_dw.shape != (C, 3, 3) or w_pw.shape != (C, C):
        raise ValueError("w_dw must be [C, 3, 3] and w_pw [C, C]")
    s = Shape(B, H, W, heads, C // heads, 2, 1)
    if out is not None and (out.dtype != x.dtype or out.shape != x.shape):
        raise ValueError("out must match x's dtype and shape")
    g = torch.empty_like(x) if out is None else out
    _check(lib().rib_cla_gate(ctypes.byref(s), _dtype_code(x.dtype), _ptr(x), _ptr(w_dw), _ptr(b_dw), _ptr(w_pw),
                              _ptr(b_pw), _ptr(g), _stream(x.device)))
    return g


class BwdPlan:
    """Preallocated backward call: workspace and the five gradients for one shape."""

    def __init__(self, q_c, k_c, v, q_p, k_p, o, lse, d_o, w: int, scale: float | None = None):
        _require_gpu(q_c, k_c, v, q_p, k_p, o, lse, d_o)
        self.shape = _shape_of(q_c, w, q_p.shape[1])
        self.dtype = _dtype_code(q_c.dtype)
        self.inputs = (q_c, k_c, v, q_p, k_p, o, lse, d_o)
        self.scale = 0.0 if scale is None else float(scale)
        self.dq = torch.empty_like(q_c)
        self.dk = torch.empty_like(q_c)
        self.dv = torch.empty_like(q_c)
        self.dqp = torch.empty(q_p.shape, dtype=torch.float32, device=q_c.device)
        self.dkp = torch.empty(q_p.shape, dtype=torch.float32, device=q_c.device)
        self.ws_bytes = bwd_workspace_size(self.shape, q_c.dtype)
        self.ws = _workspace(self.ws_bytes, q_c.device)

    def run(self, stream=None):
        """Enqueues the call on the current stream, or on `stream` (a raw hipStream_t handle)."""
        q_c, k_c, v, q_p, k_p, o, lse, d_o = self.inputs
        st = _run_stream(stream, q_c.device, (*self.inputs, self.dq, self.dk, self.dv, self.dqp, self.dkp, self.ws))
        _check(lib().rib_window_attn_bwd(ctypes.byref(self.shape), self.dtype, self.scale, _ptr(q_c), _ptr(k_c),
                                         _ptr(v), _ptr(q_p), _ptr(k_p), _ptr(o), _ptr(lse), _ptr(d_o),
                                         _ptr(self.dq), _ptr(self.dk), _ptr(self.dv), _ptr(self.dqp),
                                         _ptr(self.dkp), _ptr(self.ws), self.ws_bytes, st))
        return self.dq, self.dk, self.dv, self.dqp, self.dkp


def window_attn_bwd(q_c, k_c, v, q_p, k_p, o, lse, d_o, w: int, scale: float | None = None):
    """Returns (dQ_c, dK_c, dV, dQ_p, dK_p); dQ_p and dK_p are float32 [w*w, r]."""
    return BwdPlan(q_c, k_c, v, q_p, k_p, o, lse, d_o, w, scale).run()


# ---------------------------------------------------------------- RPB comparison

def rpb_fwd_workspace_size(shape: Shape, dtype: torch.dtype) -> int:
    return int(lib().rib_rpb_fwd_workspace_size(ctypes.byref(shape), _dtype_code(dtype)))


class RpbFwdPlan:
    """Preallocated call of the relative-position-bias comparison kernel:
    O = softmax(scale Q_c K_c^T + B) V with B gathered from ``table`` [heads, (2w-1)^2] (float32)."""

    def __init__(self, q_c, k_c, v, table, w: int, scale: float | None = None, want_lse: bool = True):
        _require_gpu(q_c, k_c, v, table)
        self.shape = _shape_of(q_c, w, 0)
        self.dtype = _dtype_code(q_c.dtype)
        for t in (k_c, v):
            if t.dtype != q_c.dtype:
                raise TypeError("Q_c, K_c and V must share one dtype")
        if table.dtype != torch.float32 or table.shape != (q_c.shape[3], (2 * w - 1) ** 2):
            raise ValueError("table must be float32 [heads, (2w - 1)^2]")
        self.inputs = (q_c, k_c, v, table)
        self.scale = 0.0 if scale is None else float(scale)
        self.o = torch.empty_like(q_c)
        s = self.shape
        self.lse = torch.empty((s.B, s.H, s.W, s.heads), dtype=torch.float32, device=q_c.device) if want_lse else None
        self.ws_bytes = rpb_fwd_workspace_size(self.shape, q_c.dtype)
        if self.ws_bytes == 0:   # the shape or dtype is rejected: report why
            _check(lib().rib_rpb_window_attn_fwd(ctypes.byref(self.shape), self.dtype, self.scale, None, None, None,
                                                 None, None, None, None, 0, None))
        self.ws = _workspace(self.ws_bytes, q_c.device)

    def run(self, stream=None):
        """Enqueues the call on the current stream, or on `stream` (a raw hipStream_t handle)."""
        q_c, k_c, v, table = self.inputs
        st = _run_stream(stream, q_c.device, (*self.inputs, self.o, self.lse, self.ws))
        _check(lib().rib_rpb_window_attn_fwd(ctypes.byref(self.shape), self.dtype, self.scale, _ptr(q_c), _ptr(k_c),
                                             _ptr(v), _ptr(table), _ptr(self.o), _ptr(self.lse), _ptr(self.ws),
                                             self.ws_bytes, st))
        return self.o, self.lse


def rpb_window_attn_fwd(q_c, k_c, v, table, w: int, scale: float | None = None, want_lse: bool = True):
    """RPB comparison attention; returns (O, LSE or None). bfloat16 only; scale defaults to 1/sqrt(d_c)."""
    return RpbFwdPlan(q_c, k_c, v, table, w, scale, want_lse).run()


KERNEL_GROUPS = {"posgen": 0, "partition": 1, "attn_fwd": 2, "unpartition": 3, "bwd_prep": 4,
                 "attn_bwd_dkv": 5, "attn_bwd_dq": 6, "pos_reduce": 7, "posgen_bwd": 8, "rpb_attn_fwd": 9,
                 "cla_gate": 10}


def kernel_timing_enable(enable: bool = True):
    """Start (or stop) bracketing each kernel group of later calls with HIP events on their stream."""
    _check(lib().rib_kernel_timing_enable(1 if enable else 0))


def kernel_timing_select(*groups: str):
    """Time only the named kernel groups of later calls (none: timing off)."""
    mask = 0
    for g in groups:
        mask |= 1 << KERNEL_GROUPS[g]
    _check(lib().rib_kernel_timing_select(mask))


def kernel_timing_read(group: str):
    """(total milliseconds, launches) of one kernel group since the last read; waits for its events."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(lib().rib_kernel_timing_read(KERNEL_GROUPS[group], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def default_scale(d_c: int, r: int) -> float:
    return 1.0 / math.sqrt(d_c + r)

"""The allocation-free forward (rib_window_attn_fwd_noalloc) against the forward with a caller
workspace, through the C ABI: two calls in a row, the second on a smaller input, then a
float32 call; both paths run the same kernels over the same workspace layout, so the outputs
are compared bit for bit, and the small call against the float64 oracle at the method's bar."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import rib_synth
import windowed_attention_implicit_amd as rib
from gpu_util import check, device, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _inputs(B, H, W, heads, w, r, dt, seed, dev):
    wl = rib_synth.custom_workload(B, H, W, heads, 32, w, r, dt, seed=seed)
    x = rib_synth.make_inputs(wl)
    pk = rib_synth.make_positional(w * w, r, dt, seed=seed)
    t = [to_gpu(x[n], dev) for n in ("q_c", "k_c", "v")] + [to_gpu(p, dev) for p in pk]
    return wl, x, pk, t


def _noalloc(t, w, dev):
    q, k, v, qp, kp = t
    shape = rib.Shape(*q.shape, w, qp.shape[1])
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:4], float("nan"), dtype=torch.float32, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    status = rib.lib().rib_window_attn_fwd_noalloc(ctypes.byref(shape), rib._dtype_code(q.dtype), 0.0, P(q), P(k),
                                                   P(v), P(qp), P(kp), P(o), P(lse), st)
    assert status == rib.RIB_OK, rib.lib().rib_last_error()
    return o, lse


def test_noalloc_matches_workspace_forward():
    dev = device()
    cases = [
        (2, 192, 192, 6, 32, 16, "bf16", 71),   # 57 MB of workspace: the 32x32 layer of the window stack
        (1, 64, 96, 2, 16, 8, "bf16", 72),      # smaller, r = 8 (positional rows packed in the workspace)
        (1, 40, 40, 2, 20, 5, "f32", 73),       # float32: the per-token kernels, windowed rows in the workspace
    ]
    for (B, H, W, heads, w, r, dt, seed) in cases:
        print(f"noalloc case {(B, H, W, heads, w, r, dt)}", flush=True)
        wl, x, pk, t = _inputs(B, H, W, heads, w, r, dt, seed, dev)
        o, lse = _noalloc(t, w, dev)
        o_ref, l_ref = rib.window_attn_fwd(*t, w)
        torch.cuda.synchronize()
        same = torch.equal(o.view(torch.int16) if dt == "bf16" else o.view(torch.int32),
                           o_ref.view(torch.int16) if dt == "bf16" else o_ref.view(torch.int32))
        assert same and torch.equal(lse, l_ref), f"{(B, H, W, heads, w, r, dt)}: outputs differ"
        if B * H * W * heads <= 1 << 16:
            ro, rl = oracle.rib_window_attn_fwd(x["q_c"].f64(), x["k_c"].f64(), x["v"].f64(), pk[0].f64(),
                                                pk[1].f64(), w)
            check(f"noalloc {dt} O", to_f64(o), ro, dt)
            assert np.abs(to_f64(lse) - rl).max() <= (1e-5 if dt == "f32" else 2e-2)

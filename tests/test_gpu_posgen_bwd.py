"""GPU parity of the position-MLP weight gradients (rib_posgen_bwd) against the oracle.

Tolerance (float32 path): every output entry is a sum over the w*w tokens of
products a_t * b_t of float32 quantities (dz * phi, d_out * h, or single
terms for the biases), formed in blocks of 32 tokens and then summed over the
blocks. The forward error of such a sum is below (32 + blocks) * 2^-24 *
sum_t |a_t b_t| plus the rounding of the factors themselves, so the test
requires |gpu - oracle| <= 2e-5 * sum_t |a_t b_t| + 1e-7 per entry, with the
magnitude sum taken from the oracle's float64 intermediates.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import rib_synth
import windowed_attention_implicit_amd as rib
from gpu_util import device, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _magnitudes(w, F, m, r, dq, dk):
    """sum_t |a_t b_t| for every entry of dW1, db1, dW2, db2 (float64, from the oracle's steps)."""
    phi = oracle.fourier_features(w, F)
    b1 = np.zeros(m["w1"].shape[0]) if m["b1"] is None else m["b1"].astype(np.float64)
    z = phi @ m["w1"].astype(np.float64).T + b1
    d_out = np.abs(np.hstack([dq, dk]).astype(np.float64))
    dz = np.abs((np.hstack([dq, dk]).astype(np.float64) @ m["w2"].astype(np.float64)) * oracle.gelu_grad(z))
    return dz.T @ np.abs(phi), dz.sum(0), d_out.T @ np.abs(oracle.gelu(z)), d_out.sum(0)


def _check(w, F, hidden, r, m, dq, dk, got):
    ref = oracle.posgen_bwd(w, F, m["w1"], m["b1"], m["w2"], m["b2"], r, dq, dk)
    mags = _magnitudes(w, F, m, r, dq, dk)
    for name, g, rf, mg in zip(("dW1", "db1", "dW2", "db2"), got, ref, mags):
        g = to_f64(g)
        assert g.shape == rf.shape, (name, g.shape, rf.shape)
        err = np.abs(g - rf)
        bound = 2e-5 * mg + 1e-7
        print(f"  {name}: max-abs {err.max():.3e}  max err/bound {np.max(err / bound):.3f}", flush=True)
        assert (err <= bound).all(), name


CASES = [  # w, F, hidden, r, seed
    (96, 16, 64, 16, 1),      # the 96 x 96 window of the headline workload
    (16, 16, 64, 8, 2),
    (33, 16, 80, 8, 3),       # ragged: 1089 tokens, not a multiple of the 32-token block
    (7, 5, 40, 3, 4),
    (2, 1, 1, 1, 5),          # smallest window and MLP
    (64, 16, 64, 32, 6),      # widest rank
]


@pytest.mark.parametrize("w,F,hidden,r,seed", CASES)
def test_posgen_bwd_matches_oracle(w, F, hidden, r, seed):
    dev = device()
    print(f"posgen_bwd w={w} F={F} hidden={hidden} r={r}", flush=True)
    m = rib_synth.make_mlp(F, hidden, r, seed)
    dq, dk = rib_synth.make_pos_grads(w * w, r, seed + 100)
    t = lambda a: torch.from_numpy(a).to(dev)
    got = rib.posgen_bwd(w, t(m["w1"]), t(m["b1"]), t(m["w2"]), t(m["b2"]), r, t(dq), t(dk), n_freq=F)
    _check(w, F, hidden, r, m, dq, dk, got)


def test_posgen_bwd_workload_weights_no_bias_deterministic():
    """The headline workload's own N(0, 0.02^2) weights with no biases; two calls give the same bits,
    and NULL db1 / db2 leave dW1 / dW2 unchanged."""
    dev = device()
    wl = rib_synth.HEADLINE
    x = rib_synth.make_inputs(wl)
    W = {k: torch.from_numpy(x[k]).to(dev) for k in ("w1", "w2")}
    dq, dk = rib_synth.make_pos_grads(wl.w * wl.w, wl.r, 7)
    tq, tk = torch.from_numpy(dq).to(dev), torch.from_numpy(dk).to(dev)
    a = rib.posgen_bwd(wl.w, W["w1"], None, W["w2"], None, wl.r, tq, tk, n_freq=wl.n_freq)
    b = rib.posgen_bwd(wl.w, W["w1"], None, W["w2"], None, wl.r, tq, tk, n_freq=wl.n_freq)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    m = {"w1": x["w1"], "b1": None, "w2": x["w2"], "b2": None}
    _check(wl.w, wl.n_freq, wl.hidden, wl.r, m, dq, dk, a)
    # NULL bias outputs through the C ABI directly
    mlp = rib._Mlp(wl.n_freq, wl.hidden, wl.r, W["w1"].data_ptr(), None, W["w2"].data_ptr(), None)
    nbytes = rib.lib().rib_posgen_bwd_workspace_size(wl.w, ctypes.byref(mlp))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dw1 = torch.full_like(a[0], float("nan"))
    dw2 = torch.full_like(a[2], float("nan"))
    st = torch.cuda.current_stream(dev).cuda_stream
    assert rib.lib().rib_posgen_bwd(wl.w, ctypes.byref(mlp), tq.data_ptr(), tk.data_ptr(), dw1.data_ptr(), None,
                                    dw2.data_ptr(), None, ws.data_ptr(), nbytes, st) == rib.RIB_OK
    torch.cuda.synchronize(dev)
    assert torch.equal(dw1, a[0]) and torch.equal(dw2, a[2])


@pytest.mark.parametrize("dtype,bar", [("f32", 1e-4), ("bf16", 3e-2)])
def test_posgen_bwd_chained_after_attention_bwd(dtype, bar):
    """The whole trainable-bias chain on the GPU (posgen -> attention forward -> attention backward ->
    posgen backward) against the same chain in the oracle from the same inputs.

    The posgen backward is linear in (dQ_p, dK_p), so the chain's error is the image of the attention
    backward's error in those sums over units. Float32 attention keeps that near 1e-6, hence a 1e-4
    relative-L2 bar. With bf16 attention dQ_p, dK_p meet the bf16 bar (relative-L2 <= 1e-2, checked by
    the attention backward tests) and the linear map may enlarge a relative error a few times, hence
    3e-2 here; a wiring mistake (swapped or transposed operands, a missing GELU') misses either bar
    by orders of magnitude."""
    dev = device()
    wl = rib_synth.custom_workload(1, 32, 32, 2, 32, 16, 8, dtype, backward=True, seed=12)
    x = rib_synth.make_inputs(wl)
    m = rib_synth.make_mlp(wl.n_freq, wl.hidden, wl.r, 13)
    t = lambda a: torch.from_numpy(a).to(dev)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    qp, kp = rib.posgen(wl.w, t(m["w1"]), t(m["b1"]), t(m["w2"]), t(m["b2"]), wl.r, out_dtype=tdt)
    q, k, v, do = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v", "d_o"))
    o, lse = rib.window_attn_fwd(q, k, v, qp, kp, wl.w)
    _, _, _, dqp, dkp = rib.window_attn_bwd(q, k, v, qp, kp, o, lse, do, wl.w)
    got = rib.posgen_bwd(wl.w, t(m["w1"]), t(m["b1"]), t(m["w2"]), t(m["b2"]), wl.r, dqp, dkp)
    rqp, rkp = oracle.posgen(wl.w, wl.n_freq, m["w1"], m["b1"], m["w2"], m["b2"], wl.r)
    ref_pos = oracle.rib_window_attn_bwd(x["q_c"].f64(), x["k_c"].f64(), x["v"].f64(), rqp, rkp,
                                         x["d_o"].f64(), wl.w)[3:]
    ref = oracle.posgen_bwd(wl.w, wl.n_freq, m["w1"], m["b1"], m["w2"], m["b2"], wl.r, *ref_pos)
    for name, g, r in zip(("dW1", "db1", "dW2", "db2"), got, ref):
        g = to_f64(g)
        rel = np.linalg.norm(g - r) / np.linalg.norm(r)
        print(f"  chained {dtype} {name}: rel-L2 {rel:.3e}", flush=True)
        assert rel <= bar, name

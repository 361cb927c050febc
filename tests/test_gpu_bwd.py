"""GPU parity of the RIB window-attention backward against the float64 oracle.

The window-size stack (windows 16, 32, 64, 96 on a 192x192 map, batch 2,
6 heads) is checked layer by layer: all units where the oracle is fast,
sampled units plus size-independent invariants where it is not, and the
positional-token gradients at the real 64x64 / 96x96 window shapes on maps
small enough for the oracle to sum every unit.
"""

import numpy as np
import pytest
import torch

import oracle
import rib_synth
import windowed_attention_implicit_amd as rib
from gpu_util import check, device, sample_units, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _gpu_fwd_bwd(wl, x, dev, qpkp=None):
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    q, k, v, do = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v", "d_o"))
    if qpkp is None:
        W = {n: torch.from_numpy(x[n]).to(dev) for n in ("w1", "w2")}
        qp, kp = rib.posgen(wl.w, W["w1"], None, W["w2"], None, wl.r, n_freq=wl.n_freq, out_dtype=dt)
        rqp, rkp = oracle.posgen(wl.w, wl.n_freq, x["w1"], None, x["w2"], None, wl.r)
    else:
        qp, kp = (to_gpu(t, dev) for t in qpkp)
        rqp, rkp = qpkp[0].f64(), qpkp[1].f64()
    o, lse = rib.window_attn_fwd(q, k, v, qp, kp, wl.w)
    grads = rib.window_attn_bwd(q, k, v, qp, kp, o, lse, do, wl.w)
    torch.cuda.synchronize()
    return grads, rqp, rkp


def _compare(wl, x, grads, rqp, rkp, units=None, tag="", pos=True):
    ref = oracle.rib_window_attn_bwd(x["q_c"].f64(), x["k_c"].f64(), x["v"].f64(), rqp, rkp, x["d_o"].f64(),
                                     wl.w, units=units)
    names = ["dQ_c", "dK_c", "dV", "dQ_p", "dK_p"]
    for i, (n, g, r) in enumerate(zip(names, grads, ref)):
        if i >= 3 and not pos:
            continue
        check(f"{tag} {n}", to_f64(g), r, wl.dtype)


@pytest.mark.parametrize("shape", [
    # B, H, W, heads, d_c, w, r, dtype
    (1, 16, 16, 1, 32, 16, 8, "f32"),
    (2, 24, 24, 2, 32, 12, 20, "f32"),
    (1, 10, 15, 2, 32, 5, 3, "f32"),
    (1, 32, 32, 2, 32, 16, 16, "bf16"),
    (1, 10, 15, 2, 32, 5, 3, "bf16"),
    (2, 14, 14, 1, 32, 7, 1, "bf16"),
    (1, 24, 48, 2, 32, 24, 17, "bf16"),
    (1, 40, 40, 1, 32, 40, 32, "bf16"),
    # windows whose side divides 64 at r <= 16: K_c and V read in their maps (several windows
    # per map row, several heads, H != W)
    (2, 16, 48, 3, 32, 8, 5, "bf16"),
    (1, 32, 96, 2, 32, 16, 12, "bf16"),
    (1, 64, 128, 2, 32, 32, 9, "bf16"),
    # windows of more than 2048 tokens
    (1, 50, 100, 2, 32, 50, 8, "bf16"),     # N = 2500: a 4-row last tile, r padded to 16
    (1, 48, 48, 3, 32, 48, 16, "bf16"),     # N = 2304: whole tiles
    # d_c = 64 (the one-thread-per-key / per-query kernels)
    (1, 10, 15, 2, 64, 5, 3, "bf16"),
    (1, 16, 16, 2, 64, 16, 20, "bf16"),
    (1, 24, 24, 1, 64, 12, 16, "f32"),
], ids=lambda s: "B{}_H{}_W{}_h{}_d{}_w{}_r{}_{}".format(*s))
def test_bwd_small_and_ragged(shape):
    dev = device()
    B, H, W, heads, d, w, r, dt = shape
    print(f"bwd edge {shape}", flush=True)
    wl = rib_synth.custom_workload(B, H, W, heads, d, w, r, dt, backward=True, seed=sum(shape[:7]) + 1)
    x = rib_synth.make_inputs(wl)
    qpkp = rib_synth.make_positional(w * w, r, dt, seed=w * 3 + r)
    grads, rqp, rkp = _gpu_fwd_bwd(wl, x, dev, qpkp)
    _compare(wl, x, grads, rqp, rkp, tag=str(shape))


@pytest.fixture(scope="module")
def stack_inputs():
    return rib_synth.make_stack_inputs()


@pytest.mark.parametrize("layer", [0, 1], ids=["w16", "w32"])
def test_bwd_stack_layers_full(stack_inputs, layer):
    dev = device()
    wl, x = rib_synth.STACK[layer], stack_inputs[layer]
    print(f"bwd {wl.name}: all {wl.units} units", flush=True)
    grads, rqp, rkp = _gpu_fwd_bwd(wl, x, dev)
    _compare(wl, x, grads, rqp, rkp, tag=wl.name)


@pytest.mark.parametrize("layer,k", [(2, 3), (3, 2)], ids=["w64", "w96"])
def test_bwd_stack_layers_sampled(stack_inputs, layer, k):
    dev = device()
    wl, x = rib_synth.STACK[layer], stack_inputs[layer]
    grads, rqp, rkp = _gpu_fwd_bwd(wl, x, dev)
    units = sample_units(wl, k, seed=layer)
    print(f"bwd {wl.name}: units {units}", flush=True)
    _compare(wl, x, grads, rqp, rkp, units=units, tag=wl.name, pos=False)
    # invariants over every unit: rows of dS sum to zero, rows of P sum to one
    dq, dk, dv, dqp, dkp = (to_f64(g) for g in grads)
    w = wl.w
    do = x["d_o"].f64()
    shp = (wl.B, wl.H // w, w, wl.W // w, w, wl.heads, wl.d_c)
    sum_dk = dk.reshape(shp).sum(axis=(2, 4))
    sum_dv = dv.reshape(shp).sum(axis=(2, 4))
    sum_do = do.reshape(shp).sum(axis=(2, 4))
    scale_k = np.abs(dk).reshape(shp).sum(axis=(2, 4)).max()
    print(f"max |sum_j dK_c| {np.abs(sum_dk).max():.3e} (sum |dK_c| {scale_k:.3e}); "
          f"max |sum dV - sum dO| {np.abs(sum_dv - sum_do).max():.3e}", flush=True)
    assert np.abs(sum_dk).max() <= 1e-2 * scale_k
    assert np.abs(sum_dv - sum_do).max() <= 2e-2 * np.abs(do).reshape(shp).sum(axis=(2, 4)).max()
    assert np.abs(dkp.sum(0)).max() <= 1e-2 * np.abs(dkp).sum(0).max()
    assert np.isfinite(dqp).all() and np.isfinite(dkp).all()


@pytest.mark.parametrize("w", [64, 96])
def test_bwd_positional_grads_real_window(w):
    """dQ_p, dK_p sum over every unit: checked on a map the oracle covers fully."""
    dev = device()
    wl = rib_synth.custom_workload(1, w, w, 3, 32, w, 16, "bf16", backward=True, seed=w)
    x = rib_synth.make_inputs(wl)
    grads, rqp, rkp = _gpu_fwd_bwd(wl, x, dev)
    _compare(wl, x, grads, rqp, rkp, tag=f"w{w} x3 heads")


def test_bwd_deterministic():
    dev = device()
    wl = rib_synth.custom_workload(2, 64, 64, 3, 32, 32, 16, "bf16", backward=True, seed=21)
    x = rib_synth.make_inputs(wl)
    g1, _, _ = _gpu_fwd_bwd(wl, x, dev)
    g2, _, _ = _gpu_fwd_bwd(wl, x, dev)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_bwd_outputs_ordered_on_caller_stream():
    """Every kernel of the backward is queued on the caller's stream: outputs poisoned with NaN
    on a non-default stream, then copied on that stream right behind the backward (no device
    synchronization), must hold the final gradients, equal bit for bit to a reference run."""
    dev = device()
    w = 48
    wl = rib_synth.custom_workload(2, 96, 96, 3, 32, w, 16, "bf16", backward=True, seed=31)
    x = rib_synth.make_inputs(wl)
    q, k, v, do = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v", "d_o"))
    qp, kp = (to_gpu(t, dev) for t in rib_synth.make_positional(w * w, 16, "bf16", seed=5))
    o, lse = rib.window_attn_fwd(q, k, v, qp, kp, w)
    ref = [g.clone() for g in rib.window_attn_bwd(q, k, v, qp, kp, o, lse, do, w)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=dev)
    got = []
    with torch.cuda.stream(s):
        plan = rib.BwdPlan(q, k, v, qp, kp, o, lse, do, w)
        outs = (plan.dq, plan.dk, plan.dv, plan.dqp, plan.dkp)
        for _ in range(3):
            for g in outs:
                g.fill_(float("nan"))
            plan.run()
            got.append([g.clone() for g in outs])
    s.synchronize()
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t
    for rep in got:
        for a, b in zip(rep, ref):
            assert torch.equal(bits(a), bits(b))


def test_bwd_empty_batch_zero_positional_grads():
    dev = device()
    e = torch.empty((0, 32, 32, 2, 32), dtype=torch.bfloat16, device=dev)
    qp = torch.randn(256, 16, device=dev).to(torch.bfloat16)
    lse = torch.empty((0, 32, 32, 2), dtype=torch.float32, device=dev)
    dq, dk, dv, dqp, dkp = rib.window_attn_bwd(e, e, e, qp, qp, e, lse, e, 16)
    torch.cuda.synchronize()
    assert dq.shape == e.shape
    assert not dqp.any() and not dkp.any()


def test_bwd_max_window_invariants():
    """w = 256 (N = 65536 tokens per unit, 2 heads): the oracle's N x N matrices do not fit, so the
    gradients are held to identities of the method that hold at any size, per unit: every row of
    dS sums to zero, so sum_j dK_hat_j = 0 (content and positional parts), and every row of P sums
    to one, so sum_j dV_j = sum_i dO_i."""
    dev = device()
    w = 256
    wl = rib_synth.custom_workload(1, 256, 256, 2, 32, w, 16, "bf16", backward=True, seed=257)
    x = rib_synth.make_inputs(wl)
    qpkp = rib_synth.make_positional(w * w, 16, "bf16", seed=5)
    (dq, dk, dv, dqp, dkp), _, _ = _gpu_fwd_bwd(wl, x, dev, qpkp)
    for t in (dq, dk, dv, dqp, dkp):
        assert torch.isfinite(t.float()).all()
    dk64, dv64 = to_f64(dk), to_f64(dv)
    do64 = x["d_o"].f64()
    for h in range(2):
        sk = dk64[0, :, :, h, :].reshape(w * w, -1).sum(0)
        mag = np.abs(dk64[0, :, :, h, :]).reshape(w * w, -1).sum(0)
        print(f"head {h}: |sum dK_c| {np.abs(sk).max():.3e} vs sum |dK_c| {mag.max():.3e}", flush=True)
        assert (np.abs(sk) <= 2e-3 * mag + 1e-3).all()
        sv = dv64[0, :, :, h, :].reshape(w * w, -1).sum(0)
        so = do64[0, :, :, h, :].reshape(w * w, -1).sum(0)
        print(f"head {h}: max |sum dV - sum dO| {np.abs(sv - so).max():.3e}", flush=True)
        # both backward kernels form the forward's bf16 scores, so P is normalized by the forward's
        # LSE up to fp32 and bf16 rounding (observed <= 8e-3 on sums of size ~256)
        assert np.abs(sv - so).max() <= 0.05
    # with one unit per head, dK_p is the sum of both heads' per-unit parts, each summing to zero
    skp = to_f64(dkp).sum(0)
    print(f"|sum dK_p| {np.abs(skp).max():.3e} vs sum |dK_p| {np.abs(to_f64(dkp)).sum(0).max():.3e}", flush=True)
    assert (np.abs(skp) <= 2e-3 * np.abs(to_f64(dkp)).sum(0) + 1e-3).all()

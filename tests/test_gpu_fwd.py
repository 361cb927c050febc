"""GPU parity of the RIB window-attention forward against the float64 oracle.

Small and ragged shapes are compared on every output; the method's full-size
workloads are compared on sampled (batch, window, head) units, which the
oracle computes one at a time, plus size-independent closed forms.
"""

import numpy as np
import pytest
import torch

import oracle
import rib_synth
import windowed_attention_implicit_amd as rib
from gpu_util import check, device, sample_units, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _run(wl, x, dev, use_posgen=True, qpkp=None):
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    q, k, v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
    if use_posgen:
        W = {n: torch.from_numpy(x[n]).to(dev) for n in ("w1", "w2")}
        qp, kp = rib.posgen(wl.w, W["w1"], None, W["w2"], None, wl.r, n_freq=wl.n_freq, out_dtype=dt)
        rqp, rkp = oracle.posgen(wl.w, wl.n_freq, x["w1"], None, x["w2"], None, wl.r)
    else:
        qp, kp = (to_gpu(t, dev) for t in qpkp)
        rqp, rkp = qpkp[0].f64(), qpkp[1].f64()
    o, lse = rib.window_attn_fwd(q, k, v, qp, kp, wl.w)
    torch.cuda.synchronize()
    return o, lse, rqp, rkp


def _compare(wl, x, o, lse, rqp, rkp, units=None, tag="", lse_rel=0.0):
    """O at the method's bar; LSE within 1e-5 (float32) or 2e-2 + lse_rel * max|LSE| (bf16)."""
    ro, rl = oracle.rib_window_attn_fwd(x["q_c"].f64(), x["k_c"].f64(), x["v"].f64(), rqp, rkp, wl.w, units=units)
    check(f"{tag} O", to_f64(o), ro, wl.dtype)
    lerr = np.nanmax(np.abs(to_f64(lse) - rl))
    tol = 1e-5 if wl.dtype == "f32" else 2e-2 + lse_rel * np.nanmax(np.abs(rl))
    print(f"{tag} LSE max-abs {lerr:.3e} (bar {tol:.3e})", flush=True)
    assert lerr <= tol


def test_fwd_w16_single_fp32():
    dev = device()
    wl = rib_synth.WORKLOADS["w16_single_fp32"]
    x = rib_synth.make_inputs(wl)
    o, lse, rqp, rkp = _run(wl, x, dev)
    _compare(wl, x, o, lse, rqp, rkp, tag=wl.name)


def test_fwd_w32_map256_full():
    dev = device()
    wl = rib_synth.WORKLOADS["w32_map256_bf16"]
    x = rib_synth.make_inputs(wl)
    o, lse, rqp, rkp = _run(wl, x, dev)
    _compare(wl, x, o, lse, rqp, rkp, tag=wl.name)


# Units of the 96 x 96 workload in the split tail of the launch (each XCD's items past its last
# whole round of workgroup slots, cut into key ranges and summed by the combine kernel): with
# 3456 items over 8 XCDs of 96 slots, XCD x runs items 432x .. 432x + 431 and its tail is the
# last 48 of them, i.e. the end of unit 12x + 10 and all of unit 12x + 11.
W96_TAIL_UNITS = (10, 11, 95)


@pytest.mark.parametrize("name,k,tail", [("w64_map128x8_bf16", 6, ()), ("w96_map192x4_bf16", 3, W96_TAIL_UNITS)])
def test_fwd_large_workloads_sampled(name, k, tail):
    dev = device()
    wl = rib_synth.WORKLOADS[name]
    x = rib_synth.make_inputs(wl)
    o, lse, rqp, rkp = _run(wl, x, dev)
    units = sample_units(wl, k, seed=1, include=tail)
    print(f"{name}: units {units}", flush=True)
    _compare(wl, x, o, lse, rqp, rkp, units=units, tag=name)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("shape", [
    # B, H, W, heads, d_c, w, r, dtype
    (1, 10, 15, 2, 32, 5, 3, "bf16"),
    (2, 14, 14, 1, 32, 7, 1, "bf16"),
    (1, 20, 20, 3, 32, 10, 16, "bf16"),
    (1, 24, 48, 2, 32, 24, 17, "bf16"),
    (1, 40, 40, 1, 32, 40, 32, "bf16"),
    (1, 2, 2, 1, 32, 2, 4, "bf16"),
    # windows whose side divides 64 with r <= 16: K_c and V read in their maps (no gather)
    (1, 16, 24, 2, 32, 8, 5, "bf16"),
    (2, 64, 48, 3, 32, 16, 16, "bf16"),
    (1, 64, 96, 2, 32, 32, 9, "bf16"),
    (1, 128, 64, 1, 32, 64, 16, "bf16"),
    # w*w >= 2048: the last partial round of workgroups is cut into key ranges and combined
    (1, 50, 100, 2, 32, 50, 8, "bf16"),    # N = 2500: a 4-key last tile, r padded to 16
    (1, 48, 48, 1, 32, 48, 32, "bf16"),    # N = 2304: whole tiles, two positional K-steps
    (1, 10, 15, 2, 32, 5, 3, "f32"),
    (2, 24, 24, 2, 32, 12, 20, "f32"),
    (1, 32, 32, 1, 32, 32, 8, "f32"),
    # d_c = 64 (the one-thread-per-query kernels)
    (1, 10, 15, 2, 64, 5, 3, "bf16"),
    (1, 24, 24, 2, 64, 12, 16, "bf16"),
    (1, 20, 20, 1, 64, 10, 32, "f32"),
], ids=lambda s: "B{}_H{}_W{}_h{}_d{}_w{}_r{}_{}".format(*s))
def test_fwd_ragged_and_edge_shapes(shape):
    dev = device()
    B, H, W, heads, d, w, r, dt = shape
    print(f"fwd edge {shape}", flush=True)
    wl = rib_synth.custom_workload(B, H, W, heads, d, w, r, dt, seed=sum(shape[:7]))
    x = rib_synth.make_inputs(wl)
    qpkp = rib_synth.make_positional(w * w, r, dt, seed=w + r)
    o, lse, rqp, rkp = _run(wl, x, dev, use_posgen=False, qpkp=qpkp)
    _compare(wl, x, o, lse, rqp, rkp, tag=str(shape))


def test_fwd_closed_forms_at_full_size():
    """At the 96x96 shape: constant V gives constant O; zero scores give O = window mean of V."""
    dev = device()
    wl = rib_synth.custom_workload(1, 192, 192, 2, 32, 96, 16, "bf16", seed=5)
    x = rib_synth.make_inputs(wl)
    q, k = to_gpu(x["q_c"], dev), to_gpu(x["k_c"], dev)
    qp, kp = (to_gpu(t, dev) for t in rib_synth.make_positional(96 * 96, 16, "bf16", seed=3))
    vc = torch.linspace(-2, 2, 32, device=dev).to(torch.bfloat16).expand(1, 192, 192, 2, 32).contiguous()
    o, _ = rib.window_attn_fwd(q, k, vc, qp, kp, 96)
    err = (o.float() - vc.float()).abs().max().item()
    print(f"constant V: max-abs {err:.3e}", flush=True)
    assert err <= 2e-2
    z = torch.zeros_like(q)
    zp = torch.zeros_like(qp)
    v = to_gpu(x["v"], dev)
    o, lse = rib.window_attn_fwd(z, z, v, zp, zp, 96)
    vw = v.float().reshape(1, 2, 96, 2, 96, 2, 32)
    mean = vw.mean(dim=(2, 4), keepdim=True).expand_as(vw).reshape(1, 192, 192, 2, 32)
    err = (o.float() - mean).abs().max().item()
    print(f"zero scores: max-abs {err:.3e}", flush=True)
    assert err <= 2e-3
    assert torch.allclose(lse, torch.full_like(lse, float(np.log(96 * 96))), atol=1e-4)


def test_fwd_deterministic_and_empty():
    dev = device()
    wl = rib_synth.custom_workload(2, 64, 64, 3, 32, 32, 16, "bf16", seed=9)
    x = rib_synth.make_inputs(wl)
    qpkp = rib_synth.make_positional(32 * 32, 16, "bf16", seed=4)
    o1, l1, _, _ = _run(wl, x, dev, use_posgen=False, qpkp=qpkp)
    o2, l2, _, _ = _run(wl, x, dev, use_posgen=False, qpkp=qpkp)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    e = torch.empty((0, 64, 64, 3, 32), dtype=torch.bfloat16, device=dev)
    qp, kp = (to_gpu(t, dev) for t in qpkp)
    o, lse = rib.window_attn_fwd(e, e, e, qp, kp, 32)
    assert o.shape == e.shape and lse.shape == (0, 64, 64, 3)


def test_fwd_bias_cancels_content():
    """Q_p K_p^T = -Q_c K_c^T makes every score zero: O is the window mean of V (the
    content and bias terms enter one dot product)."""
    dev = device()
    w, r = 8, 32
    wl = rib_synth.custom_workload(1, 8, 8, 1, 32, w, r, "f32", seed=2)
    x = rib_synth.make_inputs(wl)
    qc = x["q_c"].data.reshape(64, 32)
    kc = x["k_c"].data.reshape(64, 32)
    qp = torch.from_numpy(np.ascontiguousarray(qc)).to(dev)
    kp = torch.from_numpy(np.ascontiguousarray(-kc)).to(dev)
    q, k, v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
    o, _ = rib.window_attn_fwd(q, k, v, qp, kp, w)
    mean = v.reshape(64, 32).mean(0)
    err = (o.reshape(64, 32) - mean).abs().max().item()
    assert err <= 1e-5, err


def _many_items_workload(seed):
    """w = 24 on a 192 x 192 map with 3 heads: 192 windows x heads, each with 3 query blocks and a
    ragged 9th key tile, small enough for the oracle to check every output."""
    return rib_synth.custom_workload(1, 192, 192, 3, 32, 24, 16, "bf16", seed=seed)


def test_fwd_many_items_full():
    dev = device()
    wl = _many_items_workload(21)
    x = rib_synth.make_inputs(wl)
    o, lse, rqp, rkp = _run(wl, x, dev)
    _compare(wl, x, o, lse, rqp, rkp, tag="w24 map192 full")
    o2, lse2, _, _ = _run(wl, x, dev)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)


def test_fwd_exact_pass_forced():
    """Channel 0 of token 0's key is 127 in every window while every query has 0 there and 8 in
    channel 1: the per-query bound |q'| max|k| (~211 log2 units) overshoots the largest score (~7)
    by more than the 124 units the shifted tier absorbs (it shifts by the bound - 64), the row sums
    fall below 2^-60, and every workgroup recomputes its rows with the exact pass."""
    dev = device()
    wl = _many_items_workload(22)
    x = rib_synth.make_inputs(wl)
    q = x["q_c"].data.view(np.int16).copy()
    k = x["k_c"].data.view(np.int16).copy()
    bf = lambda v: int(rib_synth.bf16_bits(np.array([v], np.float32))[0].view(np.int16))
    q[..., 0] = bf(0.0)
    q[..., 1] = bf(8.0)
    k[:, ::24, ::24, :, 0] = bf(127.0)   # token 0 of every 24 x 24 window
    x["q_c"] = rib_synth.Tensor("bf16", q.view(x["q_c"].data.dtype))
    x["k_c"] = rib_synth.Tensor("bf16", k.view(x["k_c"].data.dtype))
    o, lse, rqp, rkp = _run(wl, x, dev)
    _compare(wl, x, o, lse, rqp, rkp, tag="exact pass")


def _combine_launches(fn):
    """Runs fn() with the split-tail combine timed; returns how many combines it launched."""
    rib.kernel_timing_select("unpartition")
    rib.kernel_timing_read("unpartition")
    try:
        fn()
        return rib.kernel_timing_read("unpartition")[1]
    finally:
        rib.kernel_timing_select()


def test_fwd_split_tail_mixed_passes():
    """w = 48 (N = 2304) on a 96 x 96 map, 2 heads: 72 work items, fewer than one round of
    workgroup slots, so every item is cut into key ranges. Every query is 7.84375 in channel 1
    and 0 elsewhere (scaled by scale * log2(e) it rounds to bf16 within 3.3e-4, so the large
    scores below keep their accuracy). Key token 0 of each window carries 96 in channel 0,
    which no query sees but which lifts the per-query bound |q'| max |k_hat| to ~157 log2 units,
    so the rows take the shifted tier with shift ~93 (the bound - 64); key token 2000 carries 40
    in channel 1 (score ~65). Ranges without token 2000 (scores below ~8) underflow and take the
    exact pass with their own running max; the range with it keeps the shift, so the combine
    adds pieces with different shifts."""
    dev = device()
    wl = rib_synth.custom_workload(1, 96, 96, 2, 32, 48, 16, "bf16", seed=48)
    x = rib_synth.make_inputs(wl)
    q = x["q_c"].data.view(np.int16).copy()
    k = x["k_c"].data.view(np.int16).copy()
    bf = lambda v: int(rib_synth.bf16_bits(np.array([v], np.float32))[0].view(np.int16))
    q[...] = bf(0.0)
    q[..., 1] = bf(7.84375)
    k[:, ::48, ::48, :, 0] = bf(96.0)                 # token 0 of every 48 x 48 window
    ty, tx = divmod(2000, 48)
    k[:, ty::48, tx::48, :, 1] = bf(40.0)             # token 2000
    x["q_c"] = rib_synth.Tensor("bf16", q.view(x["q_c"].data.dtype))
    x["k_c"] = rib_synth.Tensor("bf16", k.view(x["k_c"].data.dtype))
    out = {}
    n = _combine_launches(lambda: out.update(zip(("o", "lse", "rqp", "rkp"), _run(wl, x, dev))))
    print(f"split combines launched: {n}", flush=True)
    assert n == 1
    # LSE ~45: the bf16 rounding of the pre-scaled query (relative 3.3e-4 here) is ~0.014 of it
    _compare(wl, x, out["o"], out["lse"], out["rqp"], out["rkp"], tag="split tail, mixed passes", lse_rel=2.0 ** -9)


def test_fwd_split_tail_at_full_size_launches():
    """The 96 x 96 workload (batch 4, 6 heads: 3456 work items over 512 workgroup slots)
    combines a split tail; w = 32 (16 key tiles) never splits."""
    dev = device()
    for (B, w, expect) in ((4, 96, 1), (2, 32, 0)):
        wl = rib_synth.custom_workload(B, 192, 192, 6, 32, w, 16, "bf16", seed=w)
        x = rib_synth.make_inputs(wl)
        q, k, v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
        qp, kp = (to_gpu(t, dev) for t in rib_synth.make_positional(w * w, 16, "bf16", seed=w))
        n = _combine_launches(lambda: rib.window_attn_fwd(q, k, v, qp, kp, w))
        print(f"w = {w}: split combines {n}", flush=True)
        assert n == expect


@pytest.mark.parametrize("kind", ["overflow", "underflow"])
def test_fwd_map_kv_exact_pass(kind):
    """Windows whose side divides 64 run without a key-norm bound: the fast pass takes exp2 of the
    unshifted scores and checks its row sums and accumulators afterwards. Overflow: token 0's key
    and every query carry 60 in channel 0, so scores reach ~750 log2 units and exp2 overflows.
    Underflow: every query carries -60 and every key +60 there, so every score is below -700 and
    every P underflows. Either way the workgroups rerun with the exact pass."""
    dev = device()
    wl = rib_synth.custom_workload(1, 32, 48, 2, 32, 16, 16, "bf16", seed=30 if kind == "overflow" else 31)
    x = rib_synth.make_inputs(wl)
    bf = lambda v: rib_synth.bf16_bits(np.asarray(v, np.float32)).view(np.int16)
    q = x["q_c"].data.view(np.int16).copy()
    k = x["k_c"].data.view(np.int16).copy()
    if kind == "overflow":
        q[..., 0] = bf(60.0)
        k[:, ::16, ::16, :, 0] = bf(60.0)
    else:
        q[..., 0] = bf(-60.0)
        k[..., 0] = bf(60.0)
    x["q_c"] = rib_synth.Tensor("bf16", q.view(x["q_c"].data.dtype))
    x["k_c"] = rib_synth.Tensor("bf16", k.view(x["k_c"].data.dtype))
    o, lse, rqp, rkp = _run(wl, x, dev)
    # scores of hundreds of log2 units: the bf16 query operand's relative rounding shows in the LSE
    _compare(wl, x, o, lse, rqp, rkp, tag=f"map K/V, {kind}", lse_rel=2 * 2.0 ** -9)


def test_fwd_shifted_tier_large_scores():
    """Every query is 20 in channel 0; key channel 0 is uniform in [-16, 16], so the per-query
    bound |q'| max |k_hat| exceeds 64 log2 units and the bound is nearly tight (the best key of
    every window scores within a few units of it): the workgroups take the shifted exponent
    tier, whose row sums stay far above the underflow guard, so no exact pass runs."""
    dev = device()
    wl = rib_synth.custom_workload(1, 96, 96, 2, 32, 48, 16, "bf16", seed=64)
    x = rib_synth.make_inputs(wl)
    q = x["q_c"].data.view(np.int16).copy()
    bf = lambda v: rib_synth.bf16_bits(np.asarray(v, np.float32)).view(np.int16)
    q[...] = bf(0.0)
    q[..., 0] = bf(20.0)
    kk = x["k_c"].data.view(np.int16).copy()
    rng = np.random.default_rng(65)
    kk[..., 0] = bf(rng.uniform(-16.0, 16.0, size=kk.shape[:-1]))
    kk[:, ::48, ::48, :, 0] = bf(16.0)                # token 0 of every window: the bound is reached
    x["q_c"] = rib_synth.Tensor("bf16", q.view(x["q_c"].data.dtype))
    x["k_c"] = rib_synth.Tensor("bf16", kk.view(x["k_c"].data.dtype))
    o, lse, rqp, rkp = _run(wl, x, dev)
    # the query enters the score MFMAs as bf16(scale log2(e) q): a relative rounding of up to 2^-9
    # per score, 0.1 at these LSEs of ~49; O does not depend on a per-row shift and keeps the bar
    _compare(wl, x, o, lse, rqp, rkp, tag="shifted tier, large scores", lse_rel=2 * 2.0 ** -9)


def test_fwd_shifted_tier_large_values():
    """V scaled by 2^41 (above the 2^40 limit of the unshifted tier) gives O scaled by 2^41: the
    shifted tier on the same scores reproduces the unscaled result."""
    dev = device()
    wl = rib_synth.custom_workload(1, 96, 96, 2, 32, 48, 16, "bf16", seed=66)
    x = rib_synth.make_inputs(wl)
    o, lse, rqp, rkp = _run(wl, x, dev)
    big = 2.0 ** 41
    q, k, v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
    w1, w2 = torch.from_numpy(x["w1"]).to(dev), torch.from_numpy(x["w2"]).to(dev)
    qp, kp = rib.posgen(wl.w, w1, None, w2, None, wl.r, n_freq=wl.n_freq)
    o2, lse2 = rib.window_attn_fwd(q, k, (v.float() * big).to(torch.bfloat16), qp, kp, wl.w)
    torch.cuda.synchronize()
    _compare(wl, x, (o2.float() / big).to(torch.bfloat16), lse2, rqp, rkp, tag="shifted tier, V * 2^41")
    _compare(wl, x, o, lse, rqp, rkp, tag="unshifted tier, same inputs")


def test_fwd_plan_on_raw_stream():
    """FwdPlan.run(stream=...) with a raw stream handle (the plan's buffers recorded on that
    stream) gives the bits of a run on the current stream."""
    dev = device()
    wl = rib_synth.custom_workload(1, 64, 64, 2, 32, 32, 16, "bf16", seed=12)
    x = rib_synth.make_inputs(wl)
    q, k, v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
    qp, kp = (to_gpu(t, dev) for t in rib_synth.make_positional(32 * 32, 16, "bf16", seed=12))
    o_ref, l_ref = rib.window_attn_fwd(q, k, v, qp, kp, 32)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    plan = rib.FwdPlan(q, k, v, qp, kp, 32)
    o, lse = plan.run(stream=side.cuda_stream)
    side.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, l_ref)


def test_fwd_max_window_sampled_rows():
    """The largest window (w = 256, N = 65536 tokens per unit, 2 heads): each output row depends
    only on its own query row and every key, so the oracle computes sampled rows exactly, with
    the whole key set, without the full N x N matrix."""
    dev = device()
    w = 256
    wl = rib_synth.custom_workload(1, 256, 256, 2, 32, w, 16, "bf16", seed=256)
    x = rib_synth.make_inputs(wl)
    o, lse, rqp, rkp = _run(wl, x, dev)
    rng = np.random.default_rng(7)
    rows = np.sort(np.concatenate([[0, 1, w - 1, w * w - 1], rng.choice(w * w, 60, replace=False)]))
    scale = rib.default_scale(32, 16)
    tok = lambda t, h: t.f64()[0, :, :, h, :].reshape(w * w, -1)
    og, lg = to_f64(o), to_f64(lse)
    for h in range(2):
        ro, rl, _ = oracle.attention_window_fwd(tok(x["q_c"], h)[rows], tok(x["k_c"], h), tok(x["v"], h),
                                                rqp[rows], rkp, scale)
        check(f"w256 head {h} O rows", og[0, :, :, h, :].reshape(w * w, -1)[rows], ro, "bf16")
        lerr = np.abs(lg[0, :, :, h].reshape(-1)[rows] - rl).max()
        assert lerr <= 2e-2, lerr
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()

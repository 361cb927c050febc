"""GPU parity of posgen and of the window partition / unpartition gather."""

import numpy as np
import pytest
import torch

import oracle
import rib_synth
import windowed_attention_implicit_amd as rib
from gpu_util import device, to_f64, to_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w,r", [(16, 8), (32, 8), (64, 16), (96, 16), (5, 3), (7, 32), (2, 1), (256, 16)])
def test_posgen_f32_matches_oracle(w, r):
    dev = device()
    print(f"posgen f32 w={w} r={r}", flush=True)
    rng = np.random.default_rng(w * 31 + r)
    F, Hd = 16, 64
    w1 = (0.3 * rng.standard_normal((Hd, 4 * F))).astype(np.float32)
    b1 = (0.1 * rng.standard_normal(Hd)).astype(np.float32)
    w2 = (0.3 * rng.standard_normal((2 * r, Hd))).astype(np.float32)
    b2 = (0.1 * rng.standard_normal(2 * r)).astype(np.float32)
    t = lambda a: torch.from_numpy(a).to(dev)
    qp, kp = rib.posgen(w, t(w1), t(b1), t(w2), t(b2), r, out_dtype=torch.float32)
    rqp, rkp = oracle.posgen(w, F, w1, b1, w2, b2, r)
    for name, g, ref in (("q_p", qp, rqp), ("k_p", kp, rkp)):
        err = np.abs(to_f64(g) - ref).max()
        print(f"  {name}: max-abs {err:.3e}", flush=True)
        assert err <= 1e-5, (name, err)


@pytest.mark.parametrize("wl", list(rib_synth.WORKLOADS.values()) + list(rib_synth.STACK), ids=lambda wl: wl.name)
def test_posgen_workloads(wl):
    """The workloads' own posgen (weights N(0, 0.02^2)) in their run precision."""
    dev = device()
    x = rib_synth.make_inputs(wl)
    W = {k: torch.from_numpy(x[k]).to(dev) for k in ("w1", "w2")}
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    qp, kp = rib.posgen(wl.w, W["w1"], None, W["w2"], None, wl.r, out_dtype=dt)
    rqp, rkp = oracle.posgen(wl.w, wl.n_freq, x["w1"], None, x["w2"], None, wl.r)
    for g, ref in ((qp, rqp), (kp, rkp)):
        err = np.abs(to_f64(g) - ref)
        if wl.dtype == "f32":
            assert err.max() <= 1e-5
        else:  # one bf16 rounding of each value
            assert (err <= np.abs(ref) * 2.0 ** -8 + 1e-7).all(), err.max()


def test_posgen_bias_identity_and_rank():
    """Every window shares one bias; the GPU bias Q_p K_p^T has rank <= r."""
    dev = device()
    wl = rib_synth.STACK[3]
    x = rib_synth.make_inputs(wl)
    W = {k: torch.from_numpy(x[k]).to(dev) for k in ("w1", "w2")}
    qp, kp = rib.posgen(wl.w, W["w1"], None, W["w2"], None, wl.r, out_dtype=torch.float32)
    qp2, kp2 = rib.posgen(wl.w, W["w1"], None, W["w2"], None, wl.r, out_dtype=torch.float32)
    assert torch.equal(qp, qp2) and torch.equal(kp, kp2)
    bias = to_f64(qp) @ to_f64(kp).T
    s = np.linalg.svd(bias, compute_uv=False)
    assert np.all(s[wl.r:] <= 1e-10 * s[0])


@pytest.mark.parametrize("B,H,W,heads,d,w,dt", [
    (1, 16, 16, 1, 32, 16, "f32"), (2, 12, 18, 3, 32, 6, "bf16"), (1, 10, 15, 2, 32, 5, "bf16"),
    (2, 192, 192, 6, 32, 96, "bf16"), (1, 64, 64, 2, 64, 32, "bf16"), (1, 8, 8, 4, 8, 2, "bf16"),
])
def test_partition_matches_oracle_bitwise(B, H, W, heads, d, w, dt):
    dev = device()
    print(f"partition B={B} H={H} W={W} heads={heads} d={d} w={w} {dt}", flush=True)
    wl = rib_synth.custom_workload(B, H, W, heads, d, w, 1, dt, seed=B * 7 + w)
    x = rib_synth.make_inputs(wl)["q_c"]
    xg = to_gpu(x, dev)
    xw = rib.window_partition(xg, w)
    ref_bits = oracle.window_partition(x.data, w)
    got_bits = xw.cpu().view(torch.int16 if dt == "bf16" else torch.int32).numpy()
    assert np.array_equal(got_bits.view(ref_bits.dtype), ref_bits)
    back = rib.window_unpartition(xw, B, H, W, w)
    assert torch.equal(back.view(torch.int16 if dt == "bf16" else torch.int32),
                       xg.view(torch.int16 if dt == "bf16" else torch.int32))


def test_partition_empty_batch():
    dev = device()
    x = torch.empty((0, 32, 32, 2, 32), dtype=torch.bfloat16, device=dev)
    assert rib.window_partition(x, 16).shape == (0, 2, 256, 32)

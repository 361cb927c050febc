"""GPU parity of the relative-position-bias (RPB) comparison kernel against the float64 oracle.

O = softmax(scale Q_c K_c^T + B) V with B gathered from a per-head (2w-1)^2 table. The kernel
stages the table in fp16 after multiplying it by log2(e) (the precision its interface states);
the N(0, 1) tables here are compared against the oracle on the float32 table as given, which
that rounding (at most 2^-9 in log2 units for |b| < 4) keeps well inside the bfloat16 bar. A
table with one entry of 60 is compared on its fp16 log2-unit image, because at that magnitude the
rounding alone moves the LSE by up to 0.02.
"""

import numpy as np
import pytest
import torch

import oracle
import rib_synth
import windowed_attention_implicit_amd as rib
from gpu_util import check, device, sample_units, to_f64, to_gpu

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def _run(wl, x, table, dev, scale=None):
    q, k, v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
    t = torch.from_numpy(table).to(dev)
    o, lse = rib.rpb_window_attn_fwd(q, k, v, t, wl.w, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _compare(wl, x, table, o, lse, scale=None, units=None, tag=""):
    ro, rl = oracle.rpb_window_attn_fwd(x["q_c"].f64(), x["k_c"].f64(), x["v"].f64(), table, wl.w, scale=scale,
                                        units=units)
    check(f"{tag} O", to_f64(o), ro, "bf16")
    lerr = np.nanmax(np.abs(to_f64(lse) - rl))
    print(f"{tag} LSE max-abs {lerr:.3e}", flush=True)
    assert lerr <= 2e-2


@pytest.mark.parametrize("shape", [
    # B, H, W, heads, w
    (1, 10, 15, 2, 5),      # N = 25: one partial tile
    (2, 14, 14, 1, 7),      # N = 49
    (1, 24, 24, 3, 12),     # N = 144: two tiles + a ragged 16
    (1, 32, 32, 2, 16),     # N = 256: whole tiles
    (1, 33, 33, 1, 33),     # N = 1089: 17 tiles + 1 key
    (1, 2, 2, 1, 2),        # N = 4, the smallest window
    (1, 40, 80, 2, 40),     # N = 1600, two windows per head
])
def test_rpb_small_shapes(shape):
    B, H, W, heads, w = shape
    dev = device()
    wl = rib_synth.custom_workload(B, H, W, heads, 32, w, 1, "bf16", seed=31 + w)
    x = rib_synth.make_inputs(wl)
    table = rib_synth.make_rpb_table(heads, w, seed=w)
    o, lse = _run(wl, x, table, dev)
    _compare(wl, x, table, o, lse, tag=wl.name)


def test_rpb_explicit_scale_and_negative_bias():
    dev = device()
    wl = rib_synth.custom_workload(1, 20, 20, 2, 32, 10, 1, "bf16", seed=5)
    x = rib_synth.make_inputs(wl)
    table = rib_synth.make_rpb_table(2, 10, seed=6) - 3.0   # every bias negative: the bound's maximum is < 0
    o, lse = _run(wl, x, table, dev, scale=0.37)
    _compare(wl, x, table, o, lse, scale=0.37, tag="scale 0.37, negative table")


def test_rpb_exact_pass_forced():
    """One table entry of 60 (seen only by query 0 with key N-1) makes the per-query bound overshoot
    by ~87 log2 units for every other query, so their row sums fall below 2^-60 and every workgroup
    takes the exact online-softmax pass."""
    dev = device()
    w = 9
    wl = rib_synth.custom_workload(1, 18, 18, 2, 32, w, 1, "bf16", seed=8)
    x = rib_synth.make_inputs(wl)
    table = rib_synth.make_rpb_table(2, w, seed=9)
    table[:, 0] = 60.0
    o, lse = _run(wl, x, table, dev)
    # the oracle on the fp16 log2-unit table the kernel uses
    t16 = (table.astype(np.float64) * LOG2E).astype(np.float16).astype(np.float64) / LOG2E
    _compare(wl, x, t16, o, lse, tag="exact pass")
    # query 0 of every window attends almost only to key N-1
    assert np.isfinite(to_f64(lse)).all()


def test_rpb_w96_workload_sampled():
    dev = device()
    wl = rib_synth.WORKLOADS["w96_map192x4_bf16"]
    x = rib_synth.make_inputs(wl)
    table = rib_synth.make_rpb_table(wl.heads, wl.w, seed=96)
    o, lse = _run(wl, x, table, dev)
    units = sample_units(wl, 3, seed=2)
    print(f"w96 RPB: units {units}", flush=True)
    _compare(wl, x, table, o, lse, units=units, tag="w96 RPB")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_rpb_deterministic_and_plan_reuse():
    dev = device()
    wl = rib_synth.custom_workload(1, 32, 32, 2, 32, 16, 1, "bf16", seed=12)
    x = rib_synth.make_inputs(wl)
    q, k, v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
    t = torch.from_numpy(rib_synth.make_rpb_table(2, 16, seed=13)).to(dev)
    plan = rib.RpbFwdPlan(q, k, v, t, wl.w)
    o1, l1 = (a.clone() for a in plan.run())
    o2, l2 = plan.run()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_rpb_zero_table_matches_rib_with_zero_positional_tokens():
    """With an all-zero table and scale 1/sqrt(d_c), RPB is plain attention; so is RIB with zero
    positional tokens and the same scale (a GPU-to-GPU cross-check of the two kernels, next to the
    oracle comparison of each)."""
    dev = device()
    wl = rib_synth.custom_workload(1, 24, 24, 2, 32, 12, 16, "bf16", seed=14)
    x = rib_synth.make_inputs(wl)
    q, k, v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
    t = torch.zeros((2, 23 * 23), dtype=torch.float32, device=dev)
    s = 1 / np.sqrt(32)
    o1, l1 = rib.rpb_window_attn_fwd(q, k, v, t, wl.w)
    zp = torch.zeros((wl.N, 16), dtype=torch.bfloat16, device=dev)
    o2, l2 = rib.window_attn_fwd(q, k, v, zp, zp, wl.w, scale=s)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
    assert (l1 - l2).abs().max().item() <= 2e-2

"""GPU parity of the CLA gate (G = sigmoid(PW_1x1(DW_3x3(X)))) and of the gated forward
(O' = O * G fused into the attention kernel's output stage) against the float64 oracle.

The bf16 gate rounds the depth-wise output and the point-wise weights to bf16 for the matrix
cores (the precision its interface states); G lies in (0, 1), so the bf16 bar applies as it is.
"""

import numpy as np
import pytest
import torch

import oracle
import rib_synth
import windowed_attention_implicit_amd as rib
from gpu_util import check, device, sample_units, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _weights(C, seed, dev):
    p = rib_synth.make_cla(C, seed)
    return p, {k: torch.from_numpy(v).to(dev) for k, v in p.items()}


@pytest.mark.parametrize("B,H,W,heads,dtype", [
    (2, 20, 37, 6, "bf16"),   # C = 192, a ragged last tile of 5 pixels per row
    (1, 5, 3, 1, "bf16"),     # C = 32, a map smaller than one tile
    (1, 64, 64, 8, "bf16"),   # C = 256, the largest supported
    (1, 9, 33, 3, "bf16"),    # C = 96
    (1, 1, 70, 4, "bf16"),    # C = 128, one row: both halo rows outside the map
    (3, 2, 31, 5, "bf16"),    # C = 160, two rows, W below one segment
    (1, 3, 1, 7, "bf16"),     # C = 224, a one-pixel-wide map
    (1, 12, 40, 2, "f32"),
    (2, 7, 7, 6, "f32"),
])
def test_cla_gate_parity(B, H, W, heads, dtype):
    dev = device()
    C = 32 * heads
    x = rib_synth.make_map(B, H, W, C, dtype, seed=H * W + C)
    p, t = _weights(C, seed=C + B, dev=dev)
    g = rib.cla_gate(to_gpu(x, dev), t["w_dw"], t["b_dw"], t["w_pw"], t["b_pw"], heads)
    torch.cuda.synchronize()
    ref = oracle.cla_gate(x.f64(), p["w_dw"], p["b_dw"], p["w_pw"], p["b_pw"])
    check(f"G {B}x{H}x{W}x{C} {dtype}", to_f64(g), ref, dtype)


def test_cla_gate_null_biases_and_repeat():
    dev = device()
    C = 64
    x = rib_synth.make_map(1, 16, 50, C, "bf16", seed=3)
    p, t = _weights(C, seed=4, dev=dev)
    xg = to_gpu(x, dev)
    g1 = rib.cla_gate(xg, t["w_dw"], None, t["w_pw"], None, 2)
    g2 = rib.cla_gate(xg, t["w_dw"], None, t["w_pw"], None, 2)
    torch.cuda.synchronize()
    assert torch.equal(g1, g2)
    check("G no biases", to_f64(g1), oracle.cla_gate(x.f64(), p["w_dw"], None, p["w_pw"], None), "bf16")


def _strip_rows(B, H, W, C, cus):
    """Rows per strip the bf16 gate's launcher picks: 64-pixel segments up to C = 192 (32 above), and
    the fewest rows whose strips fit one round of one workgroup per CU."""
    seg = 64 if C <= 192 else 32
    cols = B * ((W + seg - 1) // seg)
    rows = max(1, (cols * H + cus - 1) // cus)
    while rows < H and cols * ((H + rows - 1) // rows) > cus:
        rows += 1
    return rows


@pytest.mark.parametrize("B,H,W,heads", [
    (2, 162, 130, 1),   # C = 32: 2 waves, 64-pixel segments; strips of 4 rows, the last of 2
    (2, 97, 150, 3),    # C = 96: 6 waves; strips of 3 rows, the last of 1; a 22-pixel last segment
    (2, 100, 100, 7),   # C = 224: 7 waves, 32-pixel segments
    (2, 128, 96, 8),    # C = 256: 8 waves, the point-wise weights in eight rounds
])
def test_cla_gate_parity_multirow_strips(B, H, W, heads):
    """Maps on which every workgroup walks a strip of three or more rows, so the waits that count
    memory operations still in flight (the fourth halo row after the prologue, two row stores per
    step after that) run for every wave count and segment width, not only at C = 192."""
    dev = device()
    C = 32 * heads
    rows = _strip_rows(B, H, W, C, torch.cuda.get_device_properties(dev).multi_processor_count)
    print(f"CLA {B}x{H}x{W}x{C}: strips of {rows} rows", flush=True)
    assert rows >= 3
    x = rib_synth.make_map(B, H, W, C, "bf16", seed=H + W + C)
    p, t = _weights(C, seed=C + 7, dev=dev)
    g = rib.cla_gate(to_gpu(x, dev), t["w_dw"], t["b_dw"], t["w_pw"], t["b_pw"], heads)
    torch.cuda.synchronize()
    ref = oracle.cla_gate(x.f64(), p["w_dw"], p["b_dw"], p["w_pw"], p["b_pw"])
    check(f"G {B}x{H}x{W}x{C} strips of {rows}", to_f64(g), ref, "bf16")


def test_cla_gate_headline_map_full():
    """The gate of the 96x96-window workload's map (batch 4, 192 x 192, C = 192), every value."""
    dev = device()
    wl = rib_synth.HEADLINE
    C = wl.heads * wl.d_c
    x = rib_synth.make_map(wl.B, wl.H, wl.W, C, "bf16", seed=192)
    p, t = _weights(C, seed=193, dev=dev)
    g = rib.cla_gate(to_gpu(x, dev), t["w_dw"], t["b_dw"], t["w_pw"], t["b_pw"], wl.heads)
    torch.cuda.synchronize()
    check("G headline map", to_f64(g), oracle.cla_gate(x.f64(), p["w_dw"], p["b_dw"], p["w_pw"], p["b_pw"]), "bf16")


def _gated_case(wl, dev, units=None, tag=""):
    C = wl.heads * wl.d_c
    x = rib_synth.make_inputs(wl)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    xm = rib_synth.make_map(wl.B, wl.H, wl.W, C, wl.dtype, seed=wl.seed + 100)
    p, t = _weights(C, seed=wl.seed + 101, dev=dev)
    q, k, v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
    w1, w2 = torch.from_numpy(x["w1"]).to(dev), torch.from_numpy(x["w2"]).to(dev)
    qp, kp = rib.posgen(wl.w, w1, None, w2, None, wl.r, n_freq=wl.n_freq, out_dtype=dt)
    g = rib.cla_gate(to_gpu(xm, dev), t["w_dw"], t["b_dw"], t["w_pw"], t["b_pw"], wl.heads)
    og, lg = rib.window_attn_fwd_gated(q, k, v, qp, kp, g, wl.w)
    o, lse = rib.window_attn_fwd(q, k, v, qp, kp, wl.w)
    torch.cuda.synchronize()
    # the LSE is that of the ungated attention, bit for bit
    assert torch.equal(lg, lse)
    # fused gating = gating the ungated output (one extra bf16 rounding apart)
    gm = g.reshape(o.shape).float()
    tol = 1e-6 if wl.dtype == "f32" else 2 ** -7
    assert ((og.float() - o.float() * gm).abs() <= tol * (o.float() * gm).abs() + 1e-6).all()
    # against the oracle: O' = O * G with the oracle's own O and G
    rqp, rkp = oracle.posgen(wl.w, wl.n_freq, x["w1"], None, x["w2"], None, wl.r)
    ro, rl = oracle.rib_window_attn_fwd(x["q_c"].f64(), x["k_c"].f64(), x["v"].f64(), rqp, rkp, wl.w, units=units)
    rg = oracle.cla_gate(xm.f64(), p["w_dw"], p["b_dw"], p["w_pw"], p["b_pw"])
    check(f"{tag} O'", to_f64(og), oracle.cla_apply(ro, rg), wl.dtype)


@pytest.mark.parametrize("shape", [
    (1, 24, 24, 3, 32, 12, 16, "bf16"),
    (2, 14, 28, 2, 32, 7, 5, "bf16"),
    (1, 10, 15, 2, 32, 5, 3, "f32"),
    (1, 16, 16, 2, 64, 8, 16, "bf16"),   # d_c = 64: the one-thread-per-query kernel applies the gate
    (1, 48, 48, 2, 32, 48, 16, "bf16"),  # N = 2304: every item in key ranges, the combine applies the gate
    (1, 32, 48, 2, 32, 16, 16, "bf16"),  # w divides 64: K_c and V read in their maps
])
def test_gated_forward_small(shape):
    dev = device()
    wl = rib_synth.custom_workload(*shape, seed=sum(shape[:6]))
    _gated_case(wl, dev, tag=wl.name)


def test_gated_forward_w96_sampled():
    dev = device()
    wl = rib_synth.HEADLINE
    # the first and last units plus two of the split tail (the combine applies the gate there)
    units = sample_units(wl, 2, seed=5, include=(10, 11))
    print(f"gated w96: units {units}", flush=True)
    _gated_case(wl, dev, units=units, tag="gated w96")

"""Pins of the oracle's position-token generation against facts fixed outside it.

Closed forms (hand-derived fixtures), exact rational arithmetic, library
routines (numpy.linspace, torch.nn.functional) and invariants stated on the
pages: the bias is low rank, depends only on the window geometry and its
parameter count does not depend on the window size.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import rib_synth


# ---------------------------------------------------------------- coordinates

@pytest.mark.parametrize("w", [2, 3, 4, 5, 16, 32, 64, 96])
def test_coords_match_linspace(w):
    """Reading R1: linspace(-1, 1, w) with both endpoints (library routine)."""
    n, c = oracle.window_coords(w)
    np.testing.assert_allclose(c, np.linspace(-1.0, 1.0, w), rtol=0, atol=1e-15)
    assert c[0] == -1.0 and c[-1] == 1.0
    np.testing.assert_array_equal(c[::-1], -c)           # c_{w-1-i} = -c_i
    assert all(isinstance(v, int) for v in n)
    assert [Fraction(v, w - 1) for v in n] == [Fraction(2 * i - (w - 1), w - 1) for i in range(w)]


def test_coords_reject_degenerate():
    with pytest.raises(ValueError):
        oracle.window_coords(1)


# ---------------------------------------------------------------- Fourier map

def _parse_golden(path):
    sym = {"s": math.sqrt(3) / 2, "h": 0.5}
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, vals = line.split(":")
            w, F, t = (int(x) for x in head.split())
            out = []
            for tok in vals.split():
                neg = tok.startswith("-")
                base = tok[1:] if neg else tok
                v = sym[base] if base in sym else float(base)
                out.append(-v if neg else v)
            rows.append((w, F, t, np.array(out)))
    return rows


def test_fourier_hand_derived(golden_dir):
    """Hand-derived single-token features (tests/golden/fourier_hand.txt)."""
    rows = _parse_golden(os.path.join(golden_dir, "fourier_hand.txt"))
    assert len(rows) >= 9
    for w, F, t, expect in rows:
        got = oracle.fourier_features(w, F)[t]
        np.testing.assert_allclose(got, expect, rtol=0, atol=1e-14, err_msg=f"w={w} token={t}")


def _exact_feature(n_num, den, k):
    """sin/cos(2^k pi n/den) with the phase reduced exactly (Fraction mod 2)."""
    ph = (Fraction(n_num, den) * (2 ** k)) % 2
    a = math.pi * float(ph)
    return math.sin(a), math.cos(a)


@pytest.mark.parametrize("w", [7, 16, 96])
def test_fourier_matches_exact_phase_reduction(w):
    """float64 evaluation of the definition agrees with exact rational phase reduction."""
    F = 16
    feats = oracle.fourier_features(w, F)
    n, _ = oracle.window_coords(w)
    for t in [0, 1, w - 1, w, w * w // 2 + 3, w * w - 1]:
        iy, ix = divmod(t, w)
        for k in range(F):
            sx, cx = _exact_feature(n[ix], w - 1, k)
            sy, cy = _exact_feature(n[iy], w - 1, k)
            np.testing.assert_allclose(
                [feats[t, k], feats[t, F + k], feats[t, 2 * F + k], feats[t, 3 * F + k]],
                [sx, cx, sy, cy], rtol=0, atol=1e-9)


@pytest.mark.parametrize("w", [4, 16, 96])
def test_fourier_unit_circle_and_symmetry(w):
    F = 16
    f = oracle.fourier_features(w, F)
    N = w * w
    sx, cx, sy, cy = f[:, :F], f[:, F:2 * F], f[:, 2 * F:3 * F], f[:, 3 * F:]
    np.testing.assert_allclose(sx ** 2 + cx ** 2, 1.0, atol=1e-12)
    np.testing.assert_allclose(sy ** 2 + cy ** 2, 1.0, atol=1e-12)
    # mirror x -> -x: token (iy, ix) <-> (iy, w-1-ix); sin odd, cos even
    mirror = np.array([(t // w) * w + (w - 1 - t % w) for t in range(N)])
    np.testing.assert_allclose(sx[mirror], -sx, atol=1e-9)
    np.testing.assert_allclose(cx[mirror], cx, atol=1e-9)
    # transposing the window swaps the x and y blocks
    transpose = np.array([(t % w) * w + t // w for t in range(N)])
    np.testing.assert_allclose(f[transpose][:, :2 * F], f[:, 2 * F:], atol=0)


@pytest.mark.parametrize("m", [4, 5, 6])
def test_fourier_periodicity_power_of_two_windows(m):
    """For w = 2^m, w - 1 is odd and 2^m = 1 mod (w-1): column k+m repeats column k
    for k >= 1, and column m is column 0 shifted by pi (negated)."""
    w, F = 2 ** m, 16
    f = oracle.fourier_features(w, F)
    for blk in range(4):
        cols = f[:, blk * F:(blk + 1) * F]
        for k in range(1, F - m):
            np.testing.assert_allclose(cols[:, k + m], cols[:, k], atol=1e-9)
        np.testing.assert_allclose(cols[:, m], -cols[:, 0], atol=1e-9)


def test_fourier_no_repetition_w96():
    f = oracle.fourier_features(96, 16)
    for blk in range(4):
        cols = f[:, blk * 16:(blk + 1) * 16]
        for a in range(16):
            for b in range(a + 1, 16):
                assert np.abs(cols[:, a] - cols[:, b]).max() > 1e-3


# ---------------------------------------------------------------- MLP

def test_gelu_matches_torch():
    z = np.linspace(-6, 6, 1001)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu(z), ref, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("w,r", [(16, 8), (32, 16), (5, 3)])
def test_posgen_matches_torch_mlp(w, r):
    """Q_p, K_p = split(Linear(GELU(Linear(phi)))) via torch in float64 (library route)."""
    rng = np.random.default_rng(w * 100 + r)
    F, Hd = 16, 64
    w1 = rng.standard_normal((Hd, 4 * F)) * 0.3
    b1 = rng.standard_normal(Hd) * 0.1
    w2 = rng.standard_normal((2 * r, Hd)) * 0.3
    b2 = rng.standard_normal(2 * r) * 0.1
    qp, kp = oracle.posgen(w, F, w1, b1, w2, b2, r)
    phi = torch.from_numpy(oracle.fourier_features(w, F))
    h = torch.nn.functional.gelu(torch.nn.functional.linear(phi, torch.from_numpy(w1), torch.from_numpy(b1)))
    out = torch.nn.functional.linear(h, torch.from_numpy(w2), torch.from_numpy(b2)).numpy()
    np.testing.assert_allclose(qp, out[:, :r], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(kp, out[:, r:], rtol=1e-13, atol=1e-14)


def test_posgen_special_cases():
    F, Hd, r, w = 16, 64, 8, 16
    rng = np.random.default_rng(3)
    w1 = rng.standard_normal((Hd, 4 * F))
    qp, kp = oracle.posgen(w, F, w1, None, np.zeros((2 * r, Hd)), None, r)
    assert not qp.any() and not kp.any()
    b2 = np.arange(2 * r, dtype=np.float64)
    qp, kp = oracle.posgen(w, F, w1, None, np.zeros((2 * r, Hd)), b2, r)
    np.testing.assert_array_equal(qp, np.broadcast_to(b2[:r], qp.shape))
    np.testing.assert_array_equal(kp, np.broadcast_to(b2[r:], kp.shape))
    with pytest.raises(ValueError):
        oracle.posgen(w, F, w1, None, np.zeros((r, Hd)), None, r)


# ---------------------------------------------------------------- bias invariants

@pytest.mark.parametrize("w,r", [(16, 8), (32, 16)])
def test_bias_rank_at_most_r(w, r):
    """The bias Q_p K_p^T has rank <= r (rank-factorized, low-rank bias)."""
    wl = rib_synth.custom_workload(1, w, w, 1, 32, w, r, seed=7)
    x = rib_synth.make_inputs(wl)
    qp, kp = oracle.posgen(w, 16, x["w1"], x["b1"], x["w2"], x["b2"], r)
    s = np.linalg.svd(qp @ kp.T, compute_uv=False)
    assert s[0] > 0
    assert np.all(s[r:] <= 1e-12 * s[0])


def test_bias_identical_for_every_window():
    """Coordinates normalized inside each window give one bias per window size:
    recomputing them from absolute pixel positions of each window reproduces them."""
    w, H, W = 8, 24, 16
    n_ref, c_ref = oracle.window_coords(w)
    for wy in range(H // w):
        for wx in range(W // w):
            ys = np.arange(wy * w, (wy + 1) * w)
            xs = np.arange(wx * w, (wx + 1) * w)
            # numerators of the in-window coordinate, from absolute pixel rows / columns
            assert (2 * (ys - ys[0]) - (w - 1)).tolist() == n_ref
            assert (2 * (xs - xs[0]) - (w - 1)).tolist() == n_ref
            np.testing.assert_allclose(2 * (xs - xs[0]) / (w - 1) - 1, c_ref, atol=1e-15)


def test_param_count_is_what_posgen_uses_at_every_window():
    """[EN §2.A "Advantages"]: the bias parameters do not grow with the window. Every entry of
    W1, b1, W2, b2 is perturbed in turn and counted when it moves posgen's output; the count is
    the same at every window size and equals mlp_param_count (a dropped bias, an unused feature
    column or a rank mix-up would change it). w >= 4 keeps every sin feature nonzero (at w = 2
    and 3 every coordinate is a multiple of pi/2 ... pi, where sin(2^k pi x) vanishes)."""
    F, hid, r = 3, 5, 2
    rng = np.random.default_rng(31)
    params = {"w1": rng.normal(0, 0.5, (hid, 4 * F)), "b1": rng.normal(0, 0.5, hid),
              "w2": rng.normal(0, 0.5, (2 * r, hid)), "b2": rng.normal(0, 0.5, 2 * r)}
    counts = {}
    for w in (4, 7, 16):
        base = np.concatenate(oracle.posgen(w, F, params["w1"], params["b1"], params["w2"], params["b2"], r), axis=1)
        used = 0
        for name, arr in params.items():
            for idx in np.ndindex(arr.shape):
                pert = {k: v.copy() for k, v in params.items()}
                pert[name][idx] += 1e-3
                out = np.concatenate(oracle.posgen(w, F, pert["w1"], pert["b1"], pert["w2"], pert["b2"], r), axis=1)
                used += int(np.abs(out - base).max() > 1e-9)
        counts[w] = used
    assert set(counts.values()) == {oracle.mlp_param_count(F, hid, r)}, counts
    assert oracle.mlp_param_count(F, hid, r) == sum(a.size for a in params.values())

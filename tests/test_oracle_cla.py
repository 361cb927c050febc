"""Pins of the oracle's CLA gate: G = sigmoid(PW_1x1(DW_3x3(X))), O' = O * G.

The gate is checked against torch's conv2d (grouped 3x3, then 1x1) in float64, against a
brute-force per-pixel sum with explicit bounds checks, against closed forms (identity taps,
zero point-wise weights, a constant map whose border sums count the taps inside the map), for
translation equivariance away from the border, and the channel mapping of O' = O * G by a
one-hot gate.
"""

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, std=1.0):
    return std * np.random.default_rng(seed).standard_normal(shape)


def _params(C, seed):
    return (_rand((C, 3, 3), seed, 0.5), _rand(C, seed + 1, 0.2), _rand((C, C), seed + 2, 0.3),
            _rand(C, seed + 3, 0.2))


@pytest.mark.parametrize("B,H,W,C", [(2, 7, 9, 12), (1, 1, 5, 3), (1, 4, 4, 1)])
def test_cla_matches_torch_conv2d(B, H, W, C):
    x = _rand((B, H, W, C), 10 + C)
    w_dw, b_dw, w_pw, b_pw = _params(C, 20 + C)
    g = oracle.cla_gate(x, w_dw, b_dw, w_pw, b_pw)
    xt = torch.tensor(x).permute(0, 3, 1, 2)
    d = torch.nn.functional.conv2d(xt, torch.tensor(w_dw)[:, None], torch.tensor(b_dw), padding=1, groups=C)
    z = torch.nn.functional.conv2d(d, torch.tensor(w_pw)[:, :, None, None], torch.tensor(b_pw))
    ref = torch.sigmoid(z).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(g, ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.cla_depthwise3x3(x, w_dw, b_dw), d.permute(0, 2, 3, 1).numpy(),
                               rtol=0, atol=1e-13)


def test_cla_brute_force_pixels():
    B, H, W, C = 1, 3, 4, 3
    x = _rand((B, H, W, C), 1)
    w_dw, b_dw, w_pw, b_pw = _params(C, 2)
    g = oracle.cla_gate(x, w_dw, b_dw, w_pw, b_pw)
    for y in range(H):
        for xx in range(W):
            d = np.zeros(C)
            for c in range(C):
                acc = b_dw[c]
                for ky in range(3):
                    for kx in range(3):
                        yy, xs = y + ky - 1, xx + kx - 1
                        if 0 <= yy < H and 0 <= xs < W:
                            acc += w_dw[c, ky, kx] * x[0, yy, xs, c]
                d[c] = acc
            for co in range(C):
                z = b_pw[co] + sum(w_pw[co, ci] * d[ci] for ci in range(C))
                assert abs(g[0, y, xx, co] - 1 / (1 + np.exp(-z))) < 1e-14


def test_cla_closed_forms():
    B, H, W, C = 2, 5, 6, 4
    x = _rand((B, H, W, C), 3, 2.0)
    ident = np.zeros((C, 3, 3))
    ident[:, 1, 1] = 1.0
    # identity taps, identity point-wise, no biases: G = sigmoid(X)
    g = oracle.cla_gate(x, ident, None, np.eye(C), None)
    np.testing.assert_allclose(g, 1 / (1 + np.exp(-x)), rtol=0, atol=1e-15)
    # zero point-wise weights: G = sigmoid(b_pw) everywhere; zero bias too: exactly 1/2
    b_pw = np.array([-2.0, 0.0, 1.0, 3.0])
    g = oracle.cla_gate(x, _rand((C, 3, 3), 4), _rand(C, 5), np.zeros((C, C)), b_pw)
    np.testing.assert_allclose(g, np.broadcast_to(1 / (1 + np.exp(-b_pw)), g.shape), rtol=0, atol=1e-15)
    assert np.all(g[..., 1] == 0.5)


def test_cla_constant_map_border_counts():
    """X = 1, all nine taps of channel c equal to c + 1: D = (c + 1) times the number of taps inside
    the map, i.e. 9 inside, 6 on an edge, 4 in a corner (zero padding, not wrap-around)."""
    H, W, C = 4, 5, 3
    w_dw = np.ones((C, 3, 3)) * (np.arange(C) + 1.0)[:, None, None]
    d = oracle.cla_depthwise3x3(np.ones((1, H, W, C)), w_dw)
    count = np.full((H, W), 9.0)
    count[0, :] = count[-1, :] = 6.0
    count[:, 0] = count[:, -1] = 6.0
    for y, x in ((0, 0), (0, W - 1), (H - 1, 0), (H - 1, W - 1)):
        count[y, x] = 4.0
    np.testing.assert_array_equal(d[0], count[:, :, None] * (np.arange(C) + 1.0))


def test_cla_translation_equivariance():
    H, W, C = 9, 10, 3
    x = _rand((1, H, W, C), 6)
    w_dw, b_dw, w_pw, b_pw = _params(C, 7)
    xs = np.zeros_like(x)
    xs[:, 1:, 2:, :] = x[:, :-1, :-2, :]           # shift down 1, right 2, zero fill
    g = oracle.cla_gate(x, w_dw, b_dw, w_pw, b_pw)
    gs = oracle.cla_gate(xs, w_dw, b_dw, w_pw, b_pw)
    # away from every border (of both maps) the shifted gate is the gate shifted
    np.testing.assert_allclose(gs[:, 2:H - 1, 3:W - 1, :], g[:, 1:H - 2, 1:W - 3, :], rtol=0, atol=1e-14)


def test_cla_apply_channel_mapping():
    B, H, W, heads, d_c = 1, 2, 3, 3, 4
    o = _rand((B, H, W, heads, d_c), 8)
    for head, j in ((0, 0), (1, 2), (2, 3)):
        g = np.zeros((B, H, W, heads * d_c))
        g[..., head * d_c + j] = 1.0
        out = oracle.cla_apply(o, g)
        expect = np.zeros_like(o)
        expect[..., head, j] = o[..., head, j]
        np.testing.assert_array_equal(out, expect)
    g = _rand((B, H, W, heads * d_c), 9)
    np.testing.assert_allclose(oracle.cla_apply(o, g)[0, 1, 2], o[0, 1, 2] * g[0, 1, 2].reshape(heads, d_c))

"""Pins of the oracle's position-MLP backward (weight gradients from dQ_p, dK_p).

The derivative is checked against facts fixed outside the oracle's chain rule:
central finite differences of the scalar loss sum(dQ_p * Q_p) + sum(dK_p * K_p)
in float64, torch autograd (float64) on an independently built MLP, the
textbook values of the normal CDF and density inside GELU', and the Q-first /
K-second split of the MLP outputs.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _mlp(F, hidden, r, seed, scale=0.5):
    g = np.random.default_rng(seed)
    w1 = g.normal(0.0, scale, (hidden, 4 * F))
    b1 = g.normal(0.0, scale, hidden)
    w2 = g.normal(0.0, scale, (2 * r, hidden))
    b2 = g.normal(0.0, scale, 2 * r)
    return w1, b1, w2, b2


def _loss(w, F, w1, b1, w2, b2, r, dq, dk):
    qp, kp = oracle.posgen(w, F, w1, b1, w2, b2, r)
    return float((dq * qp).sum() + (dk * kp).sum())


def test_gelu_grad_closed_forms():
    """GELU'(z) = Phi(z) + z phi(z): 1/2 at 0, the textbook Phi(1) + phi(1) at 1,
    -> 1 and -> 0 far out, and Phi(-z) + Phi(z) = 1 makes GELU'(z) + GELU'(-z) = 1."""
    g = oracle.gelu_grad
    assert g(0.0) == 0.5
    # Phi(1) = 0.8413447460685429, phi(1) = 0.24197072451914337 (standard normal tables)
    assert abs(float(g(1.0)) - (0.8413447460685429 + 0.24197072451914337)) < 1e-15
    assert abs(float(g(12.0)) - 1.0) < 1e-15 and abs(float(g(-12.0))) < 1e-15
    z = np.linspace(-6, 6, 49)
    np.testing.assert_allclose(g(z) + g(-z), 1.0, rtol=0, atol=1e-14)


def test_gelu_grad_matches_difference_quotient():
    z = np.linspace(-5, 5, 81)
    h = 1e-5
    fd = (oracle.gelu(z + h) - oracle.gelu(z - h)) / (2 * h)
    np.testing.assert_allclose(oracle.gelu_grad(z), fd, rtol=0, atol=1e-9)


@pytest.mark.parametrize("w,F,hidden,r", [(3, 2, 5, 2), (4, 3, 4, 1)])
def test_posgen_bwd_finite_differences(w, F, hidden, r):
    """Every weight and bias entry against a central difference of the scalar loss."""
    w1, b1, w2, b2 = _mlp(F, hidden, r, seed=11 + w)
    g = np.random.default_rng(5 + w)
    dq, dk = g.normal(size=(w * w, r)), g.normal(size=(w * w, r))
    grads = oracle.posgen_bwd(w, F, w1, b1, w2, b2, r, dq, dk)
    params = [w1, b1, w2, b2]
    h = 1e-6
    for pi, (p, gr) in enumerate(zip(params, grads)):
        assert gr.shape == p.shape
        fd = np.zeros_like(p)
        for idx in np.ndindex(p.shape):
            up = [q.copy() for q in params]
            dn = [q.copy() for q in params]
            up[pi][idx] += h
            dn[pi][idx] -= h
            fd[idx] = (_loss(w, F, *up, r, dq, dk) - _loss(w, F, *dn, r, dq, dk)) / (2 * h)
        np.testing.assert_allclose(gr, fd, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("w,F,hidden,r", [(8, 16, 64, 8), (5, 4, 24, 3)])
def test_posgen_bwd_matches_torch_autograd(w, F, hidden, r):
    """torch autograd (float64) through nn.functional.linear / gelu(approximate='none')."""
    w1, b1, w2, b2 = _mlp(F, hidden, r, seed=3 * w + r)
    g = np.random.default_rng(w + r)
    dq, dk = g.normal(size=(w * w, r)), g.normal(size=(w * w, r))
    phi = torch.tensor(oracle.fourier_features(w, F))      # constant: no parameters
    tw = [torch.tensor(a, requires_grad=True) for a in (w1, b1, w2, b2)]
    z = torch.nn.functional.linear(phi, tw[0], tw[1])
    out = torch.nn.functional.linear(torch.nn.functional.gelu(z, approximate="none"), tw[2], tw[3])
    loss = (out[:, :r] * torch.tensor(dq)).sum() + (out[:, r:] * torch.tensor(dk)).sum()
    loss.backward()
    ours = oracle.posgen_bwd(w, F, w1, b1, w2, b2, r, dq, dk)
    for mine, t in zip(ours, tw):
        np.testing.assert_allclose(mine, t.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_posgen_bwd_split_and_linearity():
    """Q_p is the first r outputs (R6): a zero dK_p leaves the K rows of dW2 and
    db2 at zero; exchanging the roles of the two halves exchanges the dW2 / db2
    row blocks and leaves dW1, db1 unchanged; the map is linear in (dQ_p, dK_p)."""
    w, F, hidden, r = 6, 4, 16, 3
    w1, b1, w2, b2 = _mlp(F, hidden, r, seed=21)
    g = np.random.default_rng(22)
    dq, dk = g.normal(size=(w * w, r)), g.normal(size=(w * w, r))
    dw1, db1, dw2, db2 = oracle.posgen_bwd(w, F, w1, b1, w2, b2, r, dq, np.zeros_like(dk))
    assert np.all(dw2[r:] == 0) and np.all(db2[r:] == 0)
    a = oracle.posgen_bwd(w, F, w1, b1, w2, b2, r, dq, dk)
    sw2 = np.concatenate([w2[r:], w2[:r]])
    sb2 = np.concatenate([b2[r:], b2[:r]])
    b = oracle.posgen_bwd(w, F, w1, b1, sw2, sb2, r, dk, dq)
    np.testing.assert_allclose(b[0], a[0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(b[1], a[1], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(b[2], np.concatenate([a[2][r:], a[2][:r]]), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(b[3], np.concatenate([a[3][r:], a[3][:r]]), rtol=1e-13, atol=1e-13)
    c = oracle.posgen_bwd(w, F, w1, b1, w2, b2, r, 2.0 * dq - dk, dk + 0.5 * dq)
    dq2, dk2 = 2.0 * dq, 0.5 * dq
    p1 = oracle.posgen_bwd(w, F, w1, b1, w2, b2, r, dq2, dk2)
    p2 = oracle.posgen_bwd(w, F, w1, b1, w2, b2, r, -dk, dk)
    for x, y, z in zip(c, p1, p2):
        np.testing.assert_allclose(x, y + z, rtol=1e-12, atol=1e-12)


def test_posgen_bwd_zero_first_layer():
    """W1 = 0, b1 = 0: z = 0, h = GELU(0) = 0 and GELU'(0) = 1/2, so dW2 = 0,
    db2 = column sums of d_out, dW1 = (d_out W2 / 2)^T phi, db1 = sum of d_out W2 / 2."""
    w, F, hidden, r = 4, 2, 6, 2
    _, _, w2, b2 = _mlp(F, hidden, r, seed=31)
    g = np.random.default_rng(32)
    dq, dk = g.normal(size=(w * w, r)), g.normal(size=(w * w, r))
    dw1, db1, dw2, db2 = oracle.posgen_bwd(w, F, np.zeros((hidden, 4 * F)), None, w2, b2, r, dq, dk)
    d_out = np.hstack([dq, dk])
    assert np.all(dw2 == 0)
    np.testing.assert_allclose(db2, d_out.sum(0), rtol=0, atol=1e-13)
    phi = oracle.fourier_features(w, F)
    np.testing.assert_allclose(dw1, 0.5 * (d_out @ w2).T @ phi, rtol=0, atol=1e-12)
    np.testing.assert_allclose(db1, 0.5 * (d_out @ w2).sum(0), rtol=0, atol=1e-12)


def test_posgen_bwd_rejects_bad_shapes():
    w1, b1, w2, b2 = _mlp(2, 4, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.posgen_bwd(3, 2, w1, b1, w2, b2, 2, np.zeros((9, 3)), np.zeros((9, 2)))
    with pytest.raises(ValueError):
        oracle.posgen_bwd(3, 2, w1.T, b1, w2, b2, 2, np.zeros((9, 2)), np.zeros((9, 2)))

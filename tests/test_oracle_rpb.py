"""Pins of the oracle's RPB comparison path (S = scale Q_c K_c^T + B, B from a relative-position table).

The bias layout is checked by brute force over explicit coordinates, the attention against
torch's scaled_dot_product_attention with the bias as an additive mask, an all-zero table against
plain attention, and a table linear in (dy, dx) against RIB attention with explicit rank-3
positional tokens (which fixes the index convention: sign of the differences, rows vs columns).
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("w", [2, 3, 5])
def test_rpb_bias_brute_force(w):
    table = _rand((2 * w - 1) ** 2, w)
    B = oracle.rpb_bias(w, table)
    for i in range(w * w):
        yi, xi = divmod(i, w)
        for j in range(w * w):
            yj, xj = divmod(j, w)
            dy, dx = yi - yj, xi - xj
            assert B[i, j] == table[(dy + w - 1) * (2 * w - 1) + (dx + w - 1)]
    # translation structure: B[i, j] depends only on the displacement
    assert np.all(np.diag(B) == table[(w - 1) * (2 * w - 1) + (w - 1)])


def test_rpb_matches_torch_sdpa_with_additive_mask():
    w, d = 6, 32
    N = w * w
    qc, kc, v = _rand((N, d), 1), _rand((N, d), 2), _rand((N, d), 3)
    table = _rand((2 * w - 1) ** 2, 4)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.rpb_attention_window_fwd(qc, kc, v, oracle.rpb_bias(w, table), scale)
    t = lambda a: torch.tensor(a)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(qc), t(kc), t(v), attn_mask=t(oracle.rpb_bias(w, table)),
                                                            scale=scale)[0, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    S = scale * qc @ kc.T + oracle.rpb_bias(w, table)
    np.testing.assert_allclose(lse, np.log(np.exp(S).sum(1)), rtol=1e-12, atol=1e-12)


def test_rpb_zero_table_is_plain_attention():
    w, d = 5, 16
    N = w * w
    qc, kc, v = _rand((N, d), 5), _rand((N, d), 6), _rand((N, d), 7)
    o, _ = oracle.rpb_attention_window_fwd(qc, kc, v, oracle.rpb_bias(w, np.zeros((2 * w - 1) ** 2)), 0.3)
    t = lambda a: torch.tensor(a)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(qc), t(kc), t(v), scale=0.3)[0, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_rpb_linear_table_equals_rib_with_rank3_tokens():
    """table[dy, dx] = a dy + b dx + c gives B_ij = a (y_i - y_j) + b (x_i - x_j) + c, which is the RIB
    bias Q_p K_p^T of Q_p = [a y_i, b x_i, 1], K_p = [1, 1, -(a y_j + b x_j)] plus the constant c
    (softmax-invariant; it shifts the LSE by c). RIB scales the bias with the content (R8), so its
    positional query is divided by the scale."""
    w, d = 4, 8
    N = w * w
    a, b, c = 0.7, -0.3, 0.25
    dy, dx = np.meshgrid(np.arange(-(w - 1), w), np.arange(-(w - 1), w), indexing="ij")
    table = (a * dy + b * dx + c).reshape(-1)
    qc, kc, v = _rand((N, d), 8), _rand((N, d), 9), _rand((N, d), 10)
    scale = 0.4
    o_rpb, lse_rpb = oracle.rpb_attention_window_fwd(qc, kc, v, oracle.rpb_bias(w, table), scale)
    t = np.arange(N)
    y, x = t // w, t % w
    qp = np.stack([a * y, b * x, np.ones(N)], 1) / scale
    kp = np.stack([np.ones(N), np.ones(N), -(a * y + b * x)], 1)
    o_rib, lse_rib, _ = oracle.attention_window_fwd(qc, kc, v, qp, kp, scale)
    np.testing.assert_allclose(o_rpb, o_rib, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_rpb, lse_rib + c, rtol=0, atol=1e-12)


def test_rpb_map_level_windows_and_heads():
    """Every (batch, window, head) unit uses its head's table; units are independent windows."""
    B, H, W, heads, d, w = 1, 6, 9, 2, 4, 3
    g = np.random.default_rng(11)
    q, k, v = (g.standard_normal((B, H, W, heads, d)) for _ in range(3))
    table = g.standard_normal((heads, (2 * w - 1) ** 2))
    O, L = oracle.rpb_window_attn_fwd(q, k, v, table, w)
    for (wy, wx, h) in ((0, 0, 0), (1, 2, 1)):
        sl = (0, slice(wy * w, (wy + 1) * w), slice(wx * w, (wx + 1) * w), h)
        o, lse = oracle.rpb_attention_window_fwd(q[sl].reshape(-1, d), k[sl].reshape(-1, d), v[sl].reshape(-1, d),
                                                 oracle.rpb_bias(w, table[h]), 1 / math.sqrt(d))
        np.testing.assert_allclose(O[sl].reshape(-1, d), o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[sl].reshape(-1), lse, rtol=0, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.rpb_window_attn_fwd(q, k, v, table[:, :-1], w)


def test_rpb_parameter_count_grows_with_window():
    """The table holds (2w - 1)^2 entries per head, O(w^2) (unlike the RIB MLP)."""
    assert [(2 * w - 1) ** 2 for w in (16, 32, 64, 96)] == [961, 3969, 16129, 36481]
    with pytest.raises(ValueError):
        oracle.rpb_bias(4, np.zeros(48))

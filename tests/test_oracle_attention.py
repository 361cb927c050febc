"""Pins of the oracle's window partition and RIB attention (forward and backward).

Every check compares the oracle with something other than itself: the
hand-worked example in tests/golden/, the score identity stated on the pages,
torch's scaled_dot_product_attention and autograd in float64 (library
routines), brute-force central finite differences, and closed-form
invariants of softmax attention.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _rand(rng, *shape, s=1.0):
    return s * rng.standard_normal(shape)


# ---------------------------------------------------------------- partition

@pytest.mark.parametrize("B,H,W,heads,d,w", [(2, 6, 9, 2, 3, 3), (1, 8, 8, 1, 1, 4), (1, 4, 4, 3, 2, 2)])
def test_partition_bijection_brute_force(B, H, W, heads, d, w):
    x = np.arange(B * H * W * heads * d).reshape(B, H, W, heads, d)
    xw = oracle.window_partition(x, w)
    assert xw.shape == (B * (H // w) * (W // w), heads, w * w, d)
    assert sorted(xw.ravel().tolist()) == list(range(x.size))       # every element exactly once
    np.testing.assert_array_equal(oracle.window_unpartition(xw, B, H, W, w), x)
    # token t = iy*w + ix of unit u comes from pixel (wy*w+iy, wx*w+ix)
    for b in range(B):
        for wy in range(H // w):
            for wx in range(W // w):
                u = (b * (H // w) + wy) * (W // w) + wx
                for t in range(w * w):
                    iy, ix = divmod(t, w)
                    np.testing.assert_array_equal(xw[u, :, t, :], x[b, wy * w + iy, wx * w + ix])
    with pytest.raises(ValueError):
        oracle.window_partition(np.zeros((1, w + 1, w, 1, 1)), w)


# ---------------------------------------------------------------- hand example

def _parse_worked(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split(":"))
            out[k] = v.split()
    return out


def _val(tok):
    if tok.startswith("ln(") and tok.endswith(")"):
        return math.log(float(Fraction(tok[3:-1])))
    if tok == "ln2":
        return math.log(2.0)
    return float(Fraction(tok))


def test_worked_example_w2(golden_dir):
    g = _parse_worked(os.path.join(golden_dir, "worked_example_w2.txt"))
    col = lambda k: np.array([_val(t) for t in g[k]]).reshape(1, 2, 2, 1, 1)
    q_c, k_c, v, d_o = col("q_c"), col("k_c"), col("v"), col("d_o")
    q_p = np.array([_val(t) for t in g["q_p"]]).reshape(4, 1)
    k_p = np.array([_val(t) for t in g["k_p"]]).reshape(4, 1)
    scale = _val(g["scale"][0])
    O, L = oracle.rib_window_attn_fwd(q_c, k_c, v, q_p, k_p, 2, scale)
    np.testing.assert_allclose(O.ravel(), [_val(t) for t in g["o"]], rtol=1e-14)
    np.testing.assert_allclose(L.ravel(), [_val(t) for t in g["lse"]], rtol=1e-14)
    dq, dk, dv, dqp, dkp = oracle.rib_window_attn_bwd(q_c, k_c, v, q_p, k_p, d_o, 2, scale)
    ln2 = math.log(2.0)
    np.testing.assert_allclose(dv.ravel(), [_val(t) for t in g["dv"]], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(dq.ravel() / ln2, [_val(t) for t in g["dq_c_over_ln2"]], atol=1e-12)
    np.testing.assert_allclose(dqp.ravel() / ln2, [_val(t) for t in g["dq_p_over_ln2"]], atol=1e-12)
    np.testing.assert_allclose(dk.ravel() / ln2, [_val(t) for t in g["dk_c_over_ln2"]], atol=1e-12)
    np.testing.assert_allclose(dkp.ravel() / ln2, [_val(t) for t in g["dk_p_over_ln2"]], atol=1e-12)


# ---------------------------------------------------------------- forward pins

def _unit(rng, N=48, d_c=5, r=3):
    return (_rand(rng, N, d_c), _rand(rng, N, d_c), _rand(rng, N, d_c),
            _rand(rng, N, r), _rand(rng, N, r))


def test_concat_identity():
    """[Q_c,Q_p][K_c,K_p]^T = Q_c K_c^T + Q_p K_p^T (the pages' "Content + Bias" equation)."""
    rng = np.random.default_rng(1)
    qc, kc, _, qp, kp = _unit(rng, N=64, d_c=32, r=16)
    S = oracle.concat_scores(qc, kc, qp, kp, 0.37)
    ref = 0.37 * (qc @ kc.T + qp @ kp.T)
    np.testing.assert_allclose(S, ref, rtol=1e-12, atol=1e-12)


def test_softmax_rows_sum_to_one_and_lse():
    rng = np.random.default_rng(2)
    qc, kc, v, qp, kp = _unit(rng, N=100)
    O, lse, P = oracle.attention_window_fwd(qc, kc, v, qp, kp, 0.8)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    assert (P >= 0).all()
    from scipy.special import logsumexp
    S = 0.8 * (qc @ kc.T + qp @ kp.T)
    np.testing.assert_allclose(lse, logsumexp(S, axis=1), rtol=1e-13)


def test_matches_torch_sdpa_with_additive_bias():
    """torch SDPA(Q_c, K_c, V, attn_mask = scale Q_p K_p^T) = the RIB output (library route)."""
    rng = np.random.default_rng(3)
    qc, kc, v, qp, kp = _unit(rng, N=81, d_c=6, r=4)
    scale = 0.41
    O, _, _ = oracle.attention_window_fwd(qc, kc, v, qp, kp, scale)
    t = lambda a: torch.from_numpy(a)[None, None]
    bias = torch.from_numpy(scale * (qp @ kp.T))[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(qc), t(kc), t(v), attn_mask=bias, scale=scale)
    np.testing.assert_allclose(O, ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)
    # concatenated channels through SDPA (query/key width differs from value width)
    qh = torch.from_numpy(np.concatenate([qc, qp], 1))[None, None]
    kh = torch.from_numpy(np.concatenate([kc, kp], 1))[None, None]
    ref2 = torch.nn.functional.scaled_dot_product_attention(qh, kh, t(v), scale=scale)
    np.testing.assert_allclose(O, ref2[0, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_default_scale_is_sdpa_default_over_concatenated_channels():
    """default_scale (reading R8: the scale multiplies the whole concatenated product) against
    torch SDPA's own default scale, 1/sqrt of the query width, applied to [Q_c | Q_p]: the map-level
    oracle with scale=None equals SDPA with no scale argument on the concatenated channels."""
    rng = np.random.default_rng(11)
    B, H, W, heads, d_c, w, r = 1, 6, 6, 2, 5, 3, 3
    q = rng.standard_normal((B, H, W, heads, d_c))
    k = rng.standard_normal((B, H, W, heads, d_c))
    v = rng.standard_normal((B, H, W, heads, d_c))
    qp = rng.standard_normal((w * w, r))
    kp = rng.standard_normal((w * w, r))
    O, _ = oracle.rib_window_attn_fwd(q, k, v, qp, kp, w)
    qw, kw, vw, ow = (oracle.window_partition(x, w) for x in (q, k, v, O))   # [windows, heads, N, d]
    for u in range(qw.shape[0]):
        for h in range(heads):
            qh = torch.from_numpy(np.concatenate([qw[u, h], qp], 1))[None, None]
            kh = torch.from_numpy(np.concatenate([kw[u, h], kp], 1))[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, torch.from_numpy(vw[u, h])[None, None])
            np.testing.assert_allclose(ow[u, h], ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_zero_positional_tokens_reduce_to_plain_attention():
    rng = np.random.default_rng(4)
    qc, kc, v, qp, kp = _unit(rng, N=36)
    O, _, _ = oracle.attention_window_fwd(qc, kc, v, 0 * qp, 0 * kp, 0.5)
    t = lambda a: torch.from_numpy(a)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(qc), t(kc), t(v), scale=0.5)
    np.testing.assert_allclose(O, ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(5)
    qc, kc, v, qp, kp = _unit(rng, N=49)
    # constant V -> constant O
    cst = np.tile(np.array([[1.5, -2.0, 0.25, 3.0, -1.0]]), (49, 1))
    O, _, _ = oracle.attention_window_fwd(qc, kc, cst, qp, kp, 0.7)
    np.testing.assert_allclose(O, cst, atol=1e-13)
    # all scores zero -> O_i = mean_j V_j
    O, lse, _ = oracle.attention_window_fwd(0 * qc, 0 * kc, v, 0 * qp, 0 * kp, 0.7)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(0), O.shape), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(49), atol=1e-13)
    # one dominant key -> that key's value
    kc2 = kc.copy()
    kc2[17] = 60.0 * qc[3] / np.linalg.norm(qc[3])
    O, _, _ = oracle.attention_window_fwd(qc, kc2, v, 0 * qp, 0 * kp, 1.0)
    np.testing.assert_allclose(O[3], v[17], atol=1e-6)


def test_row_shift_and_permutation_invariance():
    rng = np.random.default_rng(6)
    qc, kc, v, qp, kp = _unit(rng, N=40)
    O, _, _ = oracle.attention_window_fwd(qc, kc, v, qp, kp, 0.6)
    # adding one vector u to every key shifts row i of S by scale*q_i.u: O unchanged
    u = rng.standard_normal(kc.shape[1])
    O2, _, _ = oracle.attention_window_fwd(qc, kc + u, v, qp, kp, 0.6)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    # permuting keys and values together: O unchanged
    p = rng.permutation(40)
    O3, _, _ = oracle.attention_window_fwd(qc, kc[p], v[p], qp, kp[p], 0.6)
    np.testing.assert_allclose(O3, O, atol=1e-12)
    # permuting queries permutes the rows of O
    O4, _, _ = oracle.attention_window_fwd(qc[p], kc, v, qp[p], kp, 0.6)
    np.testing.assert_allclose(O4, O[p], atol=1e-12)


def test_full_map_units_and_shared_bias():
    """The whole-map routine applies the same (Q_p, K_p) to every window and head."""
    rng = np.random.default_rng(7)
    B, H, W, heads, d, w, r = 2, 8, 12, 3, 4, 4, 2
    q, k, v = (_rand(rng, B, H, W, heads, d) for _ in range(3))
    qp, kp = _rand(rng, w * w, r), _rand(rng, w * w, r)
    O, L = oracle.rib_window_attn_fwd(q, k, v, qp, kp, w)
    assert not np.isnan(O).any() and not np.isnan(L).any()
    qw, kw, vw = (oracle.window_partition(a, w) for a in (q, k, v))
    Ow = oracle.window_partition(O, w)
    scale = 1 / math.sqrt(d + r)
    for u in range(qw.shape[0]):
        for h in range(heads):
            o, _, _ = oracle.attention_window_fwd(qw[u, h], kw[u, h], vw[u, h], qp, kp, scale)
            np.testing.assert_allclose(Ow[u, h], o, atol=1e-13)
    O2, _ = oracle.rib_window_attn_fwd(q, k, v, qp, kp, w, units=[(1, 1, 2, 2)])
    np.testing.assert_array_equal(O2[1, 4:8, 8:12, 2], O[1, 4:8, 8:12, 2])
    assert np.isnan(O2[0]).all()


# ---------------------------------------------------------------- backward pins

def _loss(qc, kc, v, qp, kp, do, scale):
    O, _, _ = oracle.attention_window_fwd(qc, kc, v, qp, kp, scale)
    return float((O * do).sum())


def test_backward_finite_differences():
    """Central differences in float64 on every input element, relative error <= 1e-7."""
    rng = np.random.default_rng(8)
    N, d_c, r, scale = 16, 3, 2, 0.55
    args = [_rand(rng, N, d_c), _rand(rng, N, d_c), _rand(rng, N, d_c), _rand(rng, N, r), _rand(rng, N, r)]
    do = _rand(rng, N, d_c)
    grads = oracle.attention_window_bwd(*args, do, scale)
    order = [0, 1, 2, 3, 4]          # qc, kc, v, qp, kp
    gmap = {0: grads[0], 1: grads[1], 2: grads[2], 3: grads[3], 4: grads[4]}
    h = 1e-5
    for a in order:
        num = np.zeros_like(args[a])
        for idx in np.ndindex(args[a].shape):
            plus = [x.copy() for x in args]
            minus = [x.copy() for x in args]
            plus[a][idx] += h
            minus[a][idx] -= h
            num[idx] = (_loss(*plus, do, scale) - _loss(*minus, do, scale)) / (2 * h)
        err = np.abs(num - gmap[a]).max() / max(np.abs(num).max(), 1e-30)
        assert err <= 1e-7, (a, err)


def test_backward_matches_torch_autograd():
    rng = np.random.default_rng(9)
    N, d_c, r, scale = 64, 8, 4, 0.3
    arrs = [_rand(rng, N, d_c), _rand(rng, N, d_c), _rand(rng, N, d_c), _rand(rng, N, r), _rand(rng, N, r)]
    do = _rand(rng, N, d_c)
    g = oracle.attention_window_bwd(*arrs, do, scale)
    ts = [torch.from_numpy(a.copy()).requires_grad_(True) for a in arrs]
    qc, kc, v, qp, kp = ts
    bias = scale * (qp @ kp.T)
    O = torch.nn.functional.scaled_dot_product_attention(qc[None, None], kc[None, None], v[None, None],
                                                         attn_mask=bias[None, None], scale=scale)[0, 0]
    (O * torch.from_numpy(do)).sum().backward()
    for got, t in zip(g, ts):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_backward_invariants():
    """Rows of dS sum to zero, so per unit sum_j dK_c[j] = 0 and sum_j dK_p[j] = 0;
    and sum_j dV_j = sum_i dO_i because rows of P sum to one."""
    rng = np.random.default_rng(10)
    N, d_c, r = 81, 6, 4
    args = [_rand(rng, N, d_c), _rand(rng, N, d_c), _rand(rng, N, d_c), _rand(rng, N, r), _rand(rng, N, r)]
    do = _rand(rng, N, d_c)
    dqc, dkc, dv, dqp, dkp = oracle.attention_window_bwd(*args, do, 0.45)
    np.testing.assert_allclose(dkc.sum(0), 0, atol=1e-12)
    np.testing.assert_allclose(dkp.sum(0), 0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(0), do.sum(0), atol=1e-12)


def test_full_map_backward_sums_positional_grads():
    rng = np.random.default_rng(11)
    B, H, W, heads, d, w, r = 1, 8, 8, 2, 3, 4, 2
    q, k, v, do = (_rand(rng, B, H, W, heads, d) for _ in range(4))
    qp, kp = _rand(rng, w * w, r), _rand(rng, w * w, r)
    dq, dk, dv, dqp, dkp = oracle.rib_window_attn_bwd(q, k, v, qp, kp, do, w)
    ts = [torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v, qp, kp)]
    # autograd through a torch window split written with reshape/permute (library route)
    def split(x):
        x = x.reshape(B, H // w, w, W // w, w, heads, d).permute(0, 1, 3, 5, 2, 4, 6)
        return x.reshape(-1, heads, w * w, d)
    scale = 1 / math.sqrt(d + r)
    bias = scale * (ts[3] @ ts[4].T)
    O = torch.nn.functional.scaled_dot_product_attention(split(ts[0]), split(ts[1]), split(ts[2]),
                                                         attn_mask=bias, scale=scale)
    (O * split(torch.from_numpy(do))).sum().backward()
    for got, t in zip((dq, dk, dv, dqp, dkp), ts):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-11, atol=1e-12)

"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case swaps one oracle function for a plausibly wrong variant (a dropped
term, a wrong sign, index or operand) and checks that at least one pin test
fails on it. Nothing here touches the GPU.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.rib as orib
import test_oracle_attention as ta
import test_oracle_posgen as tp
import test_oracle_posgen_bwd as tb
import test_oracle_rpb as tr
import test_oracle_cla as tc


def _golden():
    import os
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _scores_no_bias(qc, kc, qp, kp, scale):
    return scale * (np.asarray(qc) @ np.asarray(kc).T)


def _scores_transposed_bias(qc, kc, qp, kp, scale):
    return scale * (np.asarray(qc) @ np.asarray(kc).T + np.asarray(kp) @ np.asarray(qp).T)


def _scores_unscaled_bias(qc, kc, qp, kp, scale):
    return scale * (np.asarray(qc) @ np.asarray(kc).T) + np.asarray(qp) @ np.asarray(kp).T


def _fwd_wrong_axis(qc, kc, v, qp, kp, scale):
    S = orib.concat_scores(qc, kc, qp, kp, scale)
    E = np.exp(S - S.max(axis=0, keepdims=True))
    P = E / E.sum(axis=0, keepdims=True)
    return P @ np.asarray(v, np.float64), np.log(np.exp(S).sum(1)), P


def _bwd_missing_d(qc, kc, v, qp, kp, do, scale):
    qc, kc, v, qp, kp, do = (np.asarray(a, np.float64) for a in (qc, kc, v, qp, kp, do))
    _, _, P = orib.attention_window_fwd(qc, kc, v, qp, kp, scale)
    dS = P * (do @ v.T)                       # D term dropped
    qh = np.concatenate([qc, qp], 1)
    kh = np.concatenate([kc, kp], 1)
    dq, dk = scale * dS @ kh, scale * dS.T @ qh
    d = qc.shape[1]
    return dq[:, :d], dk[:, :d], P.T @ do, dq[:, d:], dk[:, d:]


def _bwd_unscaled(qc, kc, v, qp, kp, do, scale):
    g = list(orib.__dict__["_orig_bwd"](qc, kc, v, qp, kp, do, scale))
    return g[0], g[1] / scale, g[2], g[3], g[4] / scale


def _default_scale_content_only(d_c, rank):
    return 1.0 / math.sqrt(d_c)


def _coords_pixel_centres(w):
    n = [2 * i + 1 - w for i in range(w)]
    return n, np.array([v / w for v in n])


def _fourier_linear_freqs(w, F):
    _, c = orib.window_coords(w)
    out = np.zeros((w * w, 4 * F))
    for t in range(w * w):
        iy, ix = divmod(t, w)
        for k in range(F):
            a, b = (k + 1) * math.pi * c[ix], (k + 1) * math.pi * c[iy]
            out[t, [k, F + k, 2 * F + k, 3 * F + k]] = [math.sin(a), math.cos(a), math.sin(b), math.cos(b)]
    return out


def _fourier_interleaved(w, F):
    f = orib.__dict__["_orig_fourier"](w, F)
    return f.reshape(w * w, 4, F).transpose(0, 2, 1).reshape(w * w, 4 * F)


def _posgen_swapped(w, F, w1, b1, w2, b2, r):
    qp, kp = orib.__dict__["_orig_posgen"](w, F, w1, b1, w2, b2, r)
    return kp, qp


def _gelu_tanh(z):
    z = np.asarray(z, np.float64)
    return 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))


def _partition_col_major(x, w):
    B, H, W, heads, d = x.shape
    out = orib.__dict__["_orig_partition"](x, w)
    N = w * w
    perm = np.array([(t % w) * w + t // w for t in range(N)])
    return out[:, :, perm, :]


def _gelu_grad_cdf_only(z):
    z = np.asarray(z, np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * (1.0 + erf(z / math.sqrt(2.0)))          # the z phi(z) term dropped


def _gelu_grad_tanh(z):
    z = np.asarray(z, np.float64)
    c = math.sqrt(2 / math.pi)
    u = c * (z + 0.044715 * z ** 3)
    t = np.tanh(u)
    return 0.5 * (1 + t) + 0.5 * z * (1 - t * t) * c * (1 + 3 * 0.044715 * z * z)


def _posgen_bwd_no_gelu_grad(w, F, w1, b1, w2, b2, r, dq, dk):
    phi = orib.fourier_features(w, F)
    z = phi @ np.asarray(w1).T + (0 if b1 is None else np.asarray(b1))
    h = orib.gelu(z)
    d_out = np.hstack([dq, dk])
    dz = d_out @ np.asarray(w2)                            # GELU' missing
    return dz.T @ phi, dz.sum(0), d_out.T @ h, d_out.sum(0)


def _posgen_bwd_split_swapped(w, F, w1, b1, w2, b2, r, dq, dk):
    return orib.__dict__["_orig_posgen_bwd"](w, F, w1, b1, w2, b2, r, dk, dq)


def _posgen_bwd_w1_transposed(w, F, w1, b1, w2, b2, r, dq, dk):
    g = list(orib.__dict__["_orig_posgen_bwd"](w, F, w1, b1, w2, b2, r, dq, dk))
    return g[0].T.reshape(g[0].shape), g[1], g[2], g[3]


def _rpb_bias_reversed(w, table):
    t = np.arange(w * w)
    iy, ix = t // w, t % w
    idx = (iy[None, :] - iy[:, None] + w - 1) * (2 * w - 1) + (ix[None, :] - ix[:, None] + w - 1)   # j - i
    return np.asarray(table, np.float64)[idx]


def _rpb_bias_xy_swapped(w, table):
    t = np.arange(w * w)
    iy, ix = t // w, t % w
    idx = (ix[:, None] - ix[None, :] + w - 1) * (2 * w - 1) + (iy[:, None] - iy[None, :] + w - 1)
    return np.asarray(table, np.float64)[idx]


def _rpb_fwd_scaled_bias(qc, kc, v, bias, scale):
    return orib.__dict__["_orig_rpb_fwd"](qc, kc, v, scale * np.asarray(bias), scale)


def _cla_dw_flipped(x, w_dw, b_dw=None):
    return orib.__dict__["_orig_cla_dw"](x, np.asarray(w_dw)[:, ::-1, ::-1], b_dw)   # convolution, not correlation


def _cla_dw_wraparound(x, w_dw, b_dw=None):
    x = np.asarray(x, dtype=np.float64)
    w_dw = np.asarray(w_dw, dtype=np.float64)
    d = np.zeros(x.shape)
    for ky in range(3):
        for kx in range(3):
            d += w_dw[:, ky, kx] * np.roll(x, (1 - ky, 1 - kx), axis=(1, 2))
    return d if b_dw is None else d + np.asarray(b_dw)


def _cla_gate_pw_transposed(x, w_dw, b_dw, w_pw, b_pw):
    return orib.__dict__["_orig_cla_gate"](x, w_dw, b_dw, np.asarray(w_pw).T, b_pw)


def _cla_apply_channels_transposed(o, g):
    o = np.asarray(o, dtype=np.float64)
    B, H, W, heads, d_c = o.shape
    return o * np.asarray(g).reshape(B, H, W, d_c, heads).swapaxes(3, 4)


MUTATIONS = [
    ("concat_scores", _scores_no_bias, [(ta.test_worked_example_w2, "golden"), (ta.test_concat_identity,)]),
    ("concat_scores", _scores_transposed_bias, [(ta.test_concat_identity,), (ta.test_matches_torch_sdpa_with_additive_bias,)]),
    ("concat_scores", _scores_unscaled_bias, [(ta.test_worked_example_w2, "golden"), (ta.test_concat_identity,)]),
    ("attention_window_fwd", _fwd_wrong_axis, [(ta.test_softmax_rows_sum_to_one_and_lse,), (ta.test_closed_forms,)]),
    ("attention_window_bwd", _bwd_missing_d, [(ta.test_backward_finite_differences,), (ta.test_backward_invariants,)]),
    ("attention_window_bwd", _bwd_unscaled, [(ta.test_backward_finite_differences,), (ta.test_worked_example_w2, "golden")]),
    ("default_scale", _default_scale_content_only, [(ta.test_default_scale_is_sdpa_default_over_concatenated_channels,)]),
    ("window_coords", _coords_pixel_centres, [(tp.test_coords_match_linspace, 16), (tp.test_fourier_hand_derived, "golden")]),
    ("fourier_features", _fourier_linear_freqs, [(tp.test_fourier_hand_derived, "golden"), (tp.test_fourier_periodicity_power_of_two_windows, 4)]),
    ("fourier_features", _fourier_interleaved, [(tp.test_fourier_hand_derived, "golden")]),
    ("posgen", _posgen_swapped, [(tp.test_posgen_matches_torch_mlp, 16, 8)]),
    ("gelu", _gelu_tanh, [(tp.test_gelu_matches_torch,), (tp.test_posgen_matches_torch_mlp, 32, 16)]),
    ("window_partition", _partition_col_major, [(ta.test_partition_bijection_brute_force, 2, 6, 9, 2, 3, 3)]),
    ("gelu_grad", _gelu_grad_cdf_only, [(tb.test_gelu_grad_closed_forms,), (tb.test_posgen_bwd_finite_differences, 3, 2, 5, 2)]),
    ("gelu_grad", _gelu_grad_tanh, [(tb.test_gelu_grad_closed_forms,), (tb.test_posgen_bwd_matches_torch_autograd, 8, 16, 64, 8)]),
    ("posgen_bwd", _posgen_bwd_no_gelu_grad, [(tb.test_posgen_bwd_finite_differences, 3, 2, 5, 2)]),
    ("posgen_bwd", _posgen_bwd_split_swapped, [(tb.test_posgen_bwd_finite_differences, 3, 2, 5, 2), (tb.test_posgen_bwd_split_and_linearity,)]),
    ("posgen_bwd", _posgen_bwd_w1_transposed, [(tb.test_posgen_bwd_matches_torch_autograd, 8, 16, 64, 8)]),
    ("rpb_bias", _rpb_bias_reversed, [(tr.test_rpb_bias_brute_force, 3), (tr.test_rpb_linear_table_equals_rib_with_rank3_tokens,)]),
    ("rpb_bias", _rpb_bias_xy_swapped, [(tr.test_rpb_bias_brute_force, 3), (tr.test_rpb_linear_table_equals_rib_with_rank3_tokens,)]),
    ("rpb_attention_window_fwd", _rpb_fwd_scaled_bias, [(tr.test_rpb_matches_torch_sdpa_with_additive_mask,), (tr.test_rpb_linear_table_equals_rib_with_rank3_tokens,)]),
    ("cla_depthwise3x3", _cla_dw_flipped, [(tc.test_cla_matches_torch_conv2d, 2, 7, 9, 12), (tc.test_cla_brute_force_pixels,)]),
    ("cla_depthwise3x3", _cla_dw_wraparound, [(tc.test_cla_constant_map_border_counts,), (tc.test_cla_brute_force_pixels,)]),
    ("cla_gate", _cla_gate_pw_transposed, [(tc.test_cla_matches_torch_conv2d, 2, 7, 9, 12), (tc.test_cla_brute_force_pixels,)]),
    ("cla_apply", _cla_apply_channels_transposed, [(tc.test_cla_apply_channel_mapping,)]),
]


@pytest.mark.parametrize("name,bad,pins", MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, bad, pins):
    orig = getattr(orib, name)
    for key, fn in (("_orig_bwd", orib.attention_window_bwd), ("_orig_fourier", orib.fourier_features),
                    ("_orig_posgen", orib.posgen), ("_orig_partition", orib.window_partition),
                    ("_orig_posgen_bwd", orib.posgen_bwd), ("_orig_rpb_fwd", orib.rpb_attention_window_fwd),
                    ("_orig_cla_dw", orib.cla_depthwise3x3), ("_orig_cla_gate", orib.cla_gate)):
        monkeypatch.setitem(orib.__dict__, key, fn)
    monkeypatch.setattr(orib, name, bad)
    monkeypatch.setattr(oracle, name, bad)
    caught = []
    for pin in pins:
        fn, args = pin[0], [(_golden() if a == "golden" else a) for a in pin[1:]]
        caught.append(_fails(fn, *args))
    assert any(caught), f"no pin caught the planted mistake in {name}"
    monkeypatch.setattr(orib, name, orig)
    # the unmodified oracle passes the same pins
    monkeypatch.setattr(oracle, name, orig)
    for pin in pins:
        fn, args = pin[0], [(_golden() if a == "golden" else a) for a in pin[1:]]
        fn(*args)

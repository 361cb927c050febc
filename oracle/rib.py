"""Plain float64 CPU oracle of Rank-factorized Implicit Neural Bias (RIB) window attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): a slow, obviously correct
statement of what the GPU path computes. No blocking, fusion or reordering.

Sources: web pages on the paper "Rank-Factorized Implicit Neural Bias: Scaling
Super-Resolution Transformer with FlashAttention" (arXiv 2603.06738):

  [EN]  gist.science/paper/2603.06738        - "Technical Summary"
  [DE]  gist.science/de/paper/2603.06738     - "Technische Zusammenfassung"
  [ES]  gist.science/es/paper/2603.06738     - "Resumen tecnico"
  [ZH]  gist.science/zh/paper/2603.06738     - technical part
  [ABS] khansong-paper-with-me.hf.space      - the paper's abstract

What the pages fix:
  * each token gets a normalized 2D coordinate in [-1, 1]           [DE §2.A.1]
  * the coordinates are lifted by a Fourier-feature map             [DE §2.A.1], [EN §2.A.1]
  * a lightweight MLP maps them to low-rank Q_p and K_p             [DE §2.A.2], [EN §2.A.2]
  * Q_p, K_p are concatenated channel-wise to Q_c, K_c and the
    score is one dot product S = [Q_c,Q_p][K_c,K_p]^T
    = Q_c K_c^T + Q_p K_p^T                                         [EN §2.A.3-4 "Content + Bias"]
  * Q_p, K_p depend only on window geometry (cacheable)             [DE §2.A.4], [ZH §2.A]
  * the bias parameter count does not depend on the window size     [EN §2.A "Advantages"]
  * square windows up to 96 x 96                                    [EN §3.2], [ABS]

Readings where the pages are silent (each is also listed in the design notes):
  R1  coordinates are linspace(-1, 1, w), endpoints included
  R2  token t = iy*w + ix inside a window (row-major); x is the column
  R3  features per token: [sin(2^k pi x)]_k, [cos(2^k pi x)]_k,
      [sin(2^k pi y)]_k, [cos(2^k pi y)]_k, k = 0..F-1 ascending (4F total)
  R5  MLP = Linear -> GELU (exact erf form) -> Linear, nn.Linear layout
  R6  the first r MLP outputs are Q_p, the last r are K_p
  R7  one (Q_p, K_p) per window size, shared by every window, batch and head
  R8  scale multiplies the whole concatenated product
  R9  V is content only; O has d_c channels
  R10 non-overlapping windows, no shift, no padding; H and W divisible by w
  R14 D_i = sum_j P_ij dP_ij (textbook softmax backward)
  R17 the RPB comparison (the bias RIB replaces, S = QK^T + B): one table of
      (2w-1)^2 entries per head, B[i, j] = table[(y_i - y_j + w - 1)(2w - 1)
      + (x_i - x_j + w - 1)]; the bias is added after the scale; default
      scale 1/sqrt(d_c)
  R16 the position MLP is trained with the network: the positional gradients
      dQ_p, dK_p continue through Linear -> GELU -> Linear into dW1, db1,
      dW2, db2 by the chain rule; GELU'(z) = Phi(z) + z phi(z) (erf form, R5)
  R18 the CLA gate (depth-wise 3x3 conv, point-wise 1x1 conv, sigmoid -> G,
      O' = O * G): its input X is the attention block's input map
      [B, H, W, C] with C = heads * d_c channels; both convs carry a bias;
      the 3x3 conv is a cross-correlation over the whole map (not per window)
      with zero padding 1 ("same" size); tap w_dw[c, ky, kx] weights
      X[y + ky - 1, x + kx - 1, c]; the 1x1 conv is Z = D W_pw^T + b_pw with
      W_pw [C_out, C_in]; channel c of G gates head c // d_c, channel
      c % d_c of O

Parity pins live in ``tests/test_oracle_*.py`` (closed forms, invariants,
library routines, brute force and hand-derived fixtures in ``tests/golden/``).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "window_coords", "fourier_features", "gelu", "mlp_param_count", "posgen",
    "window_partition", "window_unpartition",
    "concat_scores", "attention_window_fwd", "attention_window_bwd",
    "rib_window_attn_fwd", "rib_window_attn_bwd", "default_scale",
    "gelu_grad", "posgen_bwd",
    "rpb_bias", "rpb_attention_window_fwd", "rpb_window_attn_fwd",
    "cla_depthwise3x3", "cla_gate", "cla_apply",
]


# ----------------------------------------------------------------------------
# Position-token generation
# ----------------------------------------------------------------------------

def window_coords(w: int):
    """Normalized in-window coordinates [DE §2.A.1: x in [-1, 1]], reading R1.

    Returns (n, c): integer numerators n_i = 2i - (w-1) and c_i = n_i / (w-1),
    i = 0..w-1, so c_0 = -1 and c_{w-1} = +1 exactly.
    """
    if w < 2:
        raise ValueError("window size must be >= 2")
    n = [2 * i - (w - 1) for i in range(w)]
    c = np.array([ni / (w - 1) for ni in n], dtype=np.float64)
    return n, c


def fourier_features(w: int, n_freq: int) -> np.ndarray:
    """Fourier-feature map of the token coordinates [DE §2.A.1], [EN §2.A.1], reading R3.

    Token t = iy*w + ix (R2) has (x, y) = (c_ix, c_iy). Its feature vector is
    [sin(2^k pi x)]_k ++ [cos(2^k pi x)]_k ++ [sin(2^k pi y)]_k ++ [cos(2^k pi y)]_k
    for k = 0..n_freq-1. Evaluated straight from the definition in float64; the
    argument reaches 2^15 pi, where float64 keeps the absolute error near 1e-11.
    """
    _, c = window_coords(w)
    N = w * w
    feats = np.zeros((N, 4 * n_freq), dtype=np.float64)
    for t in range(N):
        iy, ix = divmod(t, w)
        x, y = c[ix], c[iy]
        for k in range(n_freq):
            fx = (2.0 ** k) * math.pi * x
            fy = (2.0 ** k) * math.pi * y
            feats[t, k] = math.sin(fx)
            feats[t, n_freq + k] = math.cos(fx)
            feats[t, 2 * n_freq + k] = math.sin(fy)
            feats[t, 3 * n_freq + k] = math.cos(fy)
    return feats


def gelu(z: np.ndarray) -> np.ndarray:
    """GELU, exact form 0.5 z (1 + erf(z / sqrt 2)) (reading R5)."""
    z = np.asarray(z, dtype=np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def mlp_param_count(n_freq: int, hidden: int, rank: int) -> int:
    """Parameters of the position MLP: W1 [hidden, 4F], b1, W2 [2r, hidden], b2.

    The window size does not enter [EN §2.A "Advantages": the bias parameter
    count is independent of the window size].
    """
    return hidden * 4 * n_freq + hidden + 2 * rank * hidden + 2 * rank


def posgen(w: int, n_freq: int, w1, b1, w2, b2, rank: int):
    """Low-rank positional tokens (Q_p, K_p) of one window size [DE §2.A.1-2], [ZH §2.A].

    phi = Fourier features (N x 4F); h = GELU(phi W1^T + b1); out = h W2^T + b2
    (nn.Linear layout, R5); Q_p = out[:, :r], K_p = out[:, r:2r] (R6).
    b1 / b2 may be None (zeros). Returns float64 arrays of shape [N, r].
    """
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    hidden = w1.shape[0]
    if w1.shape != (hidden, 4 * n_freq):
        raise ValueError("w1 must be [hidden, 4*n_freq]")
    if w2.shape != (2 * rank, hidden):
        raise ValueError("w2 must be [2*rank, hidden]")
    b1 = np.zeros(hidden) if b1 is None else np.asarray(b1, dtype=np.float64)
    b2 = np.zeros(2 * rank) if b2 is None else np.asarray(b2, dtype=np.float64)
    phi = fourier_features(w, n_freq)
    h = gelu(phi @ w1.T + b1)
    out = h @ w2.T + b2
    return out[:, :rank].copy(), out[:, rank:2 * rank].copy()


def gelu_grad(z: np.ndarray) -> np.ndarray:
    """Derivative of the exact GELU (reading R5): Phi(z) + z phi(z), with Phi the
    standard normal CDF 0.5 (1 + erf(z / sqrt 2)) and phi its density
    exp(-z^2 / 2) / sqrt(2 pi)."""
    z = np.asarray(z, dtype=np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    cdf = 0.5 * (1.0 + erf(z / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    return cdf + z * pdf


def posgen_bwd(w: int, n_freq: int, w1, b1, w2, b2, rank: int, dq_p, dk_p):
    """Weight gradients of the position MLP [DE §2.A.2: a lightweight MLP maps the
    Fourier features to Q_p, K_p], reading R16.

    Given dQ_p, dK_p ([N, r] each) for the outputs of ``posgen``, with
    phi the Fourier features (no parameters), z = phi W1^T + b1, h = GELU(z)
    and d_out = [dQ_p | dK_p] (Q_p first, R6):
      dW2 = d_out^T h        db2 = sum_t d_out[t]
      dh  = d_out W2         dz  = dh * GELU'(z)
      dW1 = dz^T phi         db1 = sum_t dz[t]
    Returns float64 (dw1 [hidden, 4F], db1 [hidden], dw2 [2r, hidden], db2 [2r]).
    """
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    hidden = w1.shape[0]
    if w1.shape != (hidden, 4 * n_freq) or w2.shape != (2 * rank, hidden):
        raise ValueError("weight shapes do not match n_freq / hidden / rank")
    b1 = np.zeros(hidden) if b1 is None else np.asarray(b1, dtype=np.float64)
    N = w * w
    dq_p = np.asarray(dq_p, dtype=np.float64)
    dk_p = np.asarray(dk_p, dtype=np.float64)
    if dq_p.shape != (N, rank) or dk_p.shape != (N, rank):
        raise ValueError("dq_p and dk_p must be [w*w, rank]")
    phi = fourier_features(w, n_freq)
    z = phi @ w1.T + b1
    h = gelu(z)
    d_out = np.concatenate([dq_p, dk_p], axis=1)
    dw2 = d_out.T @ h
    db2 = d_out.sum(axis=0)
    dz = (d_out @ w2) * gelu_grad(z)
    dw1 = dz.T @ phi
    db1 = dz.sum(axis=0)
    return dw1, db1, dw2, db2


# ----------------------------------------------------------------------------
# Window partition (reading R10; the pages use square windows but never
# describe the split)
# ----------------------------------------------------------------------------

def _check_divisible(H: int, W: int, w: int):
    if H % w or W % w:
        raise ValueError("H and W must be multiples of the window size")


def window_partition(x: np.ndarray, w: int) -> np.ndarray:
    """[B, H, W, heads, d] -> [B*nWy*nWx, heads, N, d], token t = iy*w + ix (R2)."""
    B, H, W, heads, d = x.shape
    _check_divisible(H, W, w)
    out = np.empty((B * (H // w) * (W // w), heads, w * w, d), dtype=x.dtype)
    u = 0
    for b in range(B):
        for wy in range(H // w):
            for wx in range(W // w):
                for iy in range(w):
                    for ix in range(w):
                        out[u, :, iy * w + ix, :] = x[b, wy * w + iy, wx * w + ix, :, :]
                u += 1
    return out


def window_unpartition(xw: np.ndarray, B: int, H: int, W: int, w: int) -> np.ndarray:
    """Inverse of ``window_partition``."""
    _check_divisible(H, W, w)
    nwin, heads, N, d = xw.shape
    if nwin != B * (H // w) * (W // w) or N != w * w:
        raise ValueError("shape mismatch")
    out = np.empty((B, H, W, heads, d), dtype=xw.dtype)
    u = 0
    for b in range(B):
        for wy in range(H // w):
            for wx in range(W // w):
                for iy in range(w):
                    for ix in range(w):
                        out[b, wy * w + iy, wx * w + ix, :, :] = xw[u, :, iy * w + ix, :]
                u += 1
    return out


# ----------------------------------------------------------------------------
# Attention over one window and head
# ----------------------------------------------------------------------------

def default_scale(d_c: int, rank: int) -> float:
    """1 / sqrt(d_c + r): the scale every workload of the method uses (reading R8)."""
    return 1.0 / math.sqrt(d_c + rank)


def concat_scores(qc, kc, qp, kp, scale: float) -> np.ndarray:
    """S = scale * [Q_c | Q_p] [K_c | K_p]^T, explicit N x N [EN §2.A.3-4], R8.

    The positional tokens are appended channel-wise to the content tokens and
    one dot product is taken in the widened channel space.
    """
    qhat = np.concatenate([np.asarray(qc, np.float64), np.asarray(qp, np.float64)], axis=1)
    khat = np.concatenate([np.asarray(kc, np.float64), np.asarray(kp, np.float64)], axis=1)
    return scale * (qhat @ khat.T)


def attention_window_fwd(qc, kc, v, qp, kp, scale: float):
    """softmax(S) V for one window and head, with S from ``concat_scores``.

    Returns (O [N, d_c], LSE [N], P [N, N]); LSE_i = log sum_j exp(S_ij).
    """
    S = concat_scores(qc, kc, qp, kp, scale)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    O = P @ np.asarray(v, np.float64)
    lse = m[:, 0] + np.log(l[:, 0])
    return O, lse, P


def attention_window_bwd(qc, kc, v, qp, kp, do, scale: float):
    """Gradients of sum(dO * O) for one window and head (textbook softmax backward, R14).

    dV = P^T dO; dP = dO V^T; D_i = sum_j P_ij dP_ij; dS = P * (dP - D);
    d[Q_c|Q_p] = scale dS [K_c|K_p]; d[K_c|K_p] = scale dS^T [Q_c|Q_p].
    Returns (dQ_c, dK_c, dV, dQ_p, dK_p) of this unit (dQ_p, dK_p are this
    unit's share of the shared positional-token gradients).
    """
    qc = np.asarray(qc, np.float64)
    kc = np.asarray(kc, np.float64)
    v = np.asarray(v, np.float64)
    qp = np.asarray(qp, np.float64)
    kp = np.asarray(kp, np.float64)
    do = np.asarray(do, np.float64)
    _, _, P = attention_window_fwd(qc, kc, v, qp, kp, scale)
    dv = P.T @ do
    dP = do @ v.T
    D = (P * dP).sum(axis=1, keepdims=True)
    dS = P * (dP - D)
    qhat = np.concatenate([qc, qp], axis=1)
    khat = np.concatenate([kc, kp], axis=1)
    dqhat = scale * (dS @ khat)
    dkhat = scale * (dS.T @ qhat)
    d_c = qc.shape[1]
    return dqhat[:, :d_c], dkhat[:, :d_c], dv, dqhat[:, d_c:], dkhat[:, d_c:]


# ----------------------------------------------------------------------------
# Whole feature maps
# ----------------------------------------------------------------------------

def _all_units(B, H, W, w, heads):
    for b in range(B):
        for wy in range(H // w):
            for wx in range(W // w):
                for head in range(heads):
                    yield (b, wy, wx, head)


def _window_tokens(x, b, wy, wx, head, w):
    """[N, d] tokens of one window and head of a [B, H, W, heads, d] tensor (R2)."""
    blk = np.asarray(x[b, wy * w:(wy + 1) * w, wx * w:(wx + 1) * w, head, :], np.float64)
    return blk.reshape(w * w, -1)


def rib_window_attn_fwd(q_c, k_c, v, q_p, k_p, w: int, scale: float | None = None, units=None):
    """RIB window attention over a [B, H, W, heads, d_c] feature map.

    For every (batch, window, head) unit (or only the listed ``units``, tuples
    (b, wy, wx, head)) computes ``attention_window_fwd`` with the shared (Q_p, K_p)
    of this window size (R7). Returns (O [B,H,W,heads,d_c], LSE [B,H,W,heads]);
    entries of units not computed are NaN.
    """
    B, H, W, heads, d_c = q_c.shape
    _check_divisible(H, W, w)
    r = q_p.shape[1]
    if scale is None:
        scale = default_scale(d_c, r)
    O = np.full((B, H, W, heads, d_c), np.nan)
    L = np.full((B, H, W, heads), np.nan)
    for (b, wy, wx, head) in (units if units is not None else _all_units(B, H, W, w, heads)):
        o, lse, _ = attention_window_fwd(
            _window_tokens(q_c, b, wy, wx, head, w), _window_tokens(k_c, b, wy, wx, head, w),
            _window_tokens(v, b, wy, wx, head, w), q_p, k_p, scale)
        O[b, wy * w:(wy + 1) * w, wx * w:(wx + 1) * w, head, :] = o.reshape(w, w, d_c)
        L[b, wy * w:(wy + 1) * w, wx * w:(wx + 1) * w, head] = lse.reshape(w, w)
    return O, L


def rpb_bias(w: int, table) -> np.ndarray:
    """N x N relative-position bias of one head from its table (the RPB the pages contrast RIB with,
    S = QK^T + B [EN "Problem Statement"; ES §1]), reading R17: token t = iy*w + ix (R2) and
    B[i, j] = table[(y_i - y_j + w - 1) * (2w - 1) + (x_i - x_j + w - 1)]."""
    table = np.asarray(table, dtype=np.float64)
    if table.shape != ((2 * w - 1) ** 2,):
        raise ValueError("table must hold (2w - 1)^2 entries")
    t = np.arange(w * w)
    iy, ix = t // w, t % w
    idx = (iy[:, None] - iy[None, :] + w - 1) * (2 * w - 1) + (ix[:, None] - ix[None, :] + w - 1)
    return table[idx]


def rpb_attention_window_fwd(qc, kc, v, bias, scale: float):
    """softmax(scale Q_c K_c^T + B) V for one window and head (R17). Returns (O, LSE)."""
    S = scale * (np.asarray(qc, np.float64) @ np.asarray(kc, np.float64).T) + np.asarray(bias, np.float64)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return (E / l) @ np.asarray(v, np.float64), m[:, 0] + np.log(l[:, 0])


def rpb_window_attn_fwd(q_c, k_c, v, table, w: int, scale: float | None = None, units=None):
    """RPB window attention over a [B, H, W, heads, d_c] map with tables [heads, (2w - 1)^2] (R17).

    Same windowing as ``rib_window_attn_fwd``; returns (O, LSE) with NaN for units not computed.
    """
    B, H, W, heads, d_c = q_c.shape
    _check_divisible(H, W, w)
    table = np.asarray(table, dtype=np.float64)
    if table.shape != (heads, (2 * w - 1) ** 2):
        raise ValueError("table must be [heads, (2w - 1)^2]")
    if scale is None:
        scale = 1.0 / math.sqrt(d_c)
    O = np.full((B, H, W, heads, d_c), np.nan)
    L = np.full((B, H, W, heads), np.nan)
    biases = {}
    for (b, wy, wx, head) in (units if units is not None else _all_units(B, H, W, w, heads)):
        if head not in biases:
            biases[head] = rpb_bias(w, table[head])
        o, lse = rpb_attention_window_fwd(_window_tokens(q_c, b, wy, wx, head, w),
                                          _window_tokens(k_c, b, wy, wx, head, w),
                                          _window_tokens(v, b, wy, wx, head, w), biases[head], scale)
        O[b, wy * w:(wy + 1) * w, wx * w:(wx + 1) * w, head, :] = o.reshape(w, w, d_c)
        L[b, wy * w:(wy + 1) * w, wx * w:(wx + 1) * w, head] = lse.reshape(w, w)
    return O, L


def rib_window_attn_bwd(q_c, k_c, v, q_p, k_p, d_o, w: int, scale: float | None = None, units=None):
    """Backward of ``rib_window_attn_fwd`` given the upstream gradient dO.

    Returns (dQ_c, dK_c, dV [B,H,W,heads,d_c], dQ_p, dK_p [N, r]). dQ_p and dK_p
    sum the shares of the computed units (all units unless ``units`` is given);
    content gradients of units not computed are NaN.
    """
    B, H, W, heads, d_c = q_c.shape
    _check_divisible(H, W, w)
    r = q_p.shape[1]
    if scale is None:
        scale = default_scale(d_c, r)
    dQ = np.full((B, H, W, heads, d_c), np.nan)
    dK = np.full((B, H, W, heads, d_c), np.nan)
    dV = np.full((B, H, W, heads, d_c), np.nan)
    dqp = np.zeros((w * w, r))
    dkp = np.zeros((w * w, r))
    for (b, wy, wx, head) in (units if units is not None else _all_units(B, H, W, w, heads)):
        g = attention_window_bwd(
            _window_tokens(q_c, b, wy, wx, head, w), _window_tokens(k_c, b, wy, wx, head, w),
            _window_tokens(v, b, wy, wx, head, w), q_p, k_p,
            _window_tokens(d_o, b, wy, wx, head, w), scale)
        sl = (b, slice(wy * w, (wy + 1) * w), slice(wx * w, (wx + 1) * w), head)
        dQ[sl] = g[0].reshape(w, w, d_c)
        dK[sl] = g[1].reshape(w, w, d_c)
        dV[sl] = g[2].reshape(w, w, d_c)
        dqp += g[3]
        dkp += g[4]
    return dQ, dK, dV, dqp, dkp


# ----------------------------------------------------------------------------
# Convolutional local attention (CLA) gate
# ----------------------------------------------------------------------------

def cla_depthwise3x3(x, w_dw, b_dw=None) -> np.ndarray:
    """Depth-wise 3x3 convolution of a [B, H, W, C] map, zero padding 1 (R18): the first stage of the
    CLA path [EN §2.B; ZH §2.B: a 3x3 depth-wise conv]. D[y, x, c] = b[c] + sum_{ky, kx}
    w_dw[c, ky, kx] X[y + ky - 1, x + kx - 1, c], taps outside the map reading 0."""
    x = np.asarray(x, dtype=np.float64)
    B, H, W, C = x.shape
    w_dw = np.asarray(w_dw, dtype=np.float64)
    if w_dw.shape != (C, 3, 3):
        raise ValueError("w_dw must be [C, 3, 3]")
    xp = np.zeros((B, H + 2, W + 2, C))
    xp[:, 1:H + 1, 1:W + 1, :] = x
    d = np.zeros((B, H, W, C))
    for ky in range(3):
        for kx in range(3):
            d += w_dw[:, ky, kx] * xp[:, ky:ky + H, kx:kx + W, :]
    if b_dw is not None:
        d += np.asarray(b_dw, dtype=np.float64)
    return d


def cla_gate(x, w_dw, b_dw, w_pw, b_pw) -> np.ndarray:
    """Gating map G = sigmoid(PW_1x1(DW_3x3(X))) of the CLA path [EN §2.B: depth-wise conv, point-wise
    conv, sigmoid -> gating map; DE §2.B: G; ZH §2.B: 3x3 depth-wise, 1x1 point-wise] on a [B, H, W, C]
    map (R18). Returns G [B, H, W, C] (float64)."""
    d = cla_depthwise3x3(x, w_dw, b_dw)
    w_pw = np.asarray(w_pw, dtype=np.float64)
    C = d.shape[-1]
    if w_pw.shape != (C, C):
        raise ValueError("w_pw must be [C, C]")
    z = d @ w_pw.T
    if b_pw is not None:
        z += np.asarray(b_pw, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def cla_apply(o, g) -> np.ndarray:
    """O' = O * G [DE §2.B]: the attention output [B, H, W, heads, d_c] gated element-wise by
    G [B, H, W, heads * d_c], channel c of G on head c // d_c, channel c % d_c of O (R18)."""
    o = np.asarray(o, dtype=np.float64)
    B, H, W, heads, d_c = o.shape
    g = np.asarray(g, dtype=np.float64)
    if g.shape != (B, H, W, heads * d_c):
        raise ValueError("g must be [B, H, W, heads * d_c]")
    return o * g.reshape(B, H, W, heads, d_c)

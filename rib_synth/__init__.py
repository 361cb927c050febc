"""Seeded synthetic inputs for RIB window attention (shared by tests, bench and smoke).

This module holds none of the method's arithmetic: it only draws random
tensors and rounds them to the storage precision. Both the oracle side and the
GPU side consume the exact bits produced here.

Recipe (the pages' workloads are super-resolution feature maps computed from
image datasets that are not available; these tensors stand in for them with
the shapes and distributions of the five workloads below):

  * generator: numpy ``Generator(PCG64(seed))``
  * draw order: Q_c, K_c, V, W1, W2, then dO (backward workloads only); the
    window-size stack draws its layers in window order 16, 32, 64, 96
  * activations ~ N(0, 1) drawn in float32, rounded to bfloat16 with
    round-to-nearest-even for bf16 workloads (kept float32 for fp32 workloads)
  * MLP weights ~ N(0, 0.02^2) in float32, biases zero
  * scale = 1 / sqrt(d_c + r)
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

N_FREQ = 16
HIDDEN = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention call: feature map [B, H, W, heads, d_c], window w, rank r."""
    name: str
    B: int
    H: int
    W: int
    heads: int
    d_c: int
    w: int
    r: int
    dtype: str          # "f32" or "bf16"
    backward: bool
    seed: int
    n_freq: int = N_FREQ
    hidden: int = HIDDEN

    @property
    def N(self) -> int:
        return self.w * self.w

    @property
    def windows(self) -> int:
        return self.B * (self.H // self.w) * (self.W // self.w)

    @property
    def units(self) -> int:
        return self.windows * self.heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_c + self.r)


# The five workloads of the method's hot path. Index 3 (96x96 windows, bf16,
# forward) is the headline measurement; index 4 is the window-size stack with
# forward and backward, one Workload per layer.
WORKLOADS = {
    "w16_single_fp32": Workload("w16_single_fp32", 1, 16, 16, 1, 32, 16, 8, "f32", False, 1),
    "w32_map256_bf16": Workload("w32_map256_bf16", 1, 256, 256, 6, 32, 32, 8, "bf16", False, 2),
    "w64_map128x8_bf16": Workload("w64_map128x8_bf16", 8, 128, 128, 6, 32, 64, 16, "bf16", False, 3),
    "w96_map192x4_bf16": Workload("w96_map192x4_bf16", 4, 192, 192, 6, 32, 96, 16, "bf16", False, 4),
}
STACK_WINDOWS = (16, 32, 64, 96)
STACK = tuple(
    Workload(f"stack_w{w}_map192x2_bf16", 2, 192, 192, 6, 32, w, 16, "bf16", True, 5)
    for w in STACK_WINDOWS
)
HEADLINE = WORKLOADS["w96_map192x4_bf16"]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns."""
    u32 = bits.astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Tensor:
    """A synthetic tensor in storage precision: float32 values or bfloat16 bits."""
    dtype: str
    data: np.ndarray    # float32 array, or uint16 bf16 bit patterns

    def f64(self) -> np.ndarray:
        if self.dtype == "f32":
            return self.data.astype(np.float64)
        return bf16_to_f64(self.data)


def _activation(rng, shape, dtype) -> Tensor:
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "f32":
        return Tensor("f32", x)
    return Tensor("bf16", bf16_bits(x))


def make_inputs(wl: Workload, rng: np.random.Generator | None = None) -> dict:
    """Draw one workload's inputs in the fixed order Q_c, K_c, V, W1, W2, dO.

    Returns a dict: q_c, k_c, v (and d_o for backward workloads) as ``Tensor``;
    w1 [hidden, 4F], b1 [hidden], w2 [2r, hidden], b2 [2r] as float32 arrays.
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(wl.seed))
    shape = (wl.B, wl.H, wl.W, wl.heads, wl.d_c)
    out = {
        "q_c": _activation(rng, shape, wl.dtype),
        "k_c": _activation(rng, shape, wl.dtype),
        "v": _activation(rng, shape, wl.dtype),
    }
    out["w1"] = (0.02 * rng.standard_normal((wl.hidden, 4 * wl.n_freq), dtype=np.float32)).astype(np.float32)
    out["b1"] = np.zeros(wl.hidden, np.float32)
    out["w2"] = (0.02 * rng.standard_normal((2 * wl.r, wl.hidden), dtype=np.float32)).astype(np.float32)
    out["b2"] = np.zeros(2 * wl.r, np.float32)
    if wl.backward:
        out["d_o"] = _activation(rng, shape, wl.dtype)
    return out


def make_stack_inputs() -> list:
    """Inputs of the four stacked layers (windows 16, 32, 64, 96), drawn in that order from one stream."""
    rng = np.random.Generator(np.random.PCG64(STACK[0].seed))
    return [make_inputs(wl, rng) for wl in STACK]


def make_positional(N: int, r: int, dtype: str, seed: int, std: float = 0.5) -> tuple:
    """Random stand-in positional tokens (Q_p, K_p) of shape [N, r], for attention-only tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    qp = (std * rng.standard_normal((N, r), dtype=np.float32)).astype(np.float32)
    kp = (std * rng.standard_normal((N, r), dtype=np.float32)).astype(np.float32)
    if dtype == "f32":
        return Tensor("f32", qp), Tensor("f32", kp)
    return Tensor("bf16", bf16_bits(qp)), Tensor("bf16", bf16_bits(kp))


def make_mlp(n_freq: int, hidden: int, r: int, seed: int, std: float = 0.3, bias_std: float = 0.1) -> dict:
    """Position-MLP weights w1 [hidden, 4F], b1, w2 [2r, hidden], b2 (float32), larger than the
    workloads' N(0, 0.02^2) so that GELU is exercised away from its linear part."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return {
        "w1": (std * rng.standard_normal((hidden, 4 * n_freq))).astype(np.float32),
        "b1": (bias_std * rng.standard_normal(hidden)).astype(np.float32),
        "w2": (std * rng.standard_normal((2 * r, hidden))).astype(np.float32),
        "b2": (bias_std * rng.standard_normal(2 * r)).astype(np.float32),
    }


def make_pos_grads(N: int, r: int, seed: int) -> tuple:
    """Stand-in upstream gradients dQ_p, dK_p: float32 N(0, 1) of shape [N, r]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((N, r), dtype=np.float32), rng.standard_normal((N, r), dtype=np.float32))


def make_rpb_table(heads: int, w: int, seed: int, std: float = 1.0) -> np.ndarray:
    """Relative-position-bias tables of the RPB comparison: float32 N(0, std^2), [heads, (2w - 1)^2]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (std * rng.standard_normal((heads, (2 * w - 1) ** 2))).astype(np.float32)


def make_cla(C: int, seed: int) -> dict:
    """CLA gate weights (float32): depth-wise taps w_dw [C, 3, 3] ~ N(0, (1/3)^2) and bias b_dw [C],
    point-wise w_pw [C_out, C_in] ~ N(0, 1/C) and bias b_pw [C] (biases N(0, 0.1^2)), i.e. fan-in
    scaled so that the gate's pre-activation of an N(0, 1) map is of order 1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return {
        "w_dw": (rng.standard_normal((C, 3, 3)) / 3.0).astype(np.float32),
        "b_dw": (0.1 * rng.standard_normal(C)).astype(np.float32),
        "w_pw": (rng.standard_normal((C, C)) / np.sqrt(C)).astype(np.float32),
        "b_pw": (0.1 * rng.standard_normal(C)).astype(np.float32),
    }


def make_map(B: int, H: int, W: int, C: int, dtype: str, seed: int) -> Tensor:
    """A [B, H, W, C] N(0, 1) feature map (the CLA gate's input X)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _activation(rng, (B, H, W, C), dtype)


def custom_workload(B, H, W, heads, d_c, w, r, dtype="bf16", backward=False, seed=0,
                    n_freq=N_FREQ, hidden=HIDDEN) -> Workload:
    """A workload of arbitrary shape (small and ragged test cases)."""
    return Workload(f"custom_B{B}_H{H}_W{W}_h{heads}_d{d_c}_w{w}_r{r}_{dtype}", B, H, W, heads,
                    d_c, w, r, dtype, backward, seed, n_freq, hidden)

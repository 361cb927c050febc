"""Helpers shared by the GPU parity tests (not a test module)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import rib_synth

# Tolerances of the method's parity bar: float32 runs max-abs <= 1e-5; bfloat16
# runs max-abs <= 2e-2 and mean-abs <= 2e-3 on outputs and gradients. The
# relative-L2 bar (<= 1e-2) is this library's own, stricter for small outputs.
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
REL_L2 = 1e-2


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_gpu(t: rib_synth.Tensor, dev) -> torch.Tensor:
    if t.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(t.data)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).to(dev)


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def weights_gpu(x: dict, dev):
    return {k: torch.from_numpy(x[k]).to(dev) for k in ("w1", "b1", "w2", "b2")}


def check(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, rel_l2: float = REL_L2):
    """Element-wise comparison at the method's tolerance; NaN in ref marks entries not compared."""
    mask = ~np.isnan(ref)
    assert mask.any(), f"{name}: nothing to compare"
    g, r = got[mask], ref[mask]
    assert np.isfinite(g).all(), f"{name}: non-finite GPU values"
    err = np.abs(g - r)
    rl2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    msg = f"{name}: max-abs {err.max():.3e} mean-abs {err.mean():.3e} rel-l2 {rl2:.3e} ({g.size} values)"
    print(msg, flush=True)
    if dtype == "f32":
        assert err.max() <= F32_MAX_ABS, msg
    else:
        assert err.max() <= BF16_MAX_ABS and err.mean() <= BF16_MEAN_ABS, msg
    if rel_l2 is not None:
        assert rl2 <= rel_l2, msg
    return err.max(), err.mean(), rl2


def sample_units(wl: rib_synth.Workload, k: int, seed: int = 0, include=()):
    """k (batch, window-row, window-col, head) units spread over the map: the first and the last,
    k - 2 more drawn at random, plus the units whose flat indices are in `include` (heads
    innermost, the order the library numbers its units)."""
    all_units = [(b, wy, wx, h) for b in range(wl.B) for wy in range(wl.H // wl.w)
                 for wx in range(wl.W // wl.w) for h in range(wl.heads)]
    n = len(all_units)
    if k >= n:
        return all_units
    rng = np.random.default_rng(seed)
    rest = rng.permutation(np.arange(1, n - 1))[:max(k - 2, 0)].tolist()
    idx = {0, n - 1} | set(rest) | {int(i) for i in include}
    return [all_units[i] for i in sorted(idx)]

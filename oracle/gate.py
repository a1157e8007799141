"""Gate activation of the fused-gate entry points, in fp64 (CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written from the Ascend model file's gated paths (`_prefill_torch_kda`, the
decode branch of the attention forward, and its `_softplus` helper): the raw
gate projection plus the per-head, per-channel bias is passed through a
softplus scaled by -exp(A_log) or, when the layer has a gate lower bound,
through lower_bound * sigmoid(exp(A_log) * .); beta is the sigmoid of the raw
beta projection.  The raw inputs are taken exactly as stored (bf16 values
promoted to fp64).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def softplus(u: np.ndarray) -> np.ndarray:
    """relu(u) + log(1 + exp(-|u|)), the helper's overflow-free form."""
    return np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u)))


def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-z)), evaluated without overflow on either side."""
    ez = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + ez), ez / (1.0 + ez))


def activate(raw_g, raw_beta, a_log, dt_bias, lower_bound: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(g, beta) from raw_g [..., H, dk], raw_beta [..., H], a_log [H], dt_bias [H, dk].

    One decay per head (the Gated DeltaNet case): raw_g [..., H] with dt_bias [H].
    """
    x = _f64(raw_g)
    per_head = np.ndim(_f64(dt_bias)) == 1
    # one gate scale per head: [H] against per-head inputs, [H, 1] against channels
    scale = np.exp(_f64(a_log)) if per_head else np.exp(_f64(a_log))[:, None]
    u = x + _f64(dt_bias)                  # broadcast over the leading token axes
    if lower_bound is None:
        g = -scale * softplus(u)
    else:
        g = float(lower_bound) * sigmoid(scale * u)
    return g, sigmoid(_f64(raw_beta))

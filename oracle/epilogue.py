"""Output epilogue of the KDA layer in fp64 (CPU): gated RMSNorm over the value channels.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written from the Ascend model file's attention output path (`_project_out` with
`KimiRMSNorm`): each (token, head) row of the core output o, of length dv, is
divided by its root mean square (with eps added to the mean of squares inside
the root), multiplied by the norm weight (one value per channel) and by the
sigmoid of the output-gate projection of the same shape as o:

    y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate)

The inputs are taken exactly as stored (bf16 values promoted to fp64); the
page's intermediate roundings to the activation dtype are not modelled (the
GPU kernel rounds once, at its output).
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def gated_rmsnorm(o, gate, weight, eps: float) -> np.ndarray:
    """o, gate [..., dv]; weight [dv].  Returns y [..., dv] in fp64."""
    o, g, w = _f64(o), _f64(gate), _f64(weight)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + float(eps)) * w * (1.0 / (1.0 + np.exp(-g)))

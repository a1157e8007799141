"""Short causal convolution before the core, in fp64 (CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written from the Ascend model file's `KimiShortConvolution`: a depthwise causal
convolution over the fused q/k/v projection (one filter of `kernel_size` taps
per channel), run per request with a conv-state cache that holds each
request's last kernel_size - 1 inputs; prefill starts from the cached state
(or zeros) and leaves the request's last inputs in it, decode advances it by
one token.  With window w = [state (K-1 inputs, oldest first), x of the
request], output t is

    y[t, c] = sum_{j=0}^{K-1} W[j, c] * w[t + j, c]

so the last tap multiplies the current input.  The page passes the operator
no activation argument; `silu=True` applies z * sigmoid(z) to y.  Inputs are
taken exactly as stored (bf16 promoted to fp64).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def short_conv(x, weight, cu_seqlens, state: Optional[np.ndarray] = None,
               silu: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """x [T, C]; weight [K, C]; cu_seqlens [N+1]; state [N, K-1, C] or None (zeros).

    Returns (y [T, C], final_state [N, K-1, C]) in fp64.
    """
    x, w = _f64(x), _f64(weight)
    cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64)
    K, C = w.shape
    N = len(cu) - 1
    s0 = np.zeros((N, K - 1, C)) if state is None else _f64(state)
    y = np.zeros_like(x)
    fin = np.zeros((N, K - 1, C))
    for n in range(N):
        win = np.concatenate([s0[n], x[cu[n]:cu[n + 1]]], axis=0)  # [K-1+L, C]
        L = int(cu[n + 1] - cu[n])
        for t in range(L):
            acc = np.zeros(C)
            for j in range(K):
                acc += w[j] * win[t + j]
            y[cu[n] + t] = acc
        fin[n] = win[win.shape[0] - (K - 1):] if K > 1 else fin[n]
    if silu:
        y = y / (1.0 + np.exp(-y))
    return y, fin

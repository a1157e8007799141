"""Chunked (WY / UT-transform) form of the KDA forward in numpy fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the second executable statement of the same function as the C
recurrence.  It follows the chunk algorithm of the Ascend model file
(`_torch_chunk_kda`, the CPU fallback of the KDA prefill): per chunk of C tokens
it forms the decayed key-key matrix, inverts a unit lower-triangular system,
and carries the state across chunks.  Written here in the following notation,
per (sequence, head) and chunk with input state S (dk x dv):

    G[r]   = sum_{s<=r} g[s]                 cumulative log-decay in the chunk
    A[r,i] = beta_r * sum_c k[r,c] k[i,c] exp(G[r,c]-G[i,c])   for i < r, else 0
    P[r,i] = sum_c q[r,c] k[i,c] exp(G[r,c]-G[i,c])            for i <= r, else 0
    (I + A) Delta = diag(beta) (V - (exp(G) * K) S)            solved for Delta
    O      = (exp(G) * Q) S + P Delta
    S'     = diag(exp(G[last])) S + (K * exp(G[last]-G))^T Delta

with q, k already L2-normalised and q scaled.  The triangular system is solved
with a library routine; exp(G[r]-G[i]) is formed element by element, so no
reference point or rescaling enters.  A tail chunk simply has fewer rows.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np
from scipy.linalg import solve_triangular


def _l2n(x: np.ndarray) -> np.ndarray:
    """x / sqrt(sum(x^2) + 1e-6) along the last axis (the model file's `_l2_normalize`)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)


def _chunk_step(q, k, v, g, b, S):
    """One chunk for one head.  q, k, g: [L, dk]; v: [L, dv]; b: [L]; S: [dk, dv]."""
    L = q.shape[0]
    G = np.cumsum(g, axis=0)                                     # [L, dk]
    D = np.exp(G[:, None, :] - G[None, :, :])                    # [r, i, c] = exp(G_r - G_i)
    kk = np.einsum("rc,ic,ric->ri", k, k, np.where(np.tril(np.ones((L, L)), -1)[:, :, None] > 0, D, 0.0))
    qk = np.einsum("rc,ic,ric->ri", q, k, np.where(np.tril(np.ones((L, L)), 0)[:, :, None] > 0, D, 0.0))
    A = b[:, None] * kk                                          # strictly lower
    rhs = b[:, None] * (v - (np.exp(G) * k) @ S)
    Delta = solve_triangular(np.eye(L) + A, rhs, lower=True, unit_diagonal=True)
    O = (np.exp(G) * q) @ S + qk @ Delta
    GL = G[-1]
    S_new = np.exp(GL)[:, None] * S + (k * np.exp(GL[None, :] - G)).T @ Delta
    return O, S_new


def forward_chunked(q, k, v, g, beta, cu_seqlens, initial_state=None, scale: Optional[float] = None,
                    qk_l2norm: bool = True, chunk: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """Same contract as ``oracle.forward`` (numpy float inputs), chunk length ``chunk``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    if qk_l2norm:
        q, k = _l2n(q), _l2n(k)
    q = q * scale
    out = np.zeros((T, H, dv))
    fs = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else np.asarray(
                initial_state[n, h], dtype=np.float64).copy()
            for t0 in range(int(cu[n]), int(cu[n + 1]), chunk):
                t1 = min(t0 + chunk, int(cu[n + 1]))
                O, S = _chunk_step(q[t0:t1, h], k[t0:t1, h], v[t0:t1, h], g[t0:t1, h],
                                   beta[t0:t1, h], S)
                out[t0:t1, h] = O
            fs[n, h] = S
    return out, fs

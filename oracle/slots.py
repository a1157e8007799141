"""State-slot bookkeeping around the fp64 recurrence: pooled prefill and verify decode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Ascend model file keeps recurrent states in a cache of slots: its prefill
branch scatters each request's final state into the request's cache block
(`update_mamba_cache`), and its decode branches (`_decode_fused_kda`,
`_decode_gdr`) pass one state index per token at a fixed "Verify" width plus
the number of accepted tokens.  The page does not spell out what the decode
kernel does with those two; the reading taken here is:

* sequence n starts from the state in slot idx[a - 1], idx being its row of
  indices and a its accepted count clamped to [1, width] (1 when no counts
  are given);
* after its token t the state is stored in slot idx[t];
* an index outside [0, num_slots) names no slot: it reads as the zero state
  and nothing is stored there.

Each token is one step of the recurrence, computed by ``oracle.forward``;
what this module adds is only the gathering and scattering of states.  The
pool is taken to hold float32 values (as the device pool does).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import forward


def _valid(slot: int, num_slots: int) -> bool:
    return 0 <= slot < num_slots


def forward_pooled(q, k, v, g, beta, cu_seqlens, pool, slots, scale: Optional[float] = None,
                   qk_l2norm: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """Packed-varlen forward with the states in a pool.

    pool [P, H, dk, dv]; slots [N] int.  Sequence n starts from pool[slots[n]]
    (zero for an invalid slot) and its final state replaces that slot.
    Returns (out [T, H, dv], the updated pool), both float64.
    """
    pool = np.array(pool, dtype=np.float64)
    slots = np.asarray(slots, dtype=np.int64)
    P = pool.shape[0]
    N = slots.shape[0]
    s0 = np.zeros((N,) + pool.shape[1:], dtype=np.float64)
    for n in range(N):
        if _valid(int(slots[n]), P):
            s0[n] = pool[slots[n]]
    out, fs = forward(q, k, v, g, beta, cu_seqlens, s0, scale, qk_l2norm)
    for n in range(N):
        if _valid(int(slots[n]), P):
            pool[slots[n]] = fs[n]
    return out, pool


def verify(q, k, v, g, beta, pool, indices, accepted=None, scale: Optional[float] = None,
           qk_l2norm: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """Verify decode: ``width`` tokens per sequence with one state slot per token.

    q, k, g [N, W, H, dk]; v [N, W, H, dv]; beta [N, W, H]; pool [P, H, dk, dv];
    indices [N, W] int; accepted [N] int or None.  Returns (out [N, W, H, dv],
    the updated pool), both float64.
    """
    q, k, v, g, beta = (np.asarray(t.float().numpy() if hasattr(t, "float") else t, dtype=np.float64)
                        for t in (q, k, v, g, beta))
    pool = np.array(pool, dtype=np.float64)
    indices = np.asarray(indices, dtype=np.int64)
    N, W, H, dk = q.shape
    dv = v.shape[3]
    P = pool.shape[0]
    s0 = np.zeros((N, H, dk, dv), dtype=np.float64)
    for n in range(N):
        a = 1 if accepted is None else min(max(int(accepted[n]), 1), W)
        src = int(indices[n, a - 1])
        if _valid(src, P):
            s0[n] = pool[src]
    # The state after token t is the final state of the sequence's first t+1
    # tokens from s0, each a single fp64 run (``forward`` takes its initial
    # state in float32, so chaining one call per token would round the state
    # between tokens; the starting states come from the float32 pool).
    out = None
    for t in range(W):
        L = t + 1
        cu = np.arange(N + 1, dtype=np.int64) * L
        o, fs = forward(*(arr[:, :L].reshape(N * L, *arr.shape[2:]) for arr in (q, k, v, g, beta)), cu, s0,
                        scale, qk_l2norm)
        for n in range(N):
            dst = int(indices[n, t])
            if _valid(dst, P):
                pool[dst] = fs[n]
        if L == W:
            out = o.reshape(N, W, H, dv)
    return out, pool

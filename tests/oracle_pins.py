"""Pins that tie the CPU oracle to facts fixed outside the oracle itself.

Each ``pin_*`` takes a forward callable with the signature of
``oracle.forward`` and raises AssertionError when the pin does not hold.  The
same functions run against the real oracle (test_oracle_pins.py) and against
copies of it with a planted mistake (test_oracle_mutations.py), which must
fail at least one pin.

What each pin is anchored to:
  hand cases     -- values worked out with pen and paper (tests/golden/hand_cases.json)
  beta = 0       -- closed form: pure channel-wise decay, S_t = diag(exp(sum g)) S0
  retrieval      -- with beta = 1 and unit keys the delta rule stores v exactly
  one-hot keys   -- orthogonal keys remove the delta correction, leaving gated
                    causal linear attention, a masked matrix product
  memoryless     -- g = -60 erases the past: o_t = beta_t (q_t . k_t) v_t
  chunked form   -- the independently derived chunked algorithm (numpy)
  varlen/split   -- packing and state hand-off are plumbing identities
  linearity      -- with S0 = 0 the map V -> (O, S) is linear
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _l2n(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)


def pin_hand_cases(fwd):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float32)[:, None, :]
        k = np.array(c["k"], dtype=np.float32)[:, None, :]
        v = np.array(c["v"], dtype=np.float32)[:, None, :]
        g = np.array(c["g"], dtype=np.float32)[:, None, :]
        b = np.array(c["beta"], dtype=np.float32)[:, None]
        s0 = None if c["initial_state"] is None else np.array(c["initial_state"], np.float32)[None, None]
        cu = np.array([0, q.shape[0]])
        out, fs = fwd(q, k, v, g, b, cu, s0, scale=c["scale"], qk_l2norm=bool(c["qk_l2norm"]))
        # g = ln(1/2) is stored in float32, so exp(g) is 1/2 to ~3e-8 relative.
        _close(out[:, 0, :], c["expected_out"], 1e-6, c["name"] + " out")
        _close(fs[0, 0], c["expected_state"], 1e-6, c["name"] + " state")


def pin_l2norm_scale_closed_form(fwd):
    """T=1, S0=0: o = beta (k_hat . q_hat) v with k_hat, q_hat as defined."""
    r = _rng(1)
    dk, dv = 8, 5
    q = r.standard_normal((1, 1, dk)).astype(np.float32) * 3
    k = r.standard_normal((1, 1, dk)).astype(np.float32) * 0.5
    v = r.standard_normal((1, 1, dv)).astype(np.float32)
    g = -np.abs(r.standard_normal((1, 1, dk))).astype(np.float32)
    b = np.array([[0.7]], np.float32)
    scale = 0.37
    out, fs = fwd(q, k, v, g, b, np.array([0, 1]), None, scale=scale, qk_l2norm=True)
    qd, kd, vd = q.astype(np.float64)[0, 0], k.astype(np.float64)[0, 0], v.astype(np.float64)[0, 0]
    kh = kd / np.sqrt(kd @ kd + 1e-6)
    qh = scale * qd / np.sqrt(qd @ qd + 1e-6)
    bd = float(b[0, 0])                                       # float32(0.7), widened
    _close(out[0, 0], bd * (kh @ qh) * vd, 1e-12, "l2norm/scale out")
    _close(fs[0, 0], bd * np.outer(kh, vd), 1e-12, "l2norm/scale state")


def pin_beta_zero(fwd):
    """beta = 0: S_t = diag(exp(G_t)) S0, o_t = S0^T (exp(G_t) * q_hat_t), G_t = sum_{s<=t} g_s."""
    r = _rng(2)
    T, H, dk, dv = 23, 3, 6, 4
    q = r.standard_normal((T, H, dk)).astype(np.float32)
    k = r.standard_normal((T, H, dk)).astype(np.float32)
    v = r.standard_normal((T, H, dv)).astype(np.float32)
    g = (-0.3 * np.abs(r.standard_normal((T, H, dk)))).astype(np.float32)
    b = np.zeros((T, H), np.float32)
    s0 = r.standard_normal((1, H, dk, dv)).astype(np.float32)
    scale = 0.5
    out, fs = fwd(q, k, v, g, b, np.array([0, T]), s0, scale=scale, qk_l2norm=True)
    G = np.cumsum(g.astype(np.float64), axis=0)               # [T, H, dk]
    qh = scale * _l2n(q.astype(np.float64))
    S0 = s0.astype(np.float64)[0]                             # [H, dk, dv]
    want = np.einsum("thc,hcj->thj", np.exp(G) * qh, S0)
    _close(out, want, 1e-12, "beta=0 out")
    _close(fs[0], np.exp(G[-1])[:, :, None] * S0, 1e-12, "beta=0 state")


def pin_retrieval(fwd):
    """beta = 1 and unit-norm keys: S_t^T k_t = v_t for any decay, so q_t = k_t reads v_t."""
    r = _rng(3)
    T, H, dk, dv = 17, 2, 8, 8
    k = r.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k = k.astype(np.float32)
    q = k.copy()
    v = r.standard_normal((T, H, dv)).astype(np.float32)
    g = (-np.abs(r.standard_normal((T, H, dk)))).astype(np.float32)
    b = np.ones((T, H), np.float32)
    s0 = r.standard_normal((1, H, dk, dv)).astype(np.float32)
    scale = 0.25
    out, fs = fwd(q, k, v, g, b, np.array([0, T]), s0, scale=scale, qk_l2norm=False)
    # float32 keys have norm 1 only to ~1e-7, which enters linearly.
    _close(out, scale * v.astype(np.float64), 1e-5, "retrieval out")
    kl = k.astype(np.float64)[-1]                             # [H, dk]
    _close(np.einsum("hcj,hc->hj", fs[0], kl), v.astype(np.float64)[-1], 1e-5, "retrieval state")


def pin_one_hot_keys(fwd):
    """Distinct one-hot keys and S0 = 0: KDA equals gated causal linear attention.

    o_t = sum_{i<=t} beta_i q_t[c_i] exp(G_t[c_i] - G_i[c_i]) v_i, with key i = e_{c_i}:
    a lower-triangular mixing matrix times V.
    """
    r = _rng(4)
    H, dk, dv = 2, 16, 5
    T = 11
    q = r.standard_normal((T, H, dk)).astype(np.float32)
    v = r.standard_normal((T, H, dv)).astype(np.float32)
    g = (-0.4 * np.abs(r.standard_normal((T, H, dk)))).astype(np.float32)
    b = r.uniform(0.1, 1.0, (T, H)).astype(np.float32)
    k = np.zeros((T, H, dk), np.float32)
    ch = np.stack([r.permutation(dk)[:T] for _ in range(H)], axis=1)   # [T, H] distinct channels
    for t in range(T):
        for h in range(H):
            k[t, h, ch[t, h]] = 1.0
    scale = 1.0
    out, fs = fwd(q, k, v, g, b, np.array([0, T]), None, scale=scale, qk_l2norm=False)
    G = np.cumsum(g.astype(np.float64), axis=0)
    q, v, b = q.astype(np.float64), v.astype(np.float64), b.astype(np.float64)
    for h in range(H):
        M = np.zeros((T, T))
        for t in range(T):
            for i in range(t + 1):
                c = ch[i, h]
                M[t, i] = b[i, h] * q[t, h, c] * np.exp(G[t, h, c] - G[i, h, c])
        _close(out[:, h], M @ v[:, h].astype(np.float64), 1e-12, f"one-hot out h={h}")
        S = np.zeros((dk, dv))
        for i in range(T):
            c = ch[i, h]
            S[c] += b[i, h] * np.exp(G[-1, h, c] - G[i, h, c]) * v[i, h]
        _close(fs[0, h], S, 1e-12, f"one-hot state h={h}")


def pin_causal_linear_attention(fwd):
    """g = 0 and orthogonal one-hot keys: plain causal linear attention tril(Q K^T) diag(beta) V."""
    r = _rng(5)
    T, H, dk, dv = 9, 1, 12, 3
    q = r.standard_normal((T, H, dk)).astype(np.float32)
    v = r.standard_normal((T, H, dv)).astype(np.float32)
    g = np.zeros((T, H, dk), np.float32)
    b = r.uniform(0.1, 1.0, (T, H)).astype(np.float32)
    k = np.zeros((T, H, dk), np.float32)
    for t, c in enumerate(r.permutation(dk)[:T]):
        k[t, 0, c] = 1.0
    out, _ = fwd(q, k, v, g, b, np.array([0, T]), None, scale=1.0, qk_l2norm=False)
    Q, K, V = (x.astype(np.float64)[:, 0] for x in (q, k, v))
    want = np.tril(Q @ K.T) @ (b[:, 0:1].astype(np.float64) * V)
    _close(out[:, 0], want, 1e-12, "causal linear attention")


def pin_memoryless(fwd):
    """g = -60: exp(g) ~ 1e-26 erases the past, o_t = beta_t (q_hat_t . k_hat_t) v_t."""
    r = _rng(6)
    T, H, dk, dv = 7, 2, 8, 6
    q = r.standard_normal((T, H, dk)).astype(np.float32)
    k = r.standard_normal((T, H, dk)).astype(np.float32)
    v = r.standard_normal((T, H, dv)).astype(np.float32)
    g = np.full((T, H, dk), -60.0, np.float32)
    b = r.uniform(0.1, 1.0, (T, H)).astype(np.float32)
    s0 = r.standard_normal((1, H, dk, dv)).astype(np.float32)
    scale = 0.3
    out, fs = fwd(q, k, v, g, b, np.array([0, T]), s0, scale=scale, qk_l2norm=True)
    qh = scale * _l2n(q.astype(np.float64))
    kh = _l2n(k.astype(np.float64))
    b, v = b.astype(np.float64), v.astype(np.float64)
    want = (b[..., None] * np.sum(qh * kh, axis=-1, keepdims=True)) * v
    _close(out, want, 1e-12, "memoryless out")
    _close(fs[0], b[-1][:, None, None] * np.einsum("hc,hj->hcj", kh[-1], v[-1]),
           1e-12, "memoryless state")


def pin_chunked_agrees(fwd, lengths=(100, 37, 64, 1, 65), H=2, dk=32, dv=24, chunks=(16, 32, 64)):
    """The chunked WY form (a separate derivation) and the recurrence give the same function."""
    from oracle.chunked import forward_chunked
    r = _rng(7)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q = r.standard_normal((T, H, dk)).astype(np.float32)
    k = r.standard_normal((T, H, dk)).astype(np.float32)
    v = r.standard_normal((T, H, dv)).astype(np.float32)
    from scipy.special import log_expit
    g = log_expit(r.standard_normal((T, H, dk)) + 2.0).astype(np.float32)
    b = (1 / (1 + np.exp(-r.standard_normal((T, H))))).astype(np.float32)
    s0 = (0.1 * r.standard_normal((len(lengths), H, dk, dv))).astype(np.float32)
    out, fs = fwd(q, k, v, g, b, cu, s0, scale=None, qk_l2norm=True)
    for C in chunks:
        oc, sc = forward_chunked(q, k, v, g, b, cu, s0, chunk=C)
        _close(oc / np.abs(out).max(), out / np.abs(out).max(), 1e-12, f"chunked C={C} out")
        _close(sc / np.abs(fs).max(), fs / np.abs(fs).max(), 1e-12, f"chunked C={C} state")


def pin_varlen_and_split(fwd):
    """Packed varlen == separate runs; run(T) == run(T1) then run(T-T1) from its final state."""
    r = _rng(8)
    lengths = [13, 0, 29, 8]
    H, dk, dv = 3, 8, 8
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q = r.standard_normal((T, H, dk)).astype(np.float32)
    k = r.standard_normal((T, H, dk)).astype(np.float32)
    v = r.standard_normal((T, H, dv)).astype(np.float32)
    g = (-0.2 * np.abs(r.standard_normal((T, H, dk)))).astype(np.float32)
    b = r.uniform(0, 1, (T, H)).astype(np.float32)
    s0 = r.standard_normal((len(lengths), H, dk, dv)).astype(np.float32)
    out, fs = fwd(q, k, v, g, b, cu, s0)
    for n, L in enumerate(lengths):
        a, e = cu[n], cu[n + 1]
        o1, f1 = fwd(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], np.array([0, L]), s0[n:n + 1])
        _close(out[a:e], o1, 0.0, f"varlen seq {n} out")
        _close(fs[n], f1[0], 0.0, f"varlen seq {n} state")
        if L == 0:
            _close(fs[n], s0[n].astype(np.float64), 0.0, "empty sequence keeps its state")
    # split the third sequence at 11
    a, e, m = cu[2], cu[3], cu[2] + 11
    oa, fa = fwd(q[a:m], k[a:m], v[a:m], g[a:m], b[a:m], np.array([0, m - a]), s0[2:3])
    ob, fb = fwd(q[m:e], k[m:e], v[m:e], g[m:e], b[m:e], np.array([0, e - m]),
                 fa.astype(np.float32))
    # the hand-off state is rounded to float32 once, so agreement is to float32 precision
    _close(np.concatenate([oa, ob]), out[a:e], 1e-5, "split-call out")
    _close(fb[0], fs[2], 1e-5, "split-call state")


def pin_linearity(fwd):
    """With S0 = 0 the outputs and state are linear in V."""
    r = _rng(9)
    T, H, dk, dv = 21, 2, 8, 4
    q = r.standard_normal((T, H, dk)).astype(np.float32)
    k = r.standard_normal((T, H, dk)).astype(np.float32)
    g = (-0.3 * np.abs(r.standard_normal((T, H, dk)))).astype(np.float32)
    b = r.uniform(0, 1, (T, H)).astype(np.float32)
    # small integers, so 2 v1 - 3 v2 is exact in float32
    v1 = r.integers(-8, 9, (T, H, dv)).astype(np.float32)
    v2 = r.integers(-8, 9, (T, H, dv)).astype(np.float32)
    cu = np.array([0, T])
    o1, f1 = fwd(q, k, v1, g, b, cu, None)
    o2, f2 = fwd(q, k, v2, g, b, cu, None)
    o3, f3 = fwd(q, k, 2 * v1 - 3 * v2, g, b, cu, None)
    _close(o3, 2 * o1 - 3 * o2, 1e-12, "linearity out")
    _close(f3, 2 * f1 - 3 * f2, 1e-12, "linearity state")


ALL_PINS = [pin_hand_cases, pin_l2norm_scale_closed_form, pin_beta_zero, pin_retrieval,
            pin_one_hot_keys, pin_causal_linear_attention, pin_memoryless, pin_chunked_agrees,
            pin_varlen_and_split, pin_linearity]

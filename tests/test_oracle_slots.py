"""Pins of the state-slot oracle (oracle/slots.py) against things it does not compute itself.

* From a zero state, one step of the recurrence gives o = beta (k_hat . q_hat) v
  (the update writes k_hat beta v^T into an empty state, which is then read
  with q_hat): this fixes which slot each sequence starts from, and that a
  missing slot reads as zero.
* Every stored state equals the final state of the independent chunked
  formulation (oracle/chunked.py) run on that prefix of the sequence.
* Slots no token names keep their contents.
"""
import numpy as np
import pytest

import kda_workloads as w
from oracle import slots
from oracle.chunked import forward_chunked


def _np(t):
    return t.double().numpy()


def _zero_state_output(q, k, v, b, scale):
    qh = scale * q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + 1e-6)
    kh = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + 1e-6)
    return b[..., None] * np.sum(qh * kh, axis=-1, keepdims=True) * v


@pytest.fixture(scope="module")
def case():
    return w.make_verify(4, 3, 2, 16, dtype=w.torch.float32, extra_slots=4, seed=11)


def test_verify_starts_from_the_accepted_slot(case):
    x = case
    N, W = x.indices.shape
    idx = x.indices.numpy().copy()
    acc = np.array([1, 2, 3, 2], dtype=np.int32)
    pool = _np(x.pool).copy()
    # zero the starting slot of sequences 0 and 2 only
    for n in (0, 2):
        pool[idx[n, acc[n] - 1]] = 0.0
    out, _ = slots.verify(x.q, x.k, x.v, x.g, x.beta, pool, idx, acc, x.scale)
    ref0 = _zero_state_output(_np(x.q[:, 0]), _np(x.k[:, 0]), _np(x.v[:, 0]), _np(x.beta[:, 0]), x.scale)
    for n in range(N):
        close = np.allclose(out[n, 0], ref0[n], rtol=1e-12, atol=1e-14)
        assert close == (n in (0, 2)), n


def test_missing_slots_read_as_zero_and_are_not_written(case):
    x = case
    idx = x.indices.numpy().copy()
    P = x.pool.shape[0]
    idx[1, 0] = -1
    idx[3, 0] = P + 7
    pool_in = _np(x.pool)
    out, pool = slots.verify(x.q, x.k, x.v, x.g, x.beta, pool_in, idx, None, x.scale)
    ref0 = _zero_state_output(_np(x.q[:, 0]), _np(x.k[:, 0]), _np(x.v[:, 0]), _np(x.beta[:, 0]), x.scale)
    np.testing.assert_allclose(out[1, 0], ref0[1], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out[3, 0], ref0[3], rtol=1e-12, atol=1e-14)
    named = {int(s) for s in idx.reshape(-1) if 0 <= s < P}
    for s in range(P):
        if s not in named:
            assert np.array_equal(pool[s], pool_in[s]), s


def test_stored_states_match_the_chunked_form(case):
    x = case
    N, W = x.indices.shape
    idx = x.indices.numpy()
    acc = x.accepted.numpy()
    pool_in = _np(x.pool)
    out, pool = slots.verify(x.q, x.k, x.v, x.g, x.beta, pool_in, idx, acc, x.scale)
    for n in range(N):
        s0 = pool_in[idx[n, acc[n] - 1]][None]
        for t in range(W):
            o, fs = forward_chunked(_np(x.q[n, :t + 1]), _np(x.k[n, :t + 1]), _np(x.v[n, :t + 1]),
                                    _np(x.g[n, :t + 1]), _np(x.beta[n, :t + 1]), [0, t + 1], s0,
                                    scale=x.scale, chunk=2)
            np.testing.assert_allclose(pool[idx[n, t]], fs[0], rtol=1e-9, atol=1e-12)
            np.testing.assert_allclose(out[n, t], o[t], rtol=1e-9, atol=1e-12)


def test_accepted_counts_are_clamped(case):
    x = case
    N, W = x.indices.shape
    low = np.zeros(N, dtype=np.int32)
    high = np.full(N, W + 5, dtype=np.int32)
    o_low, p_low = slots.verify(x.q, x.k, x.v, x.g, x.beta, _np(x.pool), x.indices.numpy(), low, x.scale)
    o_one, p_one = slots.verify(x.q, x.k, x.v, x.g, x.beta, _np(x.pool), x.indices.numpy(), None, x.scale)
    o_hi, _ = slots.verify(x.q, x.k, x.v, x.g, x.beta, _np(x.pool), x.indices.numpy(), high, x.scale)
    o_w, _ = slots.verify(x.q, x.k, x.v, x.g, x.beta, _np(x.pool), x.indices.numpy(),
                          np.full(N, W, dtype=np.int32), x.scale)
    assert np.array_equal(o_low, o_one) and np.array_equal(p_low, p_one)
    assert np.array_equal(o_hi, o_w)


def test_pooled_prefill_gathers_and_scatters():
    x = w.make_prefill([5, 0, 9], 2, 16, w.torch.float32, g_mu=2.0, seed=5)
    P = 6
    gen = np.random.default_rng(3)
    pool_in = (gen.standard_normal((P, 2, 16, 16)) * 0.1).astype(np.float32).astype(np.float64)
    sl = np.array([4, 1, -1], dtype=np.int64)  # the third sequence has no slot
    out, pool = slots.forward_pooled(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool_in, sl, x.scale)
    cu = x.cu_seqlens.numpy()
    # first sequence: from slot 4, its final state back in slot 4
    o, fs = forward_chunked(_np(x.q[:5]), _np(x.k[:5]), _np(x.v[:5]), _np(x.g[:5]), _np(x.beta[:5]),
                            [0, 5], pool_in[4][None], scale=x.scale, chunk=4)
    np.testing.assert_allclose(out[:5], o, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(pool[4], fs[0], rtol=1e-9, atol=1e-12)
    # empty second sequence: its slot keeps its state
    np.testing.assert_array_equal(pool[1], pool_in[1])
    # third sequence starts from zero
    t0 = int(cu[2])
    ref0 = _zero_state_output(_np(x.q[t0]), _np(x.k[t0]), _np(x.v[t0]), _np(x.beta[t0]), x.scale)
    np.testing.assert_allclose(out[t0], ref0, rtol=1e-12, atol=1e-14)
    for s in (0, 2, 3, 5):
        np.testing.assert_array_equal(pool[s], pool_in[s])

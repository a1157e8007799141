"""Pins of the gate activation oracle (oracle/gate.py) to things other than itself.

Each check compares against a library routine (numpy's logaddexp, scipy's
expit) or a closed form, chosen so that a plausible slip fails one of them:
a dropped exp on a_log, a wrong sign, dt_bias on the wrong axis, sigmoid
in place of softplus or the reverse, or the bound applied outside the sigmoid
the wrong way round.  The activation follows the Ascend model file's gated
paths (`_prefill_torch_kda` and the decode branch of the attention forward).
"""
import math

import numpy as np
import pytest
import scipy.special as sp
import torch

from oracle import gate as G


def test_softplus_is_log_one_plus_exp():
    u = np.linspace(-60.0, 60.0, 4001)
    np.testing.assert_allclose(G.softplus(u), np.logaddexp(0.0, u), rtol=1e-14, atol=0)


def test_softplus_closed_forms():
    assert G.softplus(np.array(0.0)) == pytest.approx(math.log(2.0), rel=1e-15)
    u = np.linspace(-30.0, 30.0, 601)
    np.testing.assert_allclose(G.softplus(u) - G.softplus(-u), u, atol=1e-13)  # softplus(u) - softplus(-u) = u
    assert G.softplus(np.array(800.0)) == 800.0            # no overflow for large arguments
    assert G.softplus(np.array(-800.0)) == 0.0             # nor for very negative ones
    assert G.softplus(np.array(-30.0)) == pytest.approx(math.exp(-30.0), rel=1e-12)


def test_sigmoid_is_expit():
    z = np.linspace(-700.0, 700.0, 7001)
    np.testing.assert_allclose(G.sigmoid(z), sp.expit(z), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(G.sigmoid(z) + G.sigmoid(-z), 1.0, atol=1e-15)


def _gate_inputs(H=3, dk=5, rows=7, seed=0):
    rng = np.random.default_rng(seed)
    raw = rng.normal(-1.0, 2.0, size=(rows, H, dk))
    beta = rng.normal(0.0, 2.0, size=(rows, H))
    return raw, beta


def test_softplus_gate_scale_and_sign():
    raw, beta = _gate_inputs()
    H, dk = raw.shape[1:]
    zero = np.zeros((H, dk))
    g0, b = G.activate(raw, beta, np.zeros(H), zero)        # a_log = 0: scale exp(0) = 1
    np.testing.assert_allclose(g0, -np.logaddexp(0.0, raw), rtol=1e-14)
    np.testing.assert_allclose(b, sp.expit(beta), rtol=1e-14)
    a_log = np.log(np.array([1.0, 3.0, 16.0]))              # the gate scale is exp(a_log), per head
    g, _ = G.activate(raw, beta, a_log, zero)
    np.testing.assert_allclose(g, g0 * np.array([1.0, 3.0, 16.0])[None, :, None], rtol=1e-14)
    assert (g <= 0).all()


def test_dt_bias_is_per_head_and_channel():
    raw, beta = _gate_inputs(H=3, dk=5)
    bias = np.zeros((3, 5))
    bias[1, 3] = 0.75
    g_ref, _ = G.activate(raw, beta, np.zeros(3), np.zeros((3, 5)))
    g, _ = G.activate(raw, beta, np.zeros(3), bias)
    changed = np.abs(g - g_ref) > 0
    assert changed[:, 1, 3].all() and changed.sum() == raw.shape[0]
    shifted = raw.copy()
    shifted[:, 1, 3] += 0.75                                # the bias adds to the raw gate
    g_s, _ = G.activate(shifted, beta, np.zeros(3), np.zeros((3, 5)))
    np.testing.assert_allclose(g, g_s, rtol=1e-15)


def test_lower_bound_gate():
    raw, beta = _gate_inputs()
    H, dk = raw.shape[1:]
    zero = np.zeros((H, dk))
    g, _ = G.activate(raw, beta, np.zeros(H), zero, lower_bound=-1.0)
    np.testing.assert_allclose(g, -sp.expit(raw), rtol=1e-14)
    g2, _ = G.activate(raw, beta, np.full(H, math.log(2.0)), zero, lower_bound=-5.0)
    np.testing.assert_allclose(g2, -5.0 * sp.expit(2.0 * raw), rtol=1e-14)
    assert (g2 >= -5.0).all() and (g2 <= 0.0).all()
    mid, _ = G.activate(np.zeros((1, H, dk)), np.zeros((1, H)), np.zeros(H), zero, lower_bound=-4.0)
    np.testing.assert_allclose(mid, -2.0)                  # sigmoid(0) = 1/2
    lim, _ = G.activate(np.array([[[-1e3], [1e3]]]), np.zeros((1, 2)), np.zeros(2), np.zeros((2, 1)),
                        lower_bound=-3.0)
    assert lim[0, 0, 0] == pytest.approx(0.0, abs=1e-300) and lim[0, 1, 0] == -3.0


def test_bf16_raw_inputs_are_taken_exactly():
    raw = torch.tensor([[[0.1, -3.3]]], dtype=torch.bfloat16)
    beta = torch.tensor([[0.7]], dtype=torch.bfloat16)
    g, b = G.activate(raw, beta, np.zeros(1), np.zeros((1, 2)))
    exact = raw.double().numpy()
    np.testing.assert_allclose(g, -np.logaddexp(0.0, exact), rtol=1e-15)
    np.testing.assert_allclose(b, sp.expit(beta.double().numpy()), rtol=1e-15)


def test_per_head_activation_uses_one_scale_and_bias_per_head():
    # One decay per head (the Gated DeltaNet case): raw_g [rows, H], dt_bias [H].
    gen = np.random.default_rng(5)
    H, rows = 4, 9
    raw_g = gen.standard_normal((rows, H))
    raw_b = gen.standard_normal((rows, H))
    a_log = np.log(gen.uniform(1.0, 16.0, H))
    dt_bias = gen.standard_normal(H)
    g, b = G.activate(raw_g, raw_b, a_log, dt_bias)
    want = -np.exp(a_log)[None, :] * np.logaddexp(0.0, raw_g + dt_bias[None, :])
    np.testing.assert_allclose(g, want, rtol=1e-14)
    np.testing.assert_allclose(b, sp.expit(raw_b), rtol=1e-14)
    g2, _ = G.activate(raw_g, raw_b, a_log, dt_bias, lower_bound=-3.0)
    np.testing.assert_allclose(g2, -3.0 * sp.expit(np.exp(a_log)[None, :] * (raw_g + dt_bias[None, :])), rtol=1e-14)


def test_per_head_decay_without_updates_is_a_scalar_decay():
    # beta = 0: the state only decays, by e^{G_t} with G_t the running sum of
    # the head's scalar log-decay, so o_t = e^{G_t} S0^T q_hat_t.
    import oracle
    gen = np.random.default_rng(8)
    T, H, d = 6, 2, 8
    q = gen.standard_normal((T, H, d)).astype(np.float32)
    k = gen.standard_normal((T, H, d)).astype(np.float32)
    v = gen.standard_normal((T, H, d)).astype(np.float32)
    g = -gen.uniform(0.0, 0.5, (T, H)).astype(np.float32)
    s0 = gen.standard_normal((1, H, d, d)).astype(np.float32)
    out, fs = oracle.forward(q, k, v, g, np.zeros((T, H), np.float32), [0, T], s0, scale=0.3)
    G_t = np.cumsum(g.astype(np.float64), axis=0)                      # [T, H]
    q64 = q.astype(np.float64)
    qh = 0.3 * q64 / np.sqrt(np.sum(q64 ** 2, -1, keepdims=True) + 1e-6)
    want = np.exp(G_t)[:, :, None] * np.einsum("hcd,thc->thd", s0[0].astype(np.float64), qh)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fs[0], np.exp(G_t[-1])[:, None, None] * s0[0], rtol=1e-12, atol=1e-14)

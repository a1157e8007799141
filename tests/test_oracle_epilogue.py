"""Pins of the output-epilogue oracle (oracle/epilogue.py) against closed forms.

Each case fixes a property of y = o / sqrt(mean(o^2) + eps) * w * sigmoid(g)
that a plausible slip (mean replaced by sum, eps outside the root, the weight
or the gate dropped or applied per row, a sign) would break.
"""
import numpy as np

from oracle import epilogue


def test_hand_expanded_row():
    # o = [3, 4]: mean of squares 12.5; eps = 0.5 gives a root of exactly sqrt(13)
    o = np.array([[3.0, 4.0]])
    w = np.array([2.0, 0.5])
    g = np.array([[0.0, np.log(3.0)]])  # sigmoid: 1/2 and 3/4
    y = epilogue.gated_rmsnorm(o, g, w, eps=0.5)
    want = np.array([[3.0 / np.sqrt(13.0) * 2.0 * 0.5, 4.0 / np.sqrt(13.0) * 0.5 * 0.75]])
    assert np.allclose(y, want, rtol=1e-15, atol=0)


def test_constant_row_with_open_gate_is_unit_rms():
    # a constant row c: y = c / sqrt(c^2 + eps); with eps = 0 every entry is sign(c)
    o = np.full((3, 8), -2.5)
    y = epilogue.gated_rmsnorm(o, np.full_like(o, 60.0), np.ones(8), eps=0.0)
    assert np.allclose(y, -1.0, rtol=1e-15, atol=0)


def test_scale_invariance_without_eps():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((5, 16))
    g = rng.standard_normal((5, 16))
    w = rng.standard_normal(16)
    y1 = epilogue.gated_rmsnorm(o, g, w, eps=0.0)
    y2 = epilogue.gated_rmsnorm(7.25 * o, g, w, eps=0.0)
    assert np.allclose(y1, y2, rtol=1e-13, atol=0)


def test_rows_are_independent_and_rms_is_one():
    # with eps = 0, w = 1 and an open gate each row has a mean square of exactly one
    rng = np.random.default_rng(1)
    o = rng.standard_normal((4, 3, 64)) * np.array([1e-3, 1.0, 1e3])[None, :, None]
    y = epilogue.gated_rmsnorm(o, np.full_like(o, 60.0), np.ones(64), eps=0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-12)


def test_eps_inside_the_root():
    o = np.array([[1e-3, -1e-3]])
    y = epilogue.gated_rmsnorm(o, np.full_like(o, 60.0), np.ones(2), eps=1e-6)
    assert np.allclose(y, o / np.sqrt(1e-6 + 1e-6), rtol=1e-12)


def test_gate_and_weight_are_per_channel():
    o = np.ones((2, 4))
    g = np.array([[0.0, 60.0, -60.0, np.log(3.0)]] * 2)
    w = np.array([1.0, 2.0, 3.0, 4.0])
    y = epilogue.gated_rmsnorm(o, g, w, eps=0.0)
    want = np.array([0.5, 2.0, 3.0 / (1.0 + np.exp(60.0)), 3.0])
    assert np.allclose(y, want[None, :], rtol=1e-14)

"""Pins of the short-convolution oracle (oracle/conv.py) against closed forms.

An impulse must come out as the reversed filter (fixes the tap order and the
causal shift), one tap is a plain scaling, a split run must equal the whole run
(fixes the state plumbing), a zero state equals no state, and the activation
is z * sigmoid(z) (scipy's expit).
"""
import numpy as np
import torch
from scipy.special import expit

from oracle import conv


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def test_impulse_gives_the_reversed_filter():
    K, C, T = 4, 3, 9
    w = np.arange(1.0, 1.0 + K * C).reshape(K, C)
    x = np.zeros((T, C))
    x[2] = 1.0
    y, fin = conv.short_conv(x, w, _cu([T]), silu=False)
    for m in range(K):
        assert np.array_equal(y[2 + m], w[K - 1 - m])
    assert np.all(y[:2] == 0) and np.all(y[2 + K:] == 0)
    assert np.array_equal(fin[0], x[T - (K - 1):])


def test_one_tap_is_a_scaling():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 5))
    w = rng.standard_normal((1, 5))
    y, _ = conv.short_conv(x, w, _cu([3, 4]), silu=False)
    assert np.allclose(y, x * w[0], rtol=1e-15, atol=0)


def test_split_run_equals_whole_run():
    rng = np.random.default_rng(1)
    K, C = 4, 6
    x = rng.standard_normal((20, C))
    w = rng.standard_normal((K, C))
    s0 = rng.standard_normal((1, K - 1, C))
    y, fin = conv.short_conv(x, w, _cu([20]), s0)
    for cut in (1, 2, 3, 11):
        ya, sa = conv.short_conv(x[:cut], w, _cu([cut]), s0)
        yb, sb = conv.short_conv(x[cut:], w, _cu([20 - cut]), sa)
        assert np.allclose(np.concatenate([ya, yb]), y, rtol=1e-14, atol=1e-14)
        assert np.allclose(sb, fin, rtol=0, atol=0)


def test_requests_are_independent_and_short_ones_keep_old_state():
    rng = np.random.default_rng(2)
    K, C = 4, 2
    lens = [5, 1, 0, 2]
    x = rng.standard_normal((sum(lens), C))
    w = rng.standard_normal((K, C))
    s0 = rng.standard_normal((len(lens), K - 1, C))
    y, fin = conv.short_conv(x, w, _cu(lens), s0)
    cu = _cu(lens)
    for n, L in enumerate(lens):
        yn, fn = conv.short_conv(x[cu[n]:cu[n + 1]], w, _cu([L]), s0[n:n + 1])
        assert np.allclose(y[cu[n]:cu[n + 1]], yn) and np.allclose(fin[n], fn[0])
    # a one-token request shifts its state by one; an empty one keeps it
    assert np.array_equal(fin[1][:-1], s0[1][1:]) and np.array_equal(fin[1][-1], x[cu[1]])
    assert np.array_equal(fin[2], s0[2])


def test_zero_state_equals_no_state_and_silu():
    rng = np.random.default_rng(3)
    x = torch.randn(12, 4, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    w = rng.standard_normal((3, 4))
    y0, _ = conv.short_conv(x, w, _cu([12]), None, silu=False)
    y1, _ = conv.short_conv(x, w, _cu([12]), np.zeros((1, 2, 4)), silu=False)
    assert np.array_equal(y0, y1)
    ys, _ = conv.short_conv(x, w, _cu([12]), None, silu=True)
    assert np.allclose(ys, y0 * expit(y0), rtol=1e-15, atol=1e-300)

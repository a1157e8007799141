"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.forward)


def test_decode_is_repeated_single_token_steps():
    """The batched decode wrapper equals feeding one token at a time with the state carried."""
    import kda_workloads as w
    x = w.make_decode(3, 5, 2, 16, g_mu=2.0)
    out, fs = oracle.decode(x.q, x.k, x.v, x.g, x.beta, x.initial_state)
    S = x.initial_state.numpy()
    for t in range(x.steps):
        o, S64 = oracle.forward(x.q[t], x.k[t], x.v[t], x.g[t], x.beta[t],
                                np.arange(4), S, scale=x.scale)
        # one float32 rounding of the carried state per step
        np.testing.assert_allclose(o, out[t], rtol=0, atol=1e-6)
        S = S64.astype(np.float32)
    np.testing.assert_allclose(S, fs, rtol=0, atol=1e-6)


def test_chunked_agrees_on_tiny_fp32_workload():
    """Chunked and recurrent forms on the tiny fp32 workload (T=256, H=2, d=64), C in {16,32,64}."""
    import kda_workloads as w
    from oracle.chunked import forward_chunked
    x = w.tiny_fp32()
    out, fs = oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, None)
    for C in (16, 32, 64):
        oc, sc = forward_chunked(x.q.numpy(), x.k.numpy(), x.v.numpy(), x.g.numpy(),
                                 x.beta.numpy(), x.cu_seqlens.numpy(), None, chunk=C)
        assert np.abs(oc - out).max() / np.abs(out).max() < 1e-12
        assert np.abs(sc - fs).max() / np.abs(fs).max() < 1e-12


def test_chunked_agrees_on_kimi_shape_prefix():
    """Kimi-shaped head (d=128, g=logsigmoid(N(3,1)), bf16 inputs), T=512, 4 heads, C=64."""
    import kda_workloads as w
    from oracle.chunked import forward_chunked
    x = w.make_prefill([512], 4, 128, g_mu=3.0)
    out, fs = oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state)
    f32 = lambda t: t.float().numpy()
    oc, sc = forward_chunked(f32(x.q), f32(x.k), f32(x.v), f32(x.g), f32(x.beta),
                             x.cu_seqlens.numpy(), f32(x.initial_state), chunk=64)
    assert np.abs(oc - out).max() / np.abs(out).max() < 1e-12
    assert np.abs(sc - fs).max() / np.abs(fs).max() < 1e-12


def test_thread_count_does_not_change_result():
    """Each (sequence, head) pair runs serially, so results are bitwise stable."""
    import kda_workloads as w
    x = w.make_prefill([70, 130], 4, 32)
    a, sa = oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state)
    b, sb = oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_rejects_bad_arguments():
    q = np.zeros((4, 1, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.forward(q, q, q, q, np.zeros((4, 1), np.float32), np.array([0, 3]))
    with pytest.raises(RuntimeError):
        oracle.forward(q, q, q, q, np.zeros((4, 1), np.float32), np.array([0, 5, 4]))

"""Short causal convolution (kda_short_conv) on the GPU vs the fp64 oracle (oracle/conv.py).

Outputs: fp32 inputs within 1e-5 of max|oracle|; bf16 outputs (rounded once)
within one bf16 ulp of each oracle value plus 1e-6 of max|oracle|.  Final
states are copies of stored inputs and must match exactly.  Cases: requests
shorter than the filter, empty requests, runs of 8 tokens that cross request
boundaries, all filter lengths, with and without a starting state, SiLU on and
off, two channel blocks with a few hundred runs, in place (one token per request, and
requests of several tokens), and a split run equal to the whole run bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import conv
from tests.gpu_helpers import announce, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd  # noqa: F401  (fails loudly if libkda.so is missing)
    yield


def _inputs(lens, C, K, dtype, seed, with_state=True):
    gen = torch.Generator().manual_seed(seed)
    T, N = sum(lens), len(lens)
    x = torch.randn((T, C), generator=gen).to(dtype)
    w = (torch.randn((K, C), generator=gen) * 0.5).to(dtype)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    s0 = torch.randn((N, K - 1, C), generator=gen).to(dtype) if with_state else None
    return x, w, cu, s0


def _check(y, ys, ref, ref_s, dtype):
    g = y.double().cpu().numpy()
    m = float(np.abs(ref).max())
    if dtype == torch.float32:
        assert float(np.abs(g - ref).max()) <= 1e-5 * m
    else:
        assert bool(np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6 * m))
    if ys is not None:
        assert np.array_equal(ys.double().cpu().numpy(), ref_s)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("silu,with_state", [(True, True), (False, False)])
def test_short_conv_matches_oracle(K, dtype, silu, with_state):
    import gated_delta_rule_53_amd as kda
    lens = [0, 1, 2, 3, 17, 64, 100, 0, 15]
    x, w, cu, s0 = _inputs(lens, 384, K, dtype, seed=K * 10 + int(silu), with_state=with_state)
    announce(f"short_conv K={K} {dtype} silu={silu} state={with_state}")
    y, ys = kda.short_conv(dev(x), dev(w), dev(cu), dev(s0), silu=silu)
    torch.cuda.synchronize()
    ref, ref_s = conv.short_conv(x, w, cu.numpy(), None if s0 is None else s0, silu=silu)
    _check(y, ys if K > 1 else None, ref, ref_s, dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_short_conv_two_channel_blocks_many_runs(dtype):
    """C = 2304 spans two 2048-channel workgroup columns; 3,034 tokens are 380 runs of 8,
    dealt to the eight XCDs in contiguous ranges, with request boundaries inside runs."""
    import gated_delta_rule_53_amd as kda
    lens = [700, 0, 1, 1500, 33, 800]
    x, w, cu, s0 = _inputs(lens, 2304, 4, dtype, seed=91)
    announce(f"short_conv C=2304 T={sum(lens)} {dtype}")
    y, ys = kda.short_conv(dev(x), dev(w), dev(cu), dev(s0), silu=True)
    torch.cuda.synchronize()
    ref, ref_s = conv.short_conv(x, w, cu.numpy(), s0, silu=True)
    _check(y, ys, ref, ref_s, dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_short_conv_decode_in_place(dtype):
    import gated_delta_rule_53_amd as kda
    N, C, K = 8, 256, 4
    x, w, _, s0 = _inputs([1] * N, C, K, dtype, seed=5)
    cu = torch.arange(N + 1, dtype=torch.int32)
    announce(f"short_conv decode in place {dtype}")
    st = dev(s0)
    y, ys = kda.short_conv(dev(x), dev(w), dev(cu), st, final_state=st)
    torch.cuda.synchronize()
    ref, ref_s = conv.short_conv(x, w, cu.numpy(), s0, silu=True)
    assert ys.data_ptr() == st.data_ptr()
    _check(y, ys, ref, ref_s, dtype)


@pytest.mark.parametrize("lens", [[1, 1, 1, 1, 1, 1, 1, 2, 1, 0], [0, 5, 9, 1, 0, 30, 2, 17]],
                         ids=["T_eq_N_cross_run", "multi_token"])
@pytest.mark.parametrize("K", [2, 4])
def test_short_conv_in_place_any_lengths(lens, K):
    """In place with requests of several tokens: T == N with a 2-token request
    across the boundary of two 8-token runs (tokens 7 and 8), and a batch of
    longer requests; every request reads its old state before its new one is
    written."""
    import gated_delta_rule_53_amd as kda
    x, w, cu, s0 = _inputs(lens, 384, K, torch.float32, seed=7 + K)
    announce(f"short_conv in place lens={lens} K={K}")
    st = dev(s0)
    y, ys = kda.short_conv(dev(x), dev(w), dev(cu), st, final_state=st)
    torch.cuda.synchronize()
    ref, ref_s = conv.short_conv(x, w, cu.numpy(), s0, silu=True)
    assert ys.data_ptr() == st.data_ptr()
    _check(y, ys, ref, ref_s, torch.float32)


def test_short_conv_split_run_equals_whole_run():
    import gated_delta_rule_53_amd as kda
    x, w, cu, s0 = _inputs([300], 512, 4, torch.bfloat16, seed=6)
    announce("short_conv split run")
    d = lambda t: dev(t)
    y, ys = kda.short_conv(d(x), d(w), d(cu), d(s0))
    cut = 37
    ya, sa = kda.short_conv(d(x[:cut]), d(w), d(torch.tensor([0, cut], dtype=torch.int32)), d(s0))
    yb, sb = kda.short_conv(d(x[cut:]), d(w), d(torch.tensor([0, 300 - cut], dtype=torch.int32)), sa)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([ya, yb]), y)
    assert torch.equal(sb, ys)

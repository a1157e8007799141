"""kda_chunk_fwd_noalloc through the C ABI against kda_chunk_fwd (the entry point
it varies), on the GPU.

Both run the same kernels, the first with the library's own device array as
its workspace and the second with a workspace the caller allocates, so the
results must be identical, bit for bit; the oracle bar (2e-3 on
max|gpu - oracle| / max|oracle|) is checked as well.  Two calls in a row, the
second with a smaller input than the first (the array keeps the first call's
contents), then a problem that needs more than the array holds.
"""
import ctypes

import pytest
import torch

import kda_workloads as w
import oracle
from tests.gpu_helpers import announce, dev, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd  # noqa: F401  (fails loudly if libkda.so is missing)
    yield


def _problem(x, out_dtype):
    import gated_delta_rule_53_amd as kda
    return kda.Problem(total_tokens=x.total_tokens, num_seqs=x.num_seqs, num_heads=x.num_heads,
                       head_k=x.head_k, head_v=x.head_v, qkv_dtype=int(x.q.dtype == torch.bfloat16),
                       out_dtype=int(out_dtype == torch.bfloat16), scale=x.scale, qk_l2norm=1, chunk_size=64)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run_both(x, out_dtype=torch.float32):
    """(noalloc out, noalloc state, chunk_fwd out, chunk_fwd state) for the same inputs."""
    import gated_delta_rule_53_amd as kda
    lib = kda.raw_library()
    q, k, v, g, b, cu = (dev(t) for t in (x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens))
    s0 = dev(x.initial_state)
    prob = _problem(x, out_dtype)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    T, H, N, d = x.total_tokens, x.num_heads, x.num_seqs, x.head_k
    o1 = torch.full((T, H, d), float("nan"), dtype=out_dtype, device="cuda:0")
    f1 = torch.full((N, H, d, d), float("nan"), device="cuda:0")
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(g), _p(b), _p(cu), _p(s0),
                                   _p(o1), _p(f1), stream)
    assert st == 0, lib.kda_last_error().decode()
    o2 = torch.empty_like(o1)
    f2 = torch.empty_like(f1)
    ws_bytes = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(prob))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda:0")
    st = lib.kda_chunk_fwd(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(g), _p(b), _p(cu), _p(s0), _p(o2),
                           _p(f2), _p(ws), ws_bytes, stream)
    assert st == 0, lib.kda_last_error().decode()
    torch.cuda.synchronize()
    return o1, f1, o2, f2


def test_noalloc_matches_chunk_fwd_twice_then_smaller():
    """One sequence of 4,096 tokens at H = 32 (the 128 MiB array holds its
    workspace), then a smaller ragged batch: both identical to kda_chunk_fwd
    and within the oracle bar."""
    for x in (w.prefill_4k(), w.make_prefill([100, 64, 0, 33], 3, 128, torch.bfloat16, g_mu=2.0, seed=61)):
        announce(f"noalloc vs chunk_fwd {x.name} T={x.total_tokens} H={x.num_heads}")
        o1, f1, o2, f2 = _run_both(x)
        assert torch.equal(o1, o2) and torch.equal(f1, f2)
        ro, rs = oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state, scale=x.scale)
        eo, es = rel_err(o1, ro), rel_err(f1, rs)
        print(f"  err out {eo:.3e} state {es:.3e}")
        assert eo <= 2e-3 and es <= 2e-3, (eo, es)


def test_noalloc_paths_without_a_workspace():
    """fp32 and d = 64 inputs keep everything on chip: the array is not used."""
    for x in (w.make_prefill([90, 37], 2, 64, torch.float32, g_mu=2.0, seed=62),
              w.make_prefill([90, 37], 2, 64, torch.bfloat16, g_mu=2.0, seed=63)):
        announce(f"noalloc on-chip path {x.q.dtype} d={x.head_k}")
        o1, f1, o2, f2 = _run_both(x)
        assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_noalloc_rejects_a_problem_beyond_the_array_and_writes_nothing():
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill([4225], 32, 128, torch.bfloat16, g_mu=2.0, seed=64)
    announce("noalloc oversized problem")
    out = torch.full((x.total_tokens, 32, 128), 7.0, device="cuda:0")
    with pytest.raises(kda.KdaError) as err:
        kda.chunk_fwd_noalloc(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), dev(x.cu_seqlens), None,
                              out, None)
    assert "scratch" in str(err.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_noalloc_binding_after_other_calls():
    """The Python binding of the same entry point, after the calls above."""
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill([150, 1, 64], 2, 128, torch.bfloat16, g_mu=3.0, seed=65)
    announce("noalloc binding")
    out = torch.empty((x.total_tokens, 2, 128), dtype=torch.float32, device="cuda:0")
    fs = torch.empty((3, 2, 128, 128), device="cuda:0")
    kda.chunk_fwd_noalloc(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), dev(x.cu_seqlens),
                          dev(x.initial_state), out, fs, scale=x.scale)
    o2, f2 = kda.chunk_fwd(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), dev(x.cu_seqlens),
                           dev(x.initial_state), scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(fs, f2)

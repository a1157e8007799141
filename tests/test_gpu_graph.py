"""The library's calls captured in a HIP graph and replayed.

The calls allocate nothing, never synchronise and clear nothing with memset
(the chunk map writes every offset it later reads), so a caller may capture
them.  Each case captures one call into a torch CUDA graph, replays it several
times with eager work and synchronisations in between, and checks every replay
against the eager result, bit for bit (the same kernels on the same inputs).
"""
import pytest
import torch

import kda_workloads as w
from tests.gpu_helpers import announce, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd  # noqa: F401  (fails loudly if libkda.so is missing)
    yield


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_graph_replays_match_eager(d):
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill([100, 64, 0, 33], 3, d, torch.bfloat16, g_mu=2.0, seed=81)
    announce(f"graph prefill d={d}")
    q, k, v, g, b, cu, s0 = (dev(t) for t in (x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state))
    prob = kda.Problem(total_tokens=x.total_tokens, num_seqs=x.num_seqs, num_heads=3, head_k=d, head_v=d,
                       qkv_dtype=1, out_dtype=0, scale=x.scale, qk_l2norm=1, chunk_size=64)
    ws = torch.empty(max(kda.chunk_fwd_workspace_bytes(prob), 1), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((x.total_tokens, 3, d), dtype=torch.float32, device="cuda:0")
    fs = torch.empty_like(s0)
    ref_o, ref_s = kda.chunk_fwd(q, k, v, g, b, cu, s0, scale=x.scale, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        kda.chunk_fwd(q, k, v, g, b, cu, s0, scale=x.scale, out_dtype=torch.float32, out=out, final_state=fs,
                      workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.chunk_fwd(q, k, v, g, b, cu, s0, scale=x.scale, out_dtype=torch.float32, out=out, final_state=fs,
                      workspace=ws)
    for rep in range(4):
        out.fill_(float("nan"))
        fs.fill_(float("nan"))
        ws.fill_(0xAB)  # the workspace is rebuilt by every call
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {rep}: out differs"
        assert torch.equal(fs, ref_s), f"replay {rep}: final state differs"


def test_decode_graph_replays_match_eager():
    """A captured step advances the in-place state exactly as eager steps do."""
    import gated_delta_rule_53_amd as kda
    x = w.make_decode(8, 4, 2, 128, torch.bfloat16, seed=82)
    announce("graph decode")
    q, k, v, g, b = (dev(t[0]) for t in (x.q, x.k, x.v, x.g, x.beta))
    st_eager = dev(x.initial_state)
    st_graph = dev(x.initial_state)
    out_e = torch.empty((8, 2, 128), dtype=torch.float32, device="cuda:0")
    out_g = torch.empty_like(out_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    warm = st_graph.clone()
    with torch.cuda.stream(side):
        kda.recurrent_step(q, k, v, g, b, warm, scale=x.scale, out_dtype=torch.float32, out=out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.recurrent_step(q, k, v, g, b, st_graph, scale=x.scale, out_dtype=torch.float32, out=out_g)
    for rep in range(4):
        kda.recurrent_step(q, k, v, g, b, st_eager, scale=x.scale, out_dtype=torch.float32, out=out_e)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}: out differs"
        assert torch.equal(st_graph, st_eager), f"replay {rep}: state differs"


def _capture(fn):
    """Warm fn up on a side stream, then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


def test_conv_prefill_graph_replays_match_eager():
    """kda_chunk_fwd_conv (the convolution fused into the prefill, conv state
    updated in a separate buffer) captured and replayed."""
    import gated_delta_rule_53_amd as kda
    x = w.make_conv_prefill([100, 2, 0, 70], 2, 128, 4, seed=83)
    announce("graph conv prefill")
    xx, g, b, wt, cu, s0, cs = (dev(t) for t in (x.x, x.g, x.beta, x.weight, x.cu_seqlens, x.initial_state,
                                                  x.conv_state))
    T, N = x.x.shape[0], len(x.cu_seqlens) - 1
    prob = kda.Problem(total_tokens=T, num_seqs=N, num_heads=2, head_k=128, head_v=128, qkv_dtype=1, out_dtype=0,
                       scale=x.scale, qk_l2norm=1, chunk_size=64)
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(prob), dtype=torch.uint8, device="cuda:0")
    ref_cs = torch.empty_like(cs)
    ref_o, ref_s = kda.chunk_fwd_conv(xx, g, b, wt, cu, s0, cs, conv_state_out=ref_cs, scale=x.scale,
                                      out_dtype=torch.float32, workspace=ws)
    out = torch.empty_like(ref_o)
    fs = torch.empty_like(ref_s)
    cs_out = torch.empty_like(cs)
    graph = _capture(lambda: kda.chunk_fwd_conv(xx, g, b, wt, cu, s0, cs, conv_state_out=cs_out, scale=x.scale,
                                                out_dtype=torch.float32, out=out, final_state=fs, workspace=ws))
    for rep in range(4):
        out.fill_(float("nan"))
        fs.fill_(float("nan"))
        cs_out.zero_()
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {rep}: out differs"
        assert torch.equal(fs, ref_s), f"replay {rep}: final state differs"
        assert torch.equal(cs_out, ref_cs), f"replay {rep}: conv state differs"


def test_verify_normed_graph_replays_match_eager():
    """kda_recurrent_verify_normed captured and replayed (the pool is restored
    before each replay: the call writes the per-token states into it)."""
    import gated_delta_rule_53_amd as kda
    x = w.make_verify(6, 3, 2, 128, torch.bfloat16, g_mu=2.0, pad=1, seed=84)
    announce("graph verify normed")
    gen = torch.Generator().manual_seed(85)
    og = dev(torch.randn(tuple(x.v.shape), generator=gen).to(torch.bfloat16))
    nw = dev(1.0 + 0.1 * torch.randn((128,), generator=gen))
    q, k, v, g, b, idx, acc = (dev(t) for t in (x.q, x.k, x.v, x.g, x.beta, x.indices, x.accepted))
    pool0 = dev(x.pool)
    pool = pool0.clone()
    ref_o = kda.recurrent_verify_normed(q, k, v, g, b, pool, idx, og, nw, acc, scale=x.scale,
                                        out_dtype=torch.float32)
    ref_pool = pool.clone()
    out = torch.empty_like(ref_o)
    pool.copy_(pool0)
    graph = _capture(lambda: kda.recurrent_verify_normed(q, k, v, g, b, pool, idx, og, nw, acc, scale=x.scale,
                                                         out_dtype=torch.float32, out=out))
    for rep in range(4):
        pool.copy_(pool0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {rep}: out differs"
        assert torch.equal(pool, ref_pool), f"replay {rep}: pool differs"

"""HIP path vs the CPU oracle, element by element, through the C ABI.

Error metric: max|gpu - oracle| / max|oracle| per tensor.  Bar: 2e-3 for bf16
inputs, 1e-4 for fp32 inputs, on outputs (taken in fp32) and final states.
bf16 outputs are checked to be within one bf16 ulp of the fp32-mode output.
"""
import numpy as np
import pytest
import torch

import kda_workloads as w
import oracle
from tests.gpu_helpers import announce, dev, prefill_on_gpu, rel_err, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd  # noqa: F401  (fails loudly if libkda.so is missing)
    yield


def _oracle_prefill(x, with_state=True):
    return oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens,
                          x.initial_state if with_state else None, scale=x.scale)


def _check_prefill(x, with_state=True, out_dtype=torch.float32):
    announce(f"prefill {x.name} T={x.total_tokens} N={x.num_seqs} H={x.num_heads} "
             f"d={x.head_k} qkv={x.q.dtype} out={out_dtype} state={with_state}")
    out, fs = prefill_on_gpu(x, out_dtype=out_dtype, with_state=with_state)
    ref_o, ref_s = _oracle_prefill(x, with_state)
    tol = tol_for(x.q.dtype)
    eo, es = rel_err(out, ref_o), rel_err(fs, ref_s)
    print(f"  err out {eo:.3e} state {es:.3e} (tol {tol:.0e})")
    assert eo <= tol and es <= tol, (eo, es)
    return out, fs


# ----------------------------------------------------------------- prefill

def test_prefill_tiny_fp32_workload():
    """T=256, H=2, d=64, fp32, zero initial state, tolerance 1e-4."""
    _check_prefill(w.tiny_fp32(), with_state=False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_prefill_ragged(d, dtype):
    """Ragged lengths around the chunk size, an empty sequence, several chunks."""
    x = w.make_prefill([1, 63, 64, 65, 0, 130, 200], 3, d, dtype, g_mu=2.0, seed=11)
    _check_prefill(x)


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_many_short_sequences(d):
    """1,500 sequences of 0-70 tokens: more sequences than the device-side chunk
    map sorts (it then keeps their order and sums chunk counts over two passes),
    many empty sequences, and more state tiles than compute units (the d=128
    scan then takes two value tiles per workgroup)."""
    gen = torch.Generator().manual_seed(23)
    lens = torch.randint(0, 71, (1500,), generator=gen).tolist()
    lens[:3] = [0, 64, 65]
    x = w.make_prefill(lens, 2, d, torch.bfloat16, g_mu=2.0, seed=24, name=f"many_short_d{d}")
    _check_prefill(x)


def test_prefill_without_initial_state():
    x = w.make_prefill([97, 256], 2, 128, torch.bfloat16, g_mu=3.0, state_std=None, seed=12)
    _check_prefill(x, with_state=False)


def test_prefill_strong_decay():
    """g = logsigmoid(N(0,1)): per-chunk decay sums near -50, far below the workloads'."""
    x = w.make_prefill([192, 77], 2, 128, torch.bfloat16, g_mu=0.0, seed=13)
    _check_prefill(x)


def test_prefill_bf16_output_is_rounded_fp32_output():
    x = w.make_prefill([150, 64], 2, 128, torch.bfloat16, g_mu=2.0, seed=14)
    o32, s32 = prefill_on_gpu(x, out_dtype=torch.float32)
    o16, s16 = prefill_on_gpu(x, out_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    a, b = o16.float(), o32
    # one bf16 ulp: 2^-7 relative to the leading power of two
    ulp = torch.exp2(torch.floor(torch.log2(b.abs().clamp_min(1e-30))) - 7)
    assert bool(((a - b).abs() <= ulp).all())
    assert torch.equal(s16, s32)


def test_prefill_no_l2norm_with_unit_inputs():
    """qk_l2norm = 0 with keys and queries already of unit norm."""
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill([130], 2, 128, torch.float32, g_mu=2.0, seed=15)
    x.k = x.k / x.k.norm(dim=-1, keepdim=True)
    x.q = x.q / x.q.norm(dim=-1, keepdim=True)
    announce("prefill no-l2norm")
    out, fs = kda.chunk_fwd(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), dev(x.cu_seqlens),
                            dev(x.initial_state), scale=0.5, qk_l2norm=False)
    ro, rs = oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state, scale=0.5,
                            qk_l2norm=False)
    assert rel_err(out, ro) <= 1e-4 and rel_err(fs, rs) <= 1e-4


def test_prefill_deterministic():
    x = w.make_prefill([300, 45], 4, 128, torch.bfloat16, seed=16)
    announce("prefill determinism")
    o1, s1 = prefill_on_gpu(x)
    o2, s2 = prefill_on_gpu(x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_prefill_split_call_composition():
    """Running T tokens at once equals T1 tokens, then T-T1 more from the returned state."""
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill([250], 2, 128, torch.bfloat16, seed=17)
    announce("prefill split composition")
    q, k, v, g, b = (dev(t) for t in (x.q, x.k, x.v, x.g, x.beta))
    s0 = dev(x.initial_state)
    full_o, full_s = kda.chunk_fwd(q, k, v, g, b, None, s0, out_dtype=torch.float32)
    T1 = 100  # not a chunk multiple: the second call re-chunks from token 100
    o1, s1 = kda.chunk_fwd(q[:T1].contiguous(), k[:T1].contiguous(), v[:T1].contiguous(),
                           g[:T1].contiguous(), b[:T1].contiguous(), None, s0, out_dtype=torch.float32)
    o2, s2 = kda.chunk_fwd(q[T1:].contiguous(), k[T1:].contiguous(), v[T1:].contiguous(),
                           g[T1:].contiguous(), b[T1:].contiguous(), None, s1, out_dtype=torch.float32)
    ref_o, ref_s = _oracle_prefill(x)
    assert rel_err(torch.cat([o1, o2]), ref_o) <= 2e-3
    assert rel_err(s2, ref_s) <= 2e-3
    assert rel_err(s2, full_s.double().cpu().numpy()) <= 2e-3


def test_prefill_final_state_may_alias_initial_state():
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill([70, 129], 2, 128, torch.bfloat16, seed=18)
    announce("prefill state alias")
    ref_o, ref_s = _oracle_prefill(x)
    st = dev(x.initial_state).clone()
    out, fs = kda.chunk_fwd(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), dev(x.cu_seqlens),
                            st, final_state=st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert fs.data_ptr() == st.data_ptr()
    assert rel_err(out, ref_o) <= 2e-3 and rel_err(st, ref_s) <= 2e-3


def test_prefill_zero_tokens_keeps_states():
    import gated_delta_rule_53_amd as kda
    H, d = 2, 128
    s0 = torch.randn(3, H, d, d, device="cuda:0")
    e = torch.empty(0, H, d, device="cuda:0", dtype=torch.bfloat16)
    ef = torch.empty(0, H, d, device="cuda:0")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    announce("prefill zero tokens")
    out, fs = kda.chunk_fwd(e, e, e, ef, torch.empty(0, H, device="cuda:0"), cu, s0)
    torch.cuda.synchronize()
    assert out.shape == (0, H, d) and torch.equal(fs, s0)


def test_prefill_then_decode_continues_the_sequence():
    """Prefill of T tokens then one decode step == the oracle over T+1 tokens."""
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill([129], 2, 128, torch.bfloat16, seed=19)
    announce("prefill then decode")
    T = 128
    q, k, v, g, b = (dev(t) for t in (x.q, x.k, x.v, x.g, x.beta))
    _, st = kda.chunk_fwd(q[:T].contiguous(), k[:T].contiguous(), v[:T].contiguous(),
                          g[:T].contiguous(), b[:T].contiguous(), None, dev(x.initial_state))
    o = kda.recurrent_step(q[T:], k[T:], v[T:], g[T:], b[T:], st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_o, ref_s = _oracle_prefill(x)
    assert rel_err(o, ref_o[T:]) <= 2e-3
    assert rel_err(st, ref_s) <= 2e-3


# ------------------------------------------------------ full-size workloads

def test_prefill_4k_workload():
    """B=1, T=4096, H=32, d=128, bf16, g=logsigmoid(N(3,1)), S0 ~ N(0, 0.01^2): every element."""
    _check_prefill(w.prefill_4k())


def test_prefill_varlen8_workload():
    """8 packed sequences of U{512..8192} tokens, H=32, d=128: every element."""
    _check_prefill(w.varlen8())


def test_prefill_long_128k_workload():
    """T=131072, H=32, d=128: every output and the whole final state of all 32
    heads against the oracle.  The oracle runs over groups of 16 heads (heads
    are independent) to bound host memory; the error metric is taken over the
    whole tensors: max over groups of max|gpu - oracle|, over max|oracle|."""
    x = w.long_128k()
    announce(f"prefill {x.name} (all heads)")
    out, fs = prefill_on_gpu(x, out_dtype=torch.float32, with_state=False)
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(fs).all())
    out_c, fs_c = out.cpu(), fs.cpu()
    del out, fs
    err_o = err_s = den_o = den_s = 0.0
    H, G = x.num_heads, 16
    for h0 in range(0, H, G):
        sl = lambda t: t[:, h0:h0 + G].contiguous()
        ro, rs = oracle.forward(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), x.cu_seqlens,
                                None, scale=x.scale)
        go = out_c[:, h0:h0 + G].double().numpy()
        gs = fs_c[:, h0:h0 + G].double().numpy()
        err_o = max(err_o, float(np.abs(go - ro).max()))
        err_s = max(err_s, float(np.abs(gs - rs).max()))
        den_o = max(den_o, float(np.abs(ro).max()))
        den_s = max(den_s, float(np.abs(rs).max()))
        print(f"  heads {h0}..{h0 + G - 1} checked", flush=True)
        del ro, rs, go, gs
    eo, es = err_o / den_o, err_s / den_s
    print(f"  err out {eo:.3e} state {es:.3e}")
    assert eo <= 2e-3 and es <= 2e-3, (eo, es)


# ------------------------------------------------------------------ decode

def _decode_on_gpu(x, out_dtype=torch.float32):
    import gated_delta_rule_53_amd as kda
    q, k, v, g, b = (dev(t) for t in (x.q, x.k, x.v, x.g, x.beta))
    st = dev(x.initial_state).clone()
    outs = [kda.recurrent_step(q[t], k[t], v[t], g[t], b[t], st, scale=x.scale, out_dtype=out_dtype)
            for t in range(x.steps)]
    torch.cuda.synchronize()
    return torch.stack(outs), st


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_decode_small(d, dtype):
    x = w.make_decode(5, 7, 3, d, dtype, g_mu=2.0, seed=21)
    announce(f"decode small d={d} {dtype}")
    out, st = _decode_on_gpu(x)
    ro, rs = oracle.decode(x.q, x.k, x.v, x.g, x.beta, x.initial_state, scale=x.scale)
    tol = tol_for(dtype)
    assert rel_err(out, ro) <= tol and rel_err(st, rs) <= tol


def test_decode_bf16_output_is_rounded_fp32_output():
    x = w.make_decode(4, 3, 2, 128, torch.bfloat16, seed=22)
    o32, s32 = _decode_on_gpu(x, torch.float32)
    o16, s16 = _decode_on_gpu(x, torch.bfloat16)
    ulp = torch.exp2(torch.floor(torch.log2(o32.abs().clamp_min(1e-30))) - 7)
    assert bool(((o16.float() - o32).abs() <= ulp).all())
    assert torch.equal(s16, s32)


def test_decode_256x64_workload():
    """256 sequences x 64 steps, H=32, d=128, bf16: all 64 outputs and the final states."""
    x = w.decode_256x64()
    announce(f"decode {x.name}")
    out, st = _decode_on_gpu(x)
    ro, rs = oracle.decode(x.q, x.k, x.v, x.g, x.beta, x.initial_state, scale=x.scale)
    eo, es = rel_err(out, ro), rel_err(st, rs)
    print(f"  err out {eo:.3e} state {es:.3e}")
    assert eo <= 2e-3 and es <= 2e-3


@pytest.mark.parametrize("H", [2, 40], ids=["lane_map", "map_kernel"])
def test_prefill_malformed_cu_seqlens(H):
    """Entries outside [0, T] and a decreasing pair make their sequences empty:
    no out-of-bounds access, their final states equal their initial states, no
    output row outside the well-formed sequences is written, and the
    well-formed sequences match the oracle.  H=2: the kernels compute the chunk
    map themselves; H=40: more tiles than CUs, the chunk-map kernel and the
    two-tile scan."""
    import gated_delta_rule_53_amd as kda
    T, d = 300, 128
    x = w.make_prefill([T], H, d, torch.bfloat16, g_mu=2.0, seed=31, name="malformed_cu")
    cu = torch.tensor([-10, 100, 160, 250, 400, 300], dtype=torch.int32)
    N = cu.numel() - 1
    gen = torch.Generator().manual_seed(32)
    s0 = torch.randn((N, H, d, d), generator=gen) * 0.01
    announce(f"prefill malformed cu_seqlens H={H}")
    out = torch.full((T, H, d), float("nan"), device="cuda:0")
    out, fs = kda.chunk_fwd(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), dev(cu), dev(s0),
                            scale=x.scale, out=out, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, s = out.cpu(), fs.cpu()
    for n in (0, 3, 4):
        assert torch.equal(s[n], s0[n]), n
    assert torch.isnan(o[:100]).all() and torch.isnan(o[250:]).all()
    rows = slice(100, 250)
    ref_o, ref_s = oracle.forward(x.q[rows], x.k[rows], x.v[rows], x.g[rows], x.beta[rows],
                                  torch.tensor([0, 60, 150], dtype=torch.int32), s0[1:3], scale=x.scale)
    eo, es = rel_err(out[rows], ref_o), rel_err(fs[1:3], ref_s)
    print(f"  err out {eo:.3e} state {es:.3e}")
    assert eo <= 2e-3 and es <= 2e-3, (eo, es)

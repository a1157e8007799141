"""State-pool calls on the GPU vs the slot oracle (oracle/slots.py).

kda_recurrent_verify (verify decode, one state slot per token, accepted
counts) and kda_chunk_fwd_pooled (prefill that reads and writes its states in
pool slots).  Bars as everywhere: max|gpu - oracle| / max|oracle| <= 2e-3
(bf16 inputs), 1e-4 (fp32 inputs), on outputs and on the written slots;
slots the call does not name must come back bit for bit.  Cases cover padded
(-1) and out-of-range indices, both head sizes, the two-pass bf16 d=128 prefill
with one and with two value tiles per workgroup (40 chains > 32), the on-chip
prefill, empty sequences, the fused gate and windows of up to 12 tokens; a
bf16 output must equal the fp32 output rounded to nearest even, bit for bit.
"""
import numpy as np
import pytest
import torch

import kda_workloads as w
from oracle import gate as ogate
from oracle import slots as oslots
from tests.gpu_helpers import announce, dev, rel_err, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd  # noqa: F401  (fails loudly if libkda.so is missing)
    yield


def _check_pool(pool_gpu, pool_ref, pool_in, named, tol):
    g = pool_gpu.cpu().numpy()
    P = pool_in.shape[0]
    written = sorted(s for s in named if 0 <= s < P)
    untouched = [s for s in range(P) if s not in set(written)]
    for s in untouched:
        assert np.array_equal(g[s], pool_in[s]), f"slot {s} changed"
    es = rel_err(pool_gpu[written], pool_ref[written]) if written else 0.0
    assert es <= tol, es
    return es


# (N, W, H, d, dtype, with accepted counts, padded slots, one index past the pool)
VERIFY_CASES = [
    (8, 4, 4, 128, torch.bfloat16, True, 3, False),
    (5, 3, 2, 64, torch.float32, False, 0, True),
    (6, 1, 3, 128, torch.bfloat16, False, 1, False),
    (4, 5, 2, 64, torch.bfloat16, True, 0, True),
    (3, 2, 2, 128, torch.float32, True, 1, False),
    (3, 12, 2, 128, torch.bfloat16, True, 2, True),   # wider windows: the loop's one-token-ahead loads
    (2, 9, 2, 64, torch.float32, True, 1, False),
]


@pytest.mark.parametrize("N,W,H,d,dtype,acc,pad,past", VERIFY_CASES)
def test_verify(N, W, H, d, dtype, acc, pad, past):
    import gated_delta_rule_53_amd as kda
    x = w.make_verify(N, W, H, d, dtype, g_mu=2.0, pad=pad, seed=41 + N + W)
    idx = x.indices.clone()
    P = x.pool.shape[0]
    if past:
        idx[0, -1] = P + 3
    accepted = x.accepted if acc else None
    announce(f"verify N={N} W={W} H={H} d={d} {dtype} accepted={acc} pad={pad} past={past}")
    pool = dev(x.pool.clone())
    out = kda.recurrent_verify(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), pool, dev(idx),
                               dev(accepted), scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rp = oslots.verify(x.q, x.k, x.v, x.g, x.beta, x.pool.double().numpy(), idx.numpy(),
                           None if accepted is None else accepted.numpy(), x.scale)
    tol = tol_for(dtype)
    eo = rel_err(out, ro)
    es = _check_pool(pool, rp, x.pool.numpy(), idx.reshape(-1).tolist(), tol)
    print(f"  err out {eo:.3e} state {es:.3e} (tol {tol:.0e})")
    assert eo <= tol, eo


@pytest.mark.parametrize("lb,mu", [(None, -5.0), (-5.0, -2.0)])
def test_verify_gated(lb, mu):
    import gated_delta_rule_53_amd as kda
    N, W, H, d = 4, 3, 2, 128
    x = w.make_verify(N, W, H, d, torch.bfloat16, pad=1, seed=47)
    gi = w.make_gate(W, H, d, torch.bfloat16, mu=mu, lower_bound=lb, seed=48, lead=(N,))
    announce(f"verify gated N={N} W={W} H={H} d={d} lower_bound={lb}")
    pool = dev(x.pool.clone())
    out = kda.recurrent_verify(dev(x.q), dev(x.k), dev(x.v), dev(gi.raw_g), dev(gi.raw_beta), pool,
                               dev(x.indices), dev(x.accepted), a_log=dev(gi.a_log), dt_bias=dev(gi.dt_bias),
                               lower_bound=lb, scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    g, b = ogate.activate(gi.raw_g, gi.raw_beta, gi.a_log, gi.dt_bias, lb)
    ro, rp = oslots.verify(x.q, x.k, x.v, g, b, x.pool.double().numpy(), x.indices.numpy(), x.accepted.numpy(),
                           x.scale)
    tol = tol_for(torch.bfloat16)
    eo = rel_err(out, ro)
    es = _check_pool(pool, rp, x.pool.numpy(), x.indices.reshape(-1).tolist(), tol)
    print(f"  err out {eo:.3e} state {es:.3e} (tol {tol:.0e})")
    assert eo <= tol, eo


# (lengths, heads, d, dtype, slots, pool size)
POOLED_CASES = [
    ([100, 0, 65], 3, 128, torch.bfloat16, [4, 1, -1], 6),
    ([90, 37], 2, 64, torch.float32, [1, 0], 3),
    ([70, 130, 33, 64, 9], 8, 128, torch.bfloat16, [6, 2, 0, 9, 4], 7),
    ([64, 1], 2, 64, torch.bfloat16, [0, 2], 3),
]


@pytest.mark.parametrize("lens,H,d,dtype,sl,P", POOLED_CASES)
def test_prefill_pooled(lens, H, d, dtype, sl, P):
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill(lens, H, d, dtype, g_mu=2.0, seed=51)
    gen = torch.Generator().manual_seed(52)
    pool_in = torch.randn((P, H, d, d), generator=gen) * 0.01
    slots = torch.tensor(sl, dtype=torch.int32)
    announce(f"prefill pooled lens={lens} H={H} d={d} {dtype} slots={sl} P={P}")
    pool = dev(pool_in.clone())
    out = kda.chunk_fwd_pooled(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), pool, dev(slots),
                               dev(x.cu_seqlens), scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rp = oslots.forward_pooled(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool_in.double().numpy(),
                                   slots.numpy(), x.scale)
    tol = tol_for(dtype)
    eo = rel_err(out, ro)
    es = _check_pool(pool, rp, pool_in.numpy(), sl, tol)
    print(f"  err out {eo:.3e} state {es:.3e} (tol {tol:.0e})")
    assert eo <= tol, eo


def test_prefill_pooled_gated():
    import gated_delta_rule_53_amd as kda
    lens, H, d, P = [100, 64], 3, 128, 4
    x = w.make_prefill(lens, H, d, torch.bfloat16, g_mu=2.0, seed=55)
    gi = w.make_gate(x.total_tokens, H, d, torch.bfloat16, mu=-5.0, seed=56)
    pool_in = torch.randn((P, H, d, d), generator=torch.Generator().manual_seed(57)) * 0.01
    slots = torch.tensor([3, 0], dtype=torch.int32)
    announce(f"prefill pooled gated lens={lens} H={H} d={d}")
    pool = dev(pool_in.clone())
    out = kda.chunk_fwd_pooled(dev(x.q), dev(x.k), dev(x.v), dev(gi.raw_g), dev(gi.raw_beta), pool, dev(slots),
                               dev(x.cu_seqlens), a_log=dev(gi.a_log), dt_bias=dev(gi.dt_bias), scale=x.scale,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    g, b = ogate.activate(gi.raw_g, gi.raw_beta, gi.a_log, gi.dt_bias, None)
    ro, rp = oslots.forward_pooled(x.q, x.k, x.v, g, b, x.cu_seqlens, pool_in.double().numpy(), slots.numpy(),
                                   x.scale)
    tol = tol_for(torch.bfloat16)
    eo = rel_err(out, ro)
    es = _check_pool(pool, rp, pool_in.numpy(), [3, 0], tol)
    print(f"  err out {eo:.3e} state {es:.3e} (tol {tol:.0e})")
    assert eo <= tol, eo


# (N, W, H, d, dtype, state layout, raw gate)
VERIFY_NORMED_CASES = [
    (8, 4, 4, 128, torch.bfloat16, "dk_dv", False),
    (5, 3, 2, 64, torch.float32, "dv_dk", False),
    (4, 2, 2, 128, torch.bfloat16, "dv_dk", True),
    (3, 5, 2, 64, torch.bfloat16, "dk_dv", True),
]


@pytest.mark.parametrize("N,W,H,d,dtype,layout,raw", VERIFY_NORMED_CASES)
def test_verify_normed(N, W, H, d, dtype, layout, raw):
    """Verify decode with the output epilogue fused: outputs against the slot
    oracle followed by the epilogue oracle; the pool must equal the plain
    verify call's pool bit for bit (the same state arithmetic)."""
    import gated_delta_rule_53_amd as kda
    from oracle import epilogue
    x = w.make_verify(N, W, H, d, dtype, g_mu=2.0, pad=1, seed=53 + N + W)
    gen = torch.Generator().manual_seed(54 + d)
    og = torch.randn((N, W, H, d), generator=gen).to(dtype)
    nw = 1.0 + 0.1 * torch.randn((d,), generator=gen)
    announce(f"verify normed N={N} W={W} H={H} d={d} {dtype} layout={layout} raw_gate={raw}")
    pool_in = x.pool if layout == "dk_dv" else x.pool.transpose(-1, -2).contiguous()
    if raw:
        gi = w.make_gate(W, H, d, dtype, mu=-5.0, seed=55, lead=(N,))
        g_in, b_in = gi.raw_g, gi.raw_beta
        kw = dict(a_log=dev(gi.a_log), dt_bias=dev(gi.dt_bias))
        g_act, b_act = ogate.activate(gi.raw_g, gi.raw_beta, gi.a_log, gi.dt_bias, None)
    else:
        g_in, b_in, kw = x.g, x.beta, {}
        g_act, b_act = x.g, x.beta
    common = dict(scale=x.scale, state_layout=layout, out_dtype=torch.float32, **kw)
    pool, pool_plain = dev(pool_in.clone()), dev(pool_in.clone())
    args = (dev(x.q), dev(x.k), dev(x.v), dev(g_in), dev(b_in))
    y = kda.recurrent_verify_normed(*args, pool, dev(x.indices), dev(og), dev(nw), dev(x.accepted),
                                    norm_eps=1e-6, **common)
    kda.recurrent_verify(*args, pool_plain, dev(x.indices), dev(x.accepted), **common)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool_plain)
    ro, _ = oslots.verify(x.q, x.k, x.v, g_act, b_act, x.pool.double().numpy(), x.indices.numpy(),
                          x.accepted.numpy(), x.scale)
    ref = epilogue.gated_rmsnorm(ro, og, nw, 1e-6)
    err = rel_err(y, ref)
    print(f"  err {err:.3e}")
    assert err <= tol_for(dtype), err


@pytest.mark.parametrize("layout", ["dk_dv", "dv_dk"])
@pytest.mark.parametrize("normed", [False, True])
def test_verify_bf16_out_is_rounded_fp32_out(layout, normed):
    """The bf16 output is the fp32 output rounded to nearest even, bit for bit,
    and the written pool is the same: the output's dtype changes only its final
    rounding and store (the bench runs verify with bf16 outputs)."""
    import gated_delta_rule_53_amd as kda
    N, W, H, d = 6, 6, 4, 128
    x = w.make_verify(N, W, H, d, torch.bfloat16, g_mu=2.0, pad=1, seed=61)
    gen = torch.Generator().manual_seed(62)
    og = torch.randn((N, W, H, d), generator=gen).to(torch.bfloat16)
    nw = 1.0 + 0.1 * torch.randn((d,), generator=gen)
    announce(f"verify bf16 vs fp32 output layout={layout} normed={normed}")
    pool_in = x.pool if layout == "dk_dv" else x.pool.transpose(-1, -2).contiguous()
    args = (dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta))
    ys, pools = {}, {}
    for od in (torch.float32, torch.bfloat16):
        pool = dev(pool_in.clone())
        common = dict(scale=x.scale, state_layout=layout, out_dtype=od)
        if normed:
            ys[od] = kda.recurrent_verify_normed(*args, pool, dev(x.indices), dev(og), dev(nw), dev(x.accepted),
                                                 norm_eps=1e-6, **common)
        else:
            ys[od] = kda.recurrent_verify(*args, pool, dev(x.indices), dev(x.accepted), **common)
        pools[od] = pool
    torch.cuda.synchronize()
    assert ys[torch.bfloat16].dtype == torch.bfloat16
    assert torch.equal(pools[torch.float32], pools[torch.bfloat16])
    assert torch.equal(ys[torch.bfloat16], ys[torch.float32].to(torch.bfloat16))

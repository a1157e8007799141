"""One decay per head (the Gated DeltaNet case) on the GPU vs the oracle.

g is [rows, H] (or the raw gate [rows, H] with dt_bias [H]); the oracle
broadcasts it over the key channels, which is what the per-head decay means,
and runs the same fp64 recurrence.  Bars as everywhere: 2e-3 (bf16 inputs),
1e-4 (fp32 inputs), on outputs and final states.  Cases cover the two-pass
bf16 d=128 prefill, the on-chip prefill, decode, verify decode and the pooled
prefill, with activated and with raw gates.
"""
import pytest
import torch

import kda_workloads as w
import oracle
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


@pytest.mark.parametrize("lens,H,d,dtype", [
    ([100, 64, 33], 3, 128, torch.bfloat16),
    ([90, 37], 2, 64, torch.float32),
    ([70, 1], 2, 64, torch.bfloat16),
])
def test_prefill_per_head(lens, H, d, dtype):
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill(lens, H, d, dtype, seed=61)
    g = w.per_head_decay((x.total_tokens, H), 2.0, seed=62)
    announce(f"prefill per-head lens={lens} H={H} d={d} {dtype}")
    out, fs = kda.chunk_fwd(dev(x.q), dev(x.k), dev(x.v), dev(g), dev(x.beta), dev(x.cu_seqlens),
                            dev(x.initial_state), scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rs = oracle.forward(x.q, x.k, x.v, g, x.beta, x.cu_seqlens, x.initial_state, scale=x.scale)
    tol = tol_for(dtype)
    eo, es = rel_err(out, ro), rel_err(fs, rs)
    print(f"  err out {eo:.3e} state {es:.3e} (tol {tol:.0e})")
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("d,dtype,lb,mu", [(128, torch.bfloat16, None, -5.0), (64, torch.float32, -3.0, -2.0)])
def test_prefill_gated_per_head(d, dtype, lb, mu):
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill([100, 65], 2, d, dtype, seed=63)
    gi = w.make_gate(x.total_tokens, 2, d, dtype, mu=mu, lower_bound=lb, seed=64, per_head=True)
    announce(f"prefill gated per-head d={d} {dtype} lower_bound={lb}")
    out, fs = kda.chunk_fwd_gated(dev(x.q), dev(x.k), dev(x.v), dev(gi.raw_g), dev(gi.raw_beta), dev(gi.a_log),
                                  dev(gi.dt_bias), dev(x.cu_seqlens), dev(x.initial_state), lower_bound=lb,
                                  scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    g, b = ogate.activate(gi.raw_g, gi.raw_beta, gi.a_log, gi.dt_bias, lb)
    ro, rs = oracle.forward(x.q, x.k, x.v, g, b, x.cu_seqlens, x.initial_state, scale=x.scale)
    tol = tol_for(dtype)
    eo, es = rel_err(out, ro), rel_err(fs, rs)
    print(f"  err out {eo:.3e} state {es:.3e} (tol {tol:.0e})")
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("d,dtype,gated", [(128, torch.bfloat16, False), (64, torch.float32, False),
                                          (128, torch.bfloat16, True)])
def test_decode_per_head(d, dtype, gated):
    import gated_delta_rule_53_amd as kda
    N, H, steps = 6, 3, 3
    x = w.make_decode(N, steps, H, d, dtype, seed=65)
    state = dev(x.initial_state.clone())
    announce(f"decode per-head d={d} {dtype} gated={gated}")
    if gated:
        gi = w.make_gate(N, H, d, dtype, seed=66, lead=(steps,), per_head=True)
        g, b = ogate.activate(gi.raw_g, gi.raw_beta, gi.a_log, gi.dt_bias)
    else:
        g, b = w.per_head_decay((steps, N, H), 2.0, seed=66), x.beta
    outs = []
    for t in range(steps):
        if gated:
            outs.append(kda.recurrent_step_gated(dev(x.q[t]), dev(x.k[t]), dev(x.v[t]), dev(gi.raw_g[t]),
                                                 dev(gi.raw_beta[t]), dev(gi.a_log), dev(gi.dt_bias), state,
                                                 scale=x.scale, out_dtype=torch.float32))
        else:
            outs.append(kda.recurrent_step(dev(x.q[t]), dev(x.k[t]), dev(x.v[t]), dev(g[t]), dev(b[t]), state,
                                           scale=x.scale, out_dtype=torch.float32))
    torch.cuda.synchronize()
    ro, rs = oracle.decode(x.q, x.k, x.v, g, b, x.initial_state, scale=x.scale)
    tol = tol_for(dtype)
    eo, es = rel_err(torch.stack(outs), ro), rel_err(state, rs)
    print(f"  err out {eo:.3e} state {es:.3e} (tol {tol:.0e})")
    assert eo <= tol and es <= tol, (eo, es)


def test_verify_and_pooled_per_head():
    import gated_delta_rule_53_amd as kda
    N, W, H, d = 4, 3, 2, 128
    x = w.make_verify(N, W, H, d, torch.bfloat16, pad=1, seed=67)
    g = w.per_head_decay((N, W, H), 2.0, seed=68)
    announce("verify per-head")
    pool = dev(x.pool.clone())
    out = kda.recurrent_verify(dev(x.q), dev(x.k), dev(x.v), dev(g), dev(x.beta), pool, dev(x.indices),
                               dev(x.accepted), scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rp = oslots.verify(x.q, x.k, x.v, g, x.beta, x.pool.double().numpy(), x.indices.numpy(),
                           x.accepted.numpy(), x.scale)
    eo = rel_err(out, ro)
    named = sorted(s for s in x.indices.reshape(-1).tolist() if s >= 0)
    es = rel_err(pool[named], rp[named])
    print(f"  verify err out {eo:.3e} state {es:.3e}")
    assert eo <= 2e-3 and es <= 2e-3, (eo, es)

    p = w.make_prefill([80, 40], H, d, torch.bfloat16, seed=69)
    gp = w.per_head_decay((p.total_tokens, H), 2.0, seed=70)
    pool_in = torch.randn((3, H, d, d), generator=torch.Generator().manual_seed(71)) * 0.01
    slots = torch.tensor([2, 0], dtype=torch.int32)
    announce("pooled prefill per-head")
    pool2 = dev(pool_in.clone())
    out2 = kda.chunk_fwd_pooled(dev(p.q), dev(p.k), dev(p.v), dev(gp), dev(p.beta), pool2, dev(slots),
                                dev(p.cu_seqlens), scale=p.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro2, rp2 = oslots.forward_pooled(p.q, p.k, p.v, gp, p.beta, p.cu_seqlens, pool_in.double().numpy(),
                                     slots.numpy(), p.scale)
    eo2, es2 = rel_err(out2, ro2), rel_err(pool2[[0, 2]], rp2[[0, 2]])
    print(f"  pooled err out {eo2:.3e} state {es2:.3e}")
    assert eo2 <= 2e-3 and es2 <= 2e-3, (eo2, es2)
    assert torch.equal(pool2[1].cpu(), pool_in[1])

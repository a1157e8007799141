"""Fused gate activation on the GPU vs the oracle (activation in fp64, then the recurrence).

The reference applies oracle.gate.activate to the raw inputs exactly as
stored and feeds the activated g and beta to the recurrence oracle (which
takes float32 inputs: the fp64 g is rounded to float32 there, a relative
change near 6e-8, far below the bars).  Bars as for the ungated path:
max|gpu - oracle| / max|oracle| <= 2e-3 (bf16 inputs), 1e-4 (fp32 inputs),
on outputs and final states.  Cases cover both gate forms, the two-pass bf16
d=128 path (ragged tails included), the on-chip path (fp32 and bf16, d=64)
and decode.
"""
import numpy as np
import pytest
import torch

import kda_workloads as w
import oracle
from oracle import gate as ogate
from tests.gpu_helpers import announce, dev, rel_err, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd  # noqa: F401  (fails loudly if libkda.so is missing)
    yield


# (lengths, heads, d, dtype, lower_bound, raw-gate mean): the softplus gate draws its raw
# gate near -5 and the bounded gate near -2, mild decays that keep every chunk on the
# factored path; tests/test_gpu_domain.py takes the page's gate initialisation, whose
# decays send chunks to the exact path.
PREFILL_CASES = [
    ([100, 64, 33], 3, 128, torch.bfloat16, None, -5.0),
    ([100, 64, 33], 3, 128, torch.bfloat16, -5.0, -2.0),
    ([1, 127, 65, 0, 200], 2, 128, torch.bfloat16, None, -5.0),
    ([90, 37], 2, 64, torch.float32, None, -5.0),
    ([90, 37], 2, 64, torch.float32, -3.0, -2.0),
    ([70, 64], 2, 64, torch.bfloat16, -5.0, -2.0),
]


@pytest.mark.parametrize("lens,H,d,dtype,lb,mu", PREFILL_CASES)
def test_prefill_gated(lens, H, d, dtype, lb, mu):
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill(lens, H, d, dtype, g_mu=2.0, seed=31)
    gi = w.make_gate(x.total_tokens, H, d, dtype, mu=mu, lower_bound=lb, seed=32)
    announce(f"prefill gated lens={lens} H={H} d={d} {dtype} lower_bound={lb}")
    out, fs = kda.chunk_fwd_gated(dev(x.q), dev(x.k), dev(x.v), dev(gi.raw_g), dev(gi.raw_beta),
                                  dev(gi.a_log), dev(gi.dt_bias), dev(x.cu_seqlens), dev(x.initial_state),
                                  lower_bound=lb, scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    g, b = ogate.activate(gi.raw_g, gi.raw_beta, gi.a_log, gi.dt_bias, lb)
    ro, rs = oracle.forward(x.q, x.k, x.v, g, b, x.cu_seqlens, x.initial_state, scale=x.scale)
    tol = tol_for(dtype)
    eo, es = rel_err(out, ro), rel_err(fs, rs)
    print(f"  err out {eo:.3e} state {es:.3e} (tol {tol:.0e})")
    assert eo <= tol and es <= tol, (eo, es)


def test_prefill_gated_matches_ungated_with_activated_inputs_in_float32():
    """Same kernels, gate activated outside (fp64, rounded to float32): the two calls agree.

    The two g differ in the last float32 bit at most, which can flip the
    rounding of fp16 operands inside the bf16 path, so the bar is a quarter
    of that path's tolerance rather than float32 rounding.
    """
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill([130, 66], 2, 128, torch.bfloat16, g_mu=2.0, seed=33)
    gi = w.make_gate(x.total_tokens, 2, 128, torch.bfloat16, mu=-5.0, seed=34)
    announce("prefill gated vs ungated with activated inputs")
    args = (dev(x.cu_seqlens), dev(x.initial_state))
    o1, s1 = kda.chunk_fwd_gated(dev(x.q), dev(x.k), dev(x.v), dev(gi.raw_g), dev(gi.raw_beta),
                                 dev(gi.a_log), dev(gi.dt_bias), *args, scale=x.scale, out_dtype=torch.float32)
    g, b = ogate.activate(gi.raw_g, gi.raw_beta, gi.a_log, gi.dt_bias)
    o2, s2 = kda.chunk_fwd(dev(x.q), dev(x.k), dev(x.v), dev(torch.from_numpy(g).float()),
                           dev(torch.from_numpy(b).float()), *args, scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_err(o1, o2.double().cpu().numpy()) <= 5e-4
    assert rel_err(s1, s2.double().cpu().numpy()) <= 5e-4


@pytest.mark.parametrize("d,dtype,lb,mu", [
    (128, torch.bfloat16, None, -5.0),
    (128, torch.bfloat16, -5.0, -2.0),
    (64, torch.float32, None, -5.0),
    (64, torch.float32, -3.0, -2.0),
])
def test_decode_gated(d, dtype, lb, mu):
    import gated_delta_rule_53_amd as kda
    x = w.make_decode(5, 6, 3, d, dtype, g_mu=2.0, seed=35)  # 5 sequences, 6 steps
    gi = w.make_gate(5, 3, d, dtype, mu=mu, lower_bound=lb, seed=36, lead=(6,))
    announce(f"decode gated d={d} {dtype} lower_bound={lb}")
    q, k, v, rg, rb = (dev(t) for t in (x.q, x.k, x.v, gi.raw_g, gi.raw_beta))
    a_log, dt_bias = dev(gi.a_log), dev(gi.dt_bias)
    st = dev(x.initial_state).clone()
    outs = [kda.recurrent_step_gated(q[t], k[t], v[t], rg[t], rb[t], a_log, dt_bias, st, lower_bound=lb,
                                     scale=x.scale, out_dtype=torch.float32) for t in range(x.steps)]
    torch.cuda.synchronize()
    g, b = ogate.activate(gi.raw_g, gi.raw_beta, gi.a_log, gi.dt_bias, lb)
    ro, rs = oracle.decode(x.q, x.k, x.v, g, b, x.initial_state, scale=x.scale)
    tol = tol_for(dtype)
    eo, es = rel_err(torch.stack(outs), ro), rel_err(st, rs)
    print(f"  err out {eo:.3e} state {es:.3e} (tol {tol:.0e})")
    assert eo <= tol and es <= tol, (eo, es)

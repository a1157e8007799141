"""Decode with the output epilogue fused (kda_recurrent_step_normed) vs the oracle.

The reference is the fp64 decode oracle followed by the fp64 epilogue oracle
(oracle/epilogue.py).  Bars: 2e-3 (bf16 inputs) / 1e-4 (fp32 inputs) of
max|oracle| on the normed outputs (fp32); the state must equal the plain decode
step's state bit for bit (the same kernel arithmetic).  Cases: both head sizes,
both state layouts, activated and raw gates, one decay per head; and a bf16
output equal, bit for bit, to the fp32 output rounded to nearest even.
"""
import pytest
import torch

import kda_workloads as w
import oracle
from oracle import epilogue
from oracle import gate as ogate
from tests.gpu_helpers import announce, dev, rel_err, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd  # noqa: F401  (fails loudly if libkda.so is missing)
    yield


def tr(t):
    return t.transpose(-1, -2).contiguous()


@pytest.mark.parametrize("d,dtype,layout,raw", [
    (128, torch.bfloat16, "dk_dv", False),
    (64, torch.float32, "dv_dk", False),
    (128, torch.bfloat16, "dv_dk", True),
    (64, torch.bfloat16, "dk_dv", True),
])
def test_decode_normed(d, dtype, layout, raw):
    import gated_delta_rule_53_amd as kda
    N, H = 6, 3
    x = w.make_decode(N, 1, H, d, dtype, seed=101 + d)
    gen = torch.Generator().manual_seed(102)
    og = torch.randn((N, H, d), generator=gen).to(dtype)
    nw = 1.0 + 0.1 * torch.randn((d,), generator=gen)
    announce(f"decode normed d={d} {dtype} layout={layout} raw_gate={raw}")
    s0 = x.initial_state if layout == "dk_dv" else tr(x.initial_state)
    st, st_plain = dev(s0), dev(s0)
    if raw:
        gi = w.make_gate(1, H, d, dtype, mu=-5.0, seed=103, lead=(N,))
        g_in, b_in = gi.raw_g[:, 0], gi.raw_beta[:, 0]
        kw = dict(a_log=dev(gi.a_log), dt_bias=dev(gi.dt_bias))
        g_act, b_act = ogate.activate(gi.raw_g, gi.raw_beta, gi.a_log, gi.dt_bias, None)
        g_act, b_act = g_act.reshape(1, N, H, d), b_act.reshape(1, N, H)
        plain = lambda s: kda.recurrent_step_gated(dev(x.q[0]), dev(x.k[0]), dev(x.v[0]), dev(g_in), dev(b_in),
                                                   dev(gi.a_log), dev(gi.dt_bias), s, scale=x.scale,
                                                   out_dtype=torch.float32, state_layout=layout)
    else:
        g_in, b_in = x.g[0], x.beta[0]
        kw = {}
        g_act, b_act = x.g, x.beta
        plain = lambda s: kda.recurrent_step(dev(x.q[0]), dev(x.k[0]), dev(x.v[0]), dev(g_in), dev(b_in), s,
                                             scale=x.scale, out_dtype=torch.float32, state_layout=layout)
    y = kda.recurrent_step_normed(dev(x.q[0]), dev(x.k[0]), dev(x.v[0]), dev(g_in), dev(b_in), st, dev(og),
                                  dev(nw), norm_eps=1e-6, scale=x.scale, state_layout=layout,
                                  out_dtype=torch.float32, **kw)
    plain(st_plain)
    torch.cuda.synchronize()
    assert torch.equal(st, st_plain)
    ro, _ = oracle.decode(x.q, x.k, x.v, g_act, b_act, x.initial_state, scale=x.scale)
    ref = epilogue.gated_rmsnorm(ro[0], og, nw, 1e-6)
    err = rel_err(y, ref)
    print(f"  err {err:.3e}")
    assert err <= tol_for(dtype), err


@pytest.mark.parametrize("layout", ["dk_dv", "dv_dk"])
@pytest.mark.parametrize("normed", [False, True])
def test_decode_bf16_out_is_rounded_fp32_out(layout, normed):
    """A bf16 decode output is the fp32 output rounded to nearest even, bit for
    bit, with the same updated state (the output dtype changes only the final
    rounding and store)."""
    import gated_delta_rule_53_amd as kda
    N, H, d = 8, 4, 128
    x = w.make_decode(N, 1, H, d, torch.bfloat16, seed=111)
    gen = torch.Generator().manual_seed(112)
    og = torch.randn((N, H, d), generator=gen).to(torch.bfloat16)
    nw = 1.0 + 0.1 * torch.randn((d,), generator=gen)
    announce(f"decode bf16 vs fp32 output layout={layout} normed={normed}")
    s0 = x.initial_state if layout == "dk_dv" else tr(x.initial_state)
    args = (dev(x.q[0]), dev(x.k[0]), dev(x.v[0]), dev(x.g[0]), dev(x.beta[0]))
    ys, states = {}, {}
    for od in (torch.float32, torch.bfloat16):
        st = dev(s0)
        if normed:
            ys[od] = kda.recurrent_step_normed(*args, st, dev(og), dev(nw), norm_eps=1e-6, scale=x.scale,
                                               state_layout=layout, out_dtype=od)
        else:
            ys[od] = kda.recurrent_step(*args, st, scale=x.scale, state_layout=layout, out_dtype=od)
        states[od] = st
    torch.cuda.synchronize()
    assert ys[torch.bfloat16].dtype == torch.bfloat16
    assert torch.equal(states[torch.float32], states[torch.bfloat16])
    assert torch.equal(ys[torch.bfloat16], ys[torch.float32].to(torch.bfloat16))

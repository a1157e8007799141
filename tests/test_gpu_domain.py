"""Strong decay: chunks whose log-decay is too steep for one reference token.

The chunk form needs e^{G_r - G_i} for i <= r inside a chunk (the Ascend
Kimi-Linear model file, `_torch_chunk_kda`, forms it element by element).
The kernels factor it through a reference token while every factor stays
inside the float range, and otherwise carry k_i e^{G_r - G_i} down the rows
by products of e^{g} <= 1.  These cases reach the second path (and mix both
in one call) on both prefill paths: the two-pass bf16 d=128 path and the
on-chip fp32 / d=64 path.  Bars as everywhere: max|gpu - oracle| /
max|oracle| <= 2e-3 for bf16 inputs and 1e-4 for fp32 inputs, on outputs and
final states.

Gates come from the page's initialisation (`KimiDeltaAttention.__init__`:
A_log = log U(1, 16), here also fixed at log 16) with a zero dt_bias and raw
gates ~ N(0, 1): about -13 per token for A = 16, so a half chunk sums to
several hundred.
"""
import math

import pytest
import torch

import kda_workloads as w
import oracle
from oracle import gate as ogate
from tests.gpu_helpers import announce, dev, prefill_on_gpu, rel_err, tol_for

pytestmark = pytest.mark.gpu

PATHS = [(128, torch.bfloat16), (64, torch.bfloat16), (64, torch.float32), (128, torch.float32)]
PATH_IDS = ["bf16_d128", "bf16_d64", "f32_d64", "f32_d128"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd  # noqa: F401  (fails loudly if libkda.so is missing)
    yield


def _check(out, fs, ro, rs, dtype):
    tol = tol_for(dtype)
    eo, es = rel_err(out, ro), rel_err(fs, rs)
    print(f"  err out {eo:.3e} state {es:.3e} (tol {tol:.0e})")
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("d,dtype", PATHS, ids=PATH_IDS)
def test_memoryless_decay(d, dtype):
    """g = -60 everywhere: each token forgets everything before it (o_t is
    beta_t (q_hat_t . k_hat_t) v_t up to e^-60)."""
    x = w.make_prefill([1, 63, 64, 65, 130, 0, 7], 2, d, dtype, seed=41)
    x.g.fill_(-60.0)
    announce(f"prefill memoryless g=-60 d={d} {dtype}")
    out, fs = prefill_on_gpu(x)
    ro, rs = oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state, scale=x.scale)
    _check(out, fs, ro, rs, dtype)


@pytest.mark.parametrize("d,dtype", PATHS, ids=PATH_IDS)
def test_mixed_heads_fast_and_exact(d, dtype):
    """One call whose heads take both paths: heads with g = logsigmoid(N(3, 1))
    stay on the factored path, heads with g = logsigmoid(N(-8, 1)) (about -8
    per token) leave it, and a ragged tail cuts the last chunk short."""
    x = w.make_prefill([200, 77, 64], 4, d, dtype, g_mu=3.0, seed=42)
    gen = torch.Generator().manual_seed(43)
    strong = torch.nn.functional.logsigmoid(torch.randn(x.g[:, 1::2].shape, generator=gen) - 8.0)
    x.g[:, 1::2] = strong
    announce(f"prefill mixed heads d={d} {dtype}")
    out, fs = prefill_on_gpu(x)
    ro, rs = oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state, scale=x.scale)
    _check(out, fs, ro, rs, dtype)


@pytest.mark.parametrize("d,dtype", PATHS, ids=PATH_IDS)
def test_reference_span_threshold(d, dtype):
    """Decays just either side of where the bf16 d=128 path leaves its reference
    token: a constant g per head makes each 32-token half of a full chunk span
    32 |g|, and the limit there is 60 (|g| = 1.875).  Heads at |g| = 1.85 and
    1.87 stay on the factored path with factors near e^60, heads at 1.88 and
    1.95 take the exact one; the 24-token sequence's chunk spans at most 24 |g|
    and stays factored in every head.  Every head must meet the bar on both
    sides."""
    x = w.make_prefill([128, 24, 64], 4, d, dtype, seed=49)
    for h, gv in enumerate((-1.85, -1.87, -1.88, -1.95)):
        x.g[:, h] = gv
    announce(f"prefill reference-span threshold d={d} {dtype}")
    out, fs = prefill_on_gpu(x)
    ro, rs = oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state, scale=x.scale)
    _check(out, fs, ro, rs, dtype)


@pytest.mark.parametrize("d,dtype", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("a_log_value", [math.log(16.0), None], ids=["A16", "A_U1_16"])
def test_page_softplus_gate(d, dtype, a_log_value):
    """Softplus gate, A_log = log 16 (or log U(1, 16) per head), dt_bias = 0,
    raw gate ~ N(0, 1)."""
    import gated_delta_rule_53_amd as kda
    H = 4
    x = w.make_prefill([150, 64, 33], H, d, dtype, seed=44)
    gi = w.make_gate(x.total_tokens, H, d, dtype, mu=0.0, std=1.0, dt_std=0.0, a_log_value=a_log_value,
                     seed=45)
    announce(f"prefill page softplus gate d={d} {dtype} a_log={a_log_value}")
    out, fs = kda.chunk_fwd_gated(dev(x.q), dev(x.k), dev(x.v), dev(gi.raw_g), dev(gi.raw_beta),
                                  dev(gi.a_log), dev(gi.dt_bias), dev(x.cu_seqlens), dev(x.initial_state),
                                  scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    g, b = ogate.activate(gi.raw_g, gi.raw_beta, gi.a_log, gi.dt_bias)
    ro, rs = oracle.forward(x.q, x.k, x.v, g, b, x.cu_seqlens, x.initial_state, scale=x.scale)
    _check(out, fs, ro, rs, dtype)


@pytest.mark.parametrize("d,dtype", PATHS, ids=PATH_IDS)
def test_bounded_gate_saturated(d, dtype):
    """Bounded gate at lower_bound = -5 with raw gates ~ N(6, 1) and A = 16: the
    sigmoid saturates, so g is -5 on almost every token."""
    import gated_delta_rule_53_amd as kda
    H = 3
    x = w.make_prefill([129, 64, 1], H, d, dtype, seed=46)
    gi = w.make_gate(x.total_tokens, H, d, dtype, mu=6.0, std=1.0, a_log_value=math.log(16.0),
                     lower_bound=-5.0, seed=47)
    announce(f"prefill bounded gate saturated d={d} {dtype}")
    out, fs = kda.chunk_fwd_gated(dev(x.q), dev(x.k), dev(x.v), dev(gi.raw_g), dev(gi.raw_beta),
                                  dev(gi.a_log), dev(gi.dt_bias), dev(x.cu_seqlens), dev(x.initial_state),
                                  lower_bound=-5.0, scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    g, b = ogate.activate(gi.raw_g, gi.raw_beta, gi.a_log, gi.dt_bias, -5.0)
    assert float(g.max()) > -5.0 - 1e-6 and float(g.mean()) < -4.9
    ro, rs = oracle.forward(x.q, x.k, x.v, g, b, x.cu_seqlens, x.initial_state, scale=x.scale)
    _check(out, fs, ro, rs, dtype)


@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float32)], ids=["bf16_d128", "f32_d64"])
def test_per_head_decay_strong(d, dtype):
    """One decay per head (the Gated DeltaNet case) at -40 per token."""
    import gated_delta_rule_53_amd as kda
    x = w.make_prefill([100, 64], 2, d, dtype, seed=48)
    gh = torch.full((x.total_tokens, 2), -40.0)
    announce(f"prefill per-head decay -40 d={d} {dtype}")
    out, fs = kda.chunk_fwd(dev(x.q), dev(x.k), dev(x.v), dev(gh), dev(x.beta), dev(x.cu_seqlens),
                            dev(x.initial_state), scale=x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rs = oracle.forward(x.q, x.k, x.v, gh, x.beta, x.cu_seqlens, x.initial_state, scale=x.scale)
    _check(out, fs, ro, rs, dtype)

"""Output epilogue (kda_gated_rmsnorm) on the GPU vs the fp64 oracle (oracle/epilogue.py).

Bars as for the core: max|gpu - oracle| / max|oracle| <= 2e-3 for bf16 inputs
and 1e-4 for fp32 inputs, on float32 outputs; a bf16 output is within one bf16
ulp of rounding the float32-mode output.  Shapes cover both head sizes, a row
count that leaves the last workgroup partly empty, and in-place use.
"""
import pytest
import torch

from oracle import epilogue
from tests.gpu_helpers import announce, dev, rel_err, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_53_amd  # noqa: F401  (fails loudly if libkda.so is missing)
    yield


def _inputs(T, H, dv, dtype, seed):
    gen = torch.Generator().manual_seed(seed)
    o = (torch.randn((T, H, dv), generator=gen) * 0.3).to(dtype)
    gate = torch.randn((T, H, dv), generator=gen).to(dtype)
    weight = 1.0 + 0.1 * torch.randn((dv,), generator=gen)
    return o, gate, weight


@pytest.mark.parametrize("T,H,dv", [(1000, 3, 128), (77, 5, 64), (1, 1, 128), (4096, 32, 128)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_gated_rmsnorm_matches_oracle(T, H, dv, dtype):
    import gated_delta_rule_53_amd as kda
    o, gate, weight = _inputs(T, H, dv, dtype, seed=T + H + dv)
    announce(f"gated_rmsnorm T={T} H={H} dv={dv} {dtype}")
    y = kda.gated_rmsnorm(dev(o), dev(gate), dev(weight), eps=1e-6, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = epilogue.gated_rmsnorm(o, gate, weight, 1e-6)
    err = rel_err(y, ref)
    print(f"  err {err:.3e}")
    assert err <= tol_for(dtype), err


def test_gated_rmsnorm_bf16_output_is_rounded_fp32_output():
    import gated_delta_rule_53_amd as kda
    o, gate, weight = _inputs(300, 4, 128, torch.bfloat16, seed=90)
    y32 = kda.gated_rmsnorm(dev(o), dev(gate), dev(weight), eps=1e-5, out_dtype=torch.float32)
    y16 = kda.gated_rmsnorm(dev(o), dev(gate), dev(weight), eps=1e-5)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16
    diff = (y16.float() - y32.to(torch.bfloat16).float()).abs()
    ulp = y32.abs().clamp_min(1e-30) * 2.0 ** -7
    assert bool((diff <= ulp).all())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_gated_rmsnorm_in_place(dtype):
    import gated_delta_rule_53_amd as kda
    o, gate, weight = _inputs(513, 2, 64, dtype, seed=91)
    od = dev(o)
    ref = kda.gated_rmsnorm(od, dev(gate), dev(weight), eps=1e-6)
    kda.gated_rmsnorm(od, dev(gate), dev(weight), eps=1e-6, out=od)
    torch.cuda.synchronize()
    assert torch.equal(od, ref)

"""KDA_DEBUG=1: every call synchronises its stream and reports kernel errors.

Runs in a child process (the library reads the variable once): a prefill on
each path, a decode step, the short convolution and the output epilogue, each
checked against the oracle, so the synchronous mode returns the same results
with KDA_OK.
"""
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, ROOT)
import numpy as np, torch
import gated_delta_rule_53_amd as kda
import kda_workloads as w
import oracle
from oracle import conv, epilogue
d = lambda t: None if t is None else t.to("cuda:0").contiguous()
worst = 0.0
for dd, dt in [(128, torch.bfloat16), (64, torch.float32)]:
    x = w.make_prefill([70, 33], 2, dd, dt, seed=3)
    o, s = kda.chunk_fwd(d(x.q), d(x.k), d(x.v), d(x.g), d(x.beta), d(x.cu_seqlens), d(x.initial_state),
                         scale=x.scale, out_dtype=torch.float32)
    ro, rs = oracle.forward(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, x.initial_state, scale=x.scale)
    worst = max(worst, float(np.abs(o.double().cpu().numpy() - ro).max() / np.abs(ro).max()))
y = w.make_decode(4, 1, 2, 128, torch.bfloat16, seed=4)
st = d(y.initial_state)
o = kda.recurrent_step(d(y.q[0]), d(y.k[0]), d(y.v[0]), d(y.g[0]), d(y.beta[0]), st, scale=y.scale,
                       out_dtype=torch.float32)
ro, rs = oracle.decode(y.q, y.k, y.v, y.g, y.beta, y.initial_state, scale=y.scale)
worst = max(worst, float(np.abs(o.double().cpu().numpy() - ro[0]).max() / np.abs(ro[0]).max()))
xc = torch.randn(40, 64).float(); wc = torch.randn(4, 64).float(); cu = torch.tensor([0, 25, 40], dtype=torch.int32)
yc, sc = kda.short_conv(d(xc), d(wc), d(cu))
rc, _ = conv.short_conv(xc, wc, cu.numpy())
worst = max(worst, float(np.abs(yc.double().cpu().numpy() - rc).max() / np.abs(rc).max()))
on = torch.randn(10, 3, 128); gn = torch.randn(10, 3, 128); wn = torch.ones(128)
yn = kda.gated_rmsnorm(d(on), d(gn), d(wn))
rn = epilogue.gated_rmsnorm(on, gn, wn, 1e-6)
worst = max(worst, float(np.abs(yn.double().cpu().numpy() - rn).max() / np.abs(rn).max()))
print("WORST", worst, flush=True)
assert worst <= 2e-3, worst
""".replace("ROOT", repr(ROOT))


def test_debug_mode_gives_the_same_results():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ, KDA_DEBUG="1")
    print("\n[gpu-case] KDA_DEBUG=1 child process", file=sys.stderr, flush=True)
    res = subprocess.run([sys.executable, "-c", CHILD], env=env, capture_output=True, text=True, timeout=240)
    print(res.stdout[-2000:], res.stderr[-2000:])
    assert res.returncode == 0, res.stderr[-2000:]
    assert "WORST" in res.stdout

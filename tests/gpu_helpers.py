"""Shared helpers for the GPU parity tests (device copies, error metric, case logging)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances on max|gpu - oracle| / max|oracle| (per tensor): bf16 inputs, fp32 inputs.
TOL_BF16 = 2e-3
TOL_F32 = 1e-4


def announce(msg: str) -> None:
    """Name the case on stderr before a GPU step, flushed, so a dead run still shows it."""
    print(f"\n[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(t, device="cuda:0"):
    return None if t is None else t.to(device).contiguous()


def rel_err(gpu: torch.Tensor, ref: np.ndarray) -> float:
    """max |gpu - ref| / max |ref| (absolute error when ref is all zero)."""
    g = gpu.detach().double().cpu().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if g.size == 0:
        return 0.0
    den = float(np.abs(ref).max())
    err = float(np.abs(g - ref).max())
    return err / den if den > 0 else err


def tol_for(dtype: torch.dtype) -> float:
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def prefill_on_gpu(x, out_dtype=torch.float32, with_state=True, heads=None):
    """Run kda.chunk_fwd on a kda_workloads.PrefillInputs; returns (out, final_state)."""
    import gated_delta_rule_53_amd as kda
    q, k, v, g, b = (dev(t) for t in (x.q, x.k, x.v, x.g, x.beta))
    cu = dev(x.cu_seqlens)
    s0 = dev(x.initial_state) if with_state else None
    out, fs = kda.chunk_fwd(q, k, v, g, b, cu, s0, scale=x.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, fs

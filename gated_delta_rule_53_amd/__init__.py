"""Kimi Delta Attention (KDA) core for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libkda.so`` (declared in
``include/kda.h``).  This module only marshals arguments: it checks tensor
shapes, dtypes and devices, allocates outputs with PyTorch and passes raw
device pointers plus the current HIP stream.  Every step of the computation
runs in the library's HIP kernels; there is no fallback.  Importing works
without a GPU (argument checks still run); a missing library raises
ImportError.
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    KDA_BF16,
    KDA_F32,
    Conv,
    Gate,
    KdaError,
    Problem,
    abi_version,
    chunk_fwd,
    chunk_fwd_conv,
    chunk_fwd_gated,
    chunk_fwd_noalloc,
    chunk_fwd_pooled,
    chunk_fwd_workspace_bytes,
    gated_rmsnorm,
    library_path,
    short_conv,
    raw_library,
    recurrent_step,
    recurrent_step_gated,
    recurrent_step_normed,
    recurrent_verify,
    recurrent_verify_normed,
)

__all__ = [
    "chunk_fwd",
    "chunk_fwd_gated",
    "chunk_fwd_conv",
    "chunk_fwd_noalloc",
    "recurrent_step",
    "recurrent_step_gated",
    "recurrent_step_normed",
    "chunk_fwd_pooled",
    "recurrent_verify",
    "recurrent_verify_normed",
    "gated_rmsnorm",
    "short_conv",
    "Gate",
    "Conv",
    "chunk_fwd_workspace_bytes",
    "abi_version",
    "library_path",
    "raw_library",
    "Problem",
    "KdaError",
    "KDA_F32",
    "KDA_BF16",
]

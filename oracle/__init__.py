"""CPU fp64 oracle for the Kimi Delta Attention (KDA) core.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library in ``gated_delta_rule_53_amd`` and never imports it.

Two independent formulations live here:

* ``forward`` -- the token-by-token recurrence in plain C (``kda_oracle.c``),
  the correctness authority;
* ``chunked.forward_chunked`` -- the chunked (WY / UT transform) form in numpy
  fp64, a second derivation of the same function used to pin the first.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libkda_oracle.so")

# x86-64-v3 (AVX2 + FMA) runs on every current server host; fused multiply-add
# contraction is switched off so each product is rounded as written.
CFLAGS = ["-O2", "-march=x86-64-v3", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
          "-std=c99", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc; returns the library path."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    os.makedirs(_BUILD_DIR, exist_ok=True)
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def load(path: str):
    """Open a compiled oracle library at ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    i64, dbl, ptr = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.kda_oracle_forward.argtypes = [i64, i64, i64, i64, ptr, ptr, ptr, ptr, ptr, ptr,
                                       ptr, dbl, ctypes.c_int, ptr, ptr]
    lib.kda_oracle_forward.restype = ctypes.c_int
    lib.kda_oracle_threads.argtypes = []
    lib.kda_oracle_threads.restype = ctypes.c_int
    lib.kda_oracle_set_threads.argtypes = [ctypes.c_int]
    lib.kda_oracle_set_threads.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = load(_LIB_PATH)
    return _lib


def threads() -> int:
    """OpenMP threads the C oracle uses."""
    return int(_load().kda_oracle_threads())


def set_threads(n: int) -> None:
    """Use n OpenMP threads in later calls (the results do not depend on it)."""
    _load().kda_oracle_set_threads(int(n))


def _f32(x) -> np.ndarray:
    """Widen to a contiguous float32 numpy array (exact for bf16 and fp32 input)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward(q, k, v, g, beta, cu_seqlens, initial_state=None, scale: Optional[float] = None,
            qk_l2norm: bool = True, want_state: bool = True,
            lib=None) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Packed-varlen KDA forward, fp64, token by token.

    q, k: [T, H, dk]; v: [T, H, dv]; g: [T, H, dk], or [T, H] for one decay
    per head; beta: [T, H]; cu_seqlens: [N+1]; initial_state: [N, H, dk, dv] or None.
    Returns (out [T, H, dv] float64, final_state [N, H, dk, dv] float64 or None).
    ``lib`` selects another compiled copy of the oracle (the default is the
    one built from ``kda_oracle.c``).
    """
    qf, kf, vf, gf, bf = (_f32(t) for t in (q, k, v, g, beta))
    if gf.ndim == 2:
        # one log-decay per (token, head), the same for every key channel: the
        # scalar gate of Gated DeltaNet, a special case of the per-channel decay
        gf = np.ascontiguousarray(np.broadcast_to(gf[:, :, None], qf.shape))
    cu = np.ascontiguousarray(np.asarray(
        cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64))
    T, H, dk = qf.shape
    dv = vf.shape[2]
    N = cu.shape[0] - 1
    if kf.shape != (T, H, dk) or gf.shape != (T, H, dk) or vf.shape[:2] != (T, H) or bf.shape != (T, H):
        raise ValueError("oracle: inconsistent shapes")
    if int(cu[-1]) != T:
        raise ValueError("oracle: cu_seqlens[-1] must equal T")
    s0 = None if initial_state is None else _f32(initial_state)
    if s0 is not None and s0.shape != (N, H, dk, dv):
        raise ValueError("oracle: initial_state must be [N, H, dk, dv]")
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    out = np.empty((T, H, dv), dtype=np.float64)
    fs = np.empty((N, H, dk, dv), dtype=np.float64) if want_state else None
    rc = (lib or _load()).kda_oracle_forward(N, H, dk, dv, _ptr(cu), _ptr(qf), _ptr(kf), _ptr(vf),
                                    _ptr(gf), _ptr(bf), _ptr(s0), float(scale), int(bool(qk_l2norm)),
                                    _ptr(out), _ptr(fs))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return out, fs


def decode(q, k, v, g, beta, initial_state, scale: Optional[float] = None, qk_l2norm: bool = True):
    """Batched decode: ``steps`` tokens for each of N independent sequences.

    q, k: [steps, N, H, dk]; v: [steps, N, H, dv]; g like q; beta [steps, N, H];
    initial_state [N, H, dk, dv].  A decode step is the recurrence applied to
    one more token, so this is ``forward`` on the sequences laid out one after
    another.  Returns (out [steps, N, H, dv], final_state [N, H, dk, dv]).
    """
    qf, kf, vf, gf, bf = (_f32(t) for t in (q, k, v, g, beta))
    steps, N, H, dk = qf.shape
    dv = vf.shape[3]

    def seq_major(a):
        return np.ascontiguousarray(np.swapaxes(a, 0, 1).reshape(N * steps, *a.shape[2:]))

    cu = np.arange(N + 1, dtype=np.int64) * steps
    out, fs = forward(seq_major(qf), seq_major(kf), seq_major(vf), seq_major(gf), seq_major(bf),
                      cu, initial_state, scale, qk_l2norm)
    out = np.ascontiguousarray(np.swapaxes(out.reshape(N, steps, H, dv), 0, 1))
    return out, fs

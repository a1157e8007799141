"""ctypes binding of libkda.so: argument marshalling only."""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_F32 = 0
KDA_BF16 = 1

_STATUS_NAMES = {0: "KDA_OK", 1: "KDA_ERR_NULL_POINTER", 2: "KDA_ERR_BAD_SHAPE",
                 3: "KDA_ERR_UNSUPPORTED", 4: "KDA_ERR_WORKSPACE", 5: "KDA_ERR_HIP"}


class KdaError(RuntimeError):
    """A non-OK status from the library; ``status`` holds the code."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {detail}")


class KdaArgumentError(KdaError, ValueError):
    """Rejected arguments (status 1-4): nothing was launched."""


class Problem(ctypes.Structure):
    """Mirror of ``kda_problem_t``."""

    _fields_ = [
        ("total_tokens", ctypes.c_int64),
        ("num_seqs", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_k", ctypes.c_int32),
        ("head_v", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("qk_l2norm", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("gate_per_head", ctypes.c_int32),
        ("state_layout", ctypes.c_int32),
    ]


class Gate(ctypes.Structure):
    """Mirror of ``kda_gate_t``."""

    _fields_ = [
        ("a_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("has_lower_bound", ctypes.c_int32),
        ("lower_bound", ctypes.c_float),
    ]


class Conv(ctypes.Structure):
    """Mirror of ``kda_conv_t``."""

    _fields_ = [
        ("kernel_size", ctypes.c_int32),
        ("silu", ctypes.c_int32),
        ("weight", ctypes.c_void_p),
        ("state_in", ctypes.c_void_p),
        ("state_out", ctypes.c_void_p),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python gated_delta_rule_53_amd/build.py` "
            "(hipcc, gfx950).  There is no fallback implementation.")
    lib = ctypes.CDLL(_LIB_PATH)
    P, vp, fp, sz = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [P]
    lib.kda_chunk_fwd_workspace_bytes.restype = sz
    lib.kda_chunk_fwd.argtypes = [P, vp, vp, vp, fp, fp, vp, fp, vp, fp, vp, sz, vp]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [P, vp, vp, vp, fp, fp, vp, fp, vp, fp, vp]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_recurrent_step.argtypes = [P, vp, vp, vp, fp, fp, fp, vp, vp]
    lib.kda_recurrent_step.restype = ctypes.c_int
    G = ctypes.POINTER(Gate)
    lib.kda_chunk_fwd_gated.argtypes = [P, G, vp, vp, vp, vp, vp, vp, fp, vp, fp, vp, sz, vp]
    lib.kda_chunk_fwd_gated.restype = ctypes.c_int
    lib.kda_chunk_fwd_conv.argtypes = [P, G, ctypes.POINTER(Conv), vp, vp, vp, vp, fp, vp, fp, vp, sz, vp]
    lib.kda_chunk_fwd_conv.restype = ctypes.c_int
    lib.kda_recurrent_step_gated.argtypes = [P, G, vp, vp, vp, vp, vp, fp, vp, vp]
    lib.kda_recurrent_step_gated.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.kda_chunk_fwd_pooled.argtypes = [P, G, vp, vp, vp, vp, vp, vp, fp, i32, vp, vp, vp, sz, vp]
    lib.kda_chunk_fwd_pooled.restype = ctypes.c_int
    lib.kda_recurrent_verify.argtypes = [P, i32, G, vp, vp, vp, vp, vp, fp, i32, vp, vp, vp, vp]
    lib.kda_recurrent_verify.restype = ctypes.c_int
    lib.kda_recurrent_verify_normed.argtypes = [P, i32, G, vp, vp, vp, vp, vp, fp, i32, vp, vp, vp, fp,
                                                ctypes.c_float, vp, vp]
    lib.kda_recurrent_verify_normed.restype = ctypes.c_int
    lib.kda_gated_rmsnorm.argtypes = [ctypes.c_int64, i32, i32, i32, vp, vp, fp, ctypes.c_float, vp, vp]
    lib.kda_gated_rmsnorm.restype = ctypes.c_int
    lib.kda_short_conv.argtypes = [i32, ctypes.c_int64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_short_conv.restype = ctypes.c_int
    lib.kda_recurrent_step_normed.argtypes = [P, G, vp, vp, vp, vp, vp, fp, vp, fp, ctypes.c_float, vp, vp]
    lib.kda_recurrent_step_normed.restype = ctypes.c_int
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def raw_library() -> ctypes.CDLL:
    """The loaded C library with its signatures declared."""
    return _lib


def abi_version() -> int:
    return int(_lib.kda_abi_version())


def _check(status: int) -> None:
    if status != 0:
        detail = _lib.kda_last_error().decode(errors="replace")
        cls = KdaError if status == 5 else KdaArgumentError
        raise cls(status, detail)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return KDA_F32
    if t == torch.bfloat16:
        return KDA_BF16
    raise KdaArgumentError(3, f"unsupported dtype {t} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if tuple(t.shape) != tuple(shape):
        raise KdaArgumentError(2, f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise KdaArgumentError(3, f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise KdaArgumentError(2, f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise KdaArgumentError(2, f"{name} must be contiguous")


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# State block layouts (kda_problem_t.state_layout): S[dk][dv], or its transpose.
STATE_LAYOUTS = {"dk_dv": 0, "dv_dk": 1}


def _layout_code(state_layout: str) -> int:
    if state_layout not in STATE_LAYOUTS:
        raise KdaArgumentError(2, f"state_layout must be one of {sorted(STATE_LAYOUTS)}, got {state_layout!r}")
    return STATE_LAYOUTS[state_layout]


def _problem(T, N, H, dk, dv, qkv_dtype, out_dtype, scale, qk_l2norm, gate_per_head=False,
             state_layout: str = "dk_dv") -> Problem:
    return Problem(total_tokens=T, num_seqs=N, num_heads=H, head_k=dk, head_v=dv,
                   qkv_dtype=_dtype_code(qkv_dtype), out_dtype=_dtype_code(out_dtype),
                   scale=float(1.0 / math.sqrt(dk) if scale is None else scale),
                   qk_l2norm=int(bool(qk_l2norm)), chunk_size=64, gate_per_head=int(bool(gate_per_head)),
                   state_layout=_layout_code(state_layout))


def _gate_shape(g: torch.Tensor, lead: tuple, dk: int):
    """(per_head, expected shape) of a gate tensor: lead + (dk,), or lead alone (one decay per head)."""
    per_head = g.dim() == len(lead)
    return per_head, lead if per_head else lead + (dk,)


def chunk_fwd_workspace_bytes(problem: Problem) -> int:
    return int(_lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(problem)))


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
              initial_state: Optional[torch.Tensor] = None, *, scale: Optional[float] = None,
              state_layout: str = "dk_dv",
              qk_l2norm: bool = True, out_dtype: Optional[torch.dtype] = None,
              output_final_state: bool = True, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked KDA prefill over packed sequences (``kda_chunk_fwd``).

    q, k [T, H, dk]; v [T, H, dv] (float32 or bfloat16, all one dtype);
    g [T, H, dk] float32; beta [T, H] float32; cu_seqlens [N+1] int32 on the
    device (None: one sequence of T tokens); initial_state [N, H, dk, dv]
    float32 or None.  Returns (out [T, H, dv] in ``out_dtype`` (default: v's
    dtype), final_state [N, H, dk, dv] float32 or None).  Runs on the current
    stream of q's device.  ``final_state`` may be ``initial_state`` itself.
    ``cu_seqlens=None`` builds [0, T] on the device, and the workspace (if
    not given) and the outputs (if not given) are allocated, on every call:
    under graph capture or in allocation-free loops pass them all (or use
    ``chunk_fwd_noalloc``).
    ``state_layout="dv_dk"`` takes and returns every state block transposed,
    [..., dv, dk] (kda_problem_t.state_layout; the same for every call below).
    """
    if q.dim() != 3:
        raise KdaArgumentError(2, f"q must be [T, H, dk], got {tuple(q.shape)}")
    T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise KdaArgumentError(2, "tensors must be on a GPU device")
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=dev)
    N = cu_seqlens.numel() - 1
    _need(q, "q", (T, H, dk), None, dev)
    _need(k, "k", (T, H, dk), q.dtype, dev)
    _need(v, "v", (T, H, dv), q.dtype, dev)
    gph, gshape = _gate_shape(g, (T, H), dk)
    _need(g, "g", gshape, torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, dk, dv), torch.float32, dev)
    out_dtype = v.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((T, H, dv), dtype=out_dtype, device=dev)
    _need(out, "out", (T, H, dv), out_dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", (N, H, dk, dv), torch.float32, dev)
    prob = _problem(T, N, H, dk, dv, q.dtype, out_dtype, scale, qk_l2norm, gph, state_layout)
    ws_bytes = chunk_fwd_workspace_bytes(prob)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.kda_chunk_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                              _ptr(cu_seqlens), _ptr(initial_state), _ptr(out), _ptr(final_state),
                              _ptr(workspace), ws_len, _stream(dev)))
    return out, final_state


NOALLOC_SCRATCH_BYTES = 128 << 20  # KDA_NOALLOC_SCRATCH_BYTES


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                      beta: torch.Tensor, cu_seqlens: torch.Tensor, initial_state: Optional[torch.Tensor],
                      out: torch.Tensor, final_state: Optional[torch.Tensor], *, scale: Optional[float] = None,
                      state_layout: str = "dk_dv", qk_l2norm: bool = True) -> None:
    """``kda_chunk_fwd_noalloc``: chunk_fwd with no workspace and no allocation.

    For callers that cannot allocate device memory (graph capture, serving
    loops): every tensor, ``out`` and ``final_state`` included, comes from
    the caller, and the library's own 128 MiB device array serves as the
    workspace.  Problems needing more workspace than that are rejected.
    Calls that overlap in time on one GPU share that array and race.
    Arguments as for ``chunk_fwd``; ``out`` gives the output dtype.
    """
    if q.dim() != 3:
        raise KdaArgumentError(2, f"q must be [T, H, dk], got {tuple(q.shape)}")
    T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise KdaArgumentError(2, "tensors must be on a GPU device")
    N = cu_seqlens.numel() - 1
    _need(q, "q", (T, H, dk), None, dev)
    _need(k, "k", (T, H, dk), q.dtype, dev)
    _need(v, "v", (T, H, dv), q.dtype, dev)
    gph, gshape = _gate_shape(g, (T, H), dk)
    _need(g, "g", gshape, torch.float32, dev)
    _need(beta, "beta", (T, H), torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, dk, dv), torch.float32, dev)
    _need(out, "out", (T, H, dv), out.dtype, dev)
    if final_state is not None:
        _need(final_state, "final_state", (N, H, dk, dv), torch.float32, dev)
    prob = _problem(T, N, H, dk, dv, q.dtype, out.dtype, scale, qk_l2norm, gph, state_layout)
    _check(_lib.kda_chunk_fwd_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(cu_seqlens), _ptr(initial_state), _ptr(out), _ptr(final_state),
                                      _stream(dev)))


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                   beta: torch.Tensor, state: torch.Tensor, *, scale: Optional[float] = None,
                   state_layout: str = "dk_dv",
                   qk_l2norm: bool = True, out_dtype: Optional[torch.dtype] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step for N sequences (``kda_recurrent_step``); ``state`` is updated in place.

    q, k [N, H, dk]; v [N, H, dv]; g [N, H, dk] float32; beta [N, H] float32;
    state [N, H, dk, dv] float32.  Returns out [N, H, dv] (default: v's dtype).
    """
    if q.dim() != 3:
        raise KdaArgumentError(2, f"q must be [N, H, dk], got {tuple(q.shape)}")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise KdaArgumentError(2, "tensors must be on a GPU device")
    _need(k, "k", (N, H, dk), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    gph, gshape = _gate_shape(g, (N, H), dk)
    _need(g, "g", gshape, torch.float32, dev)
    _need(beta, "beta", (N, H), torch.float32, dev)
    _need(state, "state", (N, H, dk, dv), torch.float32, dev)
    out_dtype = v.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    _need(out, "out", (N, H, dv), out_dtype, dev)
    prob = _problem(N, N, H, dk, dv, q.dtype, out_dtype, scale, qk_l2norm, gph, state_layout)
    _check(_lib.kda_recurrent_step(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(state), _ptr(out), _stream(dev)))
    return out


def _gate(a_log: torch.Tensor, dt_bias: torch.Tensor, H: int, dk: int, lower_bound: Optional[float],
          dev, per_head: bool = False) -> Gate:
    _need(a_log, "a_log", (H,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H,) if per_head else (H, dk), torch.float32, dev)
    return Gate(a_log=a_log.data_ptr(), dt_bias=dt_bias.data_ptr(),
                has_lower_bound=int(lower_bound is not None),
                lower_bound=float(0.0 if lower_bound is None else lower_bound))


def chunk_fwd_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, raw_g: torch.Tensor,
                    raw_beta: torch.Tensor, a_log: torch.Tensor, dt_bias: torch.Tensor,
                    cu_seqlens: Optional[torch.Tensor] = None,
                    initial_state: Optional[torch.Tensor] = None, *, lower_bound: Optional[float] = None,
                    scale: Optional[float] = None, state_layout: str = "dk_dv", qk_l2norm: bool = True,
                    out_dtype: Optional[torch.dtype] = None, output_final_state: bool = True,
                    out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``chunk_fwd`` with the gate activation fused in (``kda_chunk_fwd_gated``).

    raw_g [T, H, dk] and raw_beta [T, H] in q's dtype; a_log [H] and dt_bias
    [H, dk] float32; lower_bound None (softplus gate) or a float <= 0 (bounded
    sigmoid gate).  Other arguments and the result are as for ``chunk_fwd``.
    """
    if q.dim() != 3:
        raise KdaArgumentError(2, f"q must be [T, H, dk], got {tuple(q.shape)}")
    T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise KdaArgumentError(2, "tensors must be on a GPU device")
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=dev)
    N = cu_seqlens.numel() - 1
    _need(q, "q", (T, H, dk), None, dev)
    _need(k, "k", (T, H, dk), q.dtype, dev)
    _need(v, "v", (T, H, dv), q.dtype, dev)
    gph, gshape = _gate_shape(raw_g, (T, H), dk)
    _need(raw_g, "raw_g", gshape, q.dtype, dev)
    _need(raw_beta, "raw_beta", (T, H), q.dtype, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    gate = _gate(a_log, dt_bias, H, dk, lower_bound, dev, gph)
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, dk, dv), torch.float32, dev)
    out_dtype = v.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((T, H, dv), dtype=out_dtype, device=dev)
    _need(out, "out", (T, H, dv), out_dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", (N, H, dk, dv), torch.float32, dev)
    prob = _problem(T, N, H, dk, dv, q.dtype, out_dtype, scale, qk_l2norm, gph, state_layout)
    ws_bytes = chunk_fwd_workspace_bytes(prob)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.kda_chunk_fwd_gated(ctypes.byref(prob), ctypes.byref(gate), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(raw_g), _ptr(raw_beta), _ptr(cu_seqlens), _ptr(initial_state),
                                    _ptr(out), _ptr(final_state), _ptr(workspace), ws_len, _stream(dev)))
    return out, final_state


def recurrent_step_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, raw_g: torch.Tensor,
                         raw_beta: torch.Tensor, a_log: torch.Tensor, dt_bias: torch.Tensor,
                         state: torch.Tensor, *, lower_bound: Optional[float] = None,
                         scale: Optional[float] = None, state_layout: str = "dk_dv", qk_l2norm: bool = True,
                         out_dtype: Optional[torch.dtype] = None,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``recurrent_step`` with the gate activation fused in (``kda_recurrent_step_gated``).

    raw_g [N, H, dk] and raw_beta [N, H] in q's dtype; a_log [H], dt_bias
    [H, dk] float32; ``state`` is updated in place.
    """
    if q.dim() != 3:
        raise KdaArgumentError(2, f"q must be [N, H, dk], got {tuple(q.shape)}")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise KdaArgumentError(2, "tensors must be on a GPU device")
    _need(k, "k", (N, H, dk), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    gph, gshape = _gate_shape(raw_g, (N, H), dk)
    _need(raw_g, "raw_g", gshape, q.dtype, dev)
    _need(raw_beta, "raw_beta", (N, H), q.dtype, dev)
    _need(state, "state", (N, H, dk, dv), torch.float32, dev)
    gate = _gate(a_log, dt_bias, H, dk, lower_bound, dev, gph)
    out_dtype = v.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    _need(out, "out", (N, H, dv), out_dtype, dev)
    prob = _problem(N, N, H, dk, dv, q.dtype, out_dtype, scale, qk_l2norm, gph, state_layout)
    _check(_lib.kda_recurrent_step_gated(ctypes.byref(prob), ctypes.byref(gate), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(raw_g), _ptr(raw_beta), _ptr(state), _ptr(out), _stream(dev)))
    return out


def _gate_or_none(a_log, dt_bias, H, dk, lower_bound, dev, per_head=False):
    if a_log is None:
        if dt_bias is not None or lower_bound is not None:
            raise KdaArgumentError(1, "dt_bias and lower_bound need a_log")
        return None
    if dt_bias is None:
        raise KdaArgumentError(1, "a_log needs dt_bias")
    return _gate(a_log, dt_bias, H, dk, lower_bound, dev, per_head)


def chunk_fwd_conv(qkv: torch.Tensor, g: torch.Tensor, beta: torch.Tensor, conv_weight: torch.Tensor,
                   cu_seqlens: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                   conv_state: Optional[torch.Tensor] = None, *, silu: bool = True,
                   conv_state_out: Optional[torch.Tensor] = None, a_log: Optional[torch.Tensor] = None,
                   dt_bias: Optional[torch.Tensor] = None, lower_bound: Optional[float] = None,
                   scale: Optional[float] = None, state_layout: str = "dk_dv", qk_l2norm: bool = True,
                   out_dtype: Optional[torch.dtype] = None, output_final_state: bool = True,
                   out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill with the short convolution fused in (``kda_chunk_fwd_conv``).

    qkv [T, 3, H, d] bfloat16, d = 128: the fused q/k/v projection before
    the convolution; conv_weight [K, 3 H d] bfloat16 (tap-major, K = 1..4);
    conv_state [N, K-1, 3 H d] bfloat16 or None (zeros); conv_state_out, if
    given, receives each request's last K-1 inputs (it may be conv_state).
    g, beta: float32 activated, or the raw projections in bfloat16 with
    a_log / dt_bias / lower_bound as for ``chunk_fwd_gated``.  The rest as for
    ``chunk_fwd``.  Equals ``short_conv`` followed by ``chunk_fwd`` on the
    split output.  Returns (out, final_state).
    """
    if qkv.dim() != 4 or qkv.shape[1] != 3:
        raise KdaArgumentError(2, f"qkv must be [T, 3, H, d], got {tuple(qkv.shape)}")
    T, _, H, d = qkv.shape
    dev = qkv.device
    if dev.type != "cuda":
        raise KdaArgumentError(2, "tensors must be on a GPU device")
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=dev)
    N = cu_seqlens.numel() - 1
    _need(qkv, "qkv", (T, 3, H, d), None, dev)
    if conv_weight.dim() != 2:
        raise KdaArgumentError(2, f"conv_weight must be [K, 3 H d], got {tuple(conv_weight.shape)}")
    K = conv_weight.shape[0]
    _need(conv_weight, "conv_weight", (K, 3 * H * d), qkv.dtype, dev)
    for name, st in (("conv_state", conv_state), ("conv_state_out", conv_state_out)):
        if st is not None:
            _need(st, name, (N, K - 1, 3 * H * d), qkv.dtype, dev)
    gph, gshape = _gate_shape(g, (T, H), d)
    gate = _gate_or_none(a_log, dt_bias, H, d, lower_bound, dev, gph)
    gdt = torch.float32 if gate is None else qkv.dtype
    _need(g, "g", gshape, gdt, dev)
    _need(beta, "beta", (T, H), gdt, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, d, d), torch.float32, dev)
    out_dtype = qkv.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((T, H, d), dtype=out_dtype, device=dev)
    _need(out, "out", (T, H, d), out_dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, d, d), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", (N, H, d, d), torch.float32, dev)
    prob = _problem(T, N, H, d, d, qkv.dtype, out_dtype, scale, qk_l2norm, gph, state_layout)
    ws_bytes = chunk_fwd_workspace_bytes(prob)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    conv = Conv(kernel_size=K, silu=int(bool(silu)), weight=conv_weight.data_ptr(),
                state_in=None if conv_state is None else conv_state.data_ptr(),
                state_out=None if conv_state_out is None else conv_state_out.data_ptr())
    _check(_lib.kda_chunk_fwd_conv(ctypes.byref(prob), None if gate is None else ctypes.byref(gate),
                                   ctypes.byref(conv), _ptr(qkv), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                   _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(workspace), ws_len,
                                   _stream(dev)))
    return out, final_state


def chunk_fwd_pooled(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                     beta: torch.Tensor, state_pool: torch.Tensor, state_slots: torch.Tensor,
                     cu_seqlens: Optional[torch.Tensor] = None, *, a_log: Optional[torch.Tensor] = None,
                     dt_bias: Optional[torch.Tensor] = None, lower_bound: Optional[float] = None,
                     scale: Optional[float] = None, state_layout: str = "dk_dv", qk_l2norm: bool = True,
                     out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Chunked prefill with the states in a slot pool (``kda_chunk_fwd_pooled``).

    state_pool [P, H, dk, dv] float32 is read and written: sequence n starts
    from slot state_slots[n] (int32 [N], device) and its final state goes back
    there; a slot outside [0, P) starts from zero and is not written.  Without
    a_log, g [T, H, dk] and beta [T, H] are float32; with a_log (and dt_bias,
    lower_bound as for ``chunk_fwd_gated``) they are the raw projections in
    q's dtype.  Returns out.  cu_seqlens, out and workspace: as for
    ``chunk_fwd`` (built or allocated on every call when not given).
    """
    if q.dim() != 3:
        raise KdaArgumentError(2, f"q must be [T, H, dk], got {tuple(q.shape)}")
    T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise KdaArgumentError(2, "tensors must be on a GPU device")
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=dev)
    N = cu_seqlens.numel() - 1
    gph, gshape = _gate_shape(g, (T, H), dk)
    gate = _gate_or_none(a_log, dt_bias, H, dk, lower_bound, dev, gph)
    gdt = torch.float32 if gate is None else q.dtype
    _need(q, "q", (T, H, dk), None, dev)
    _need(k, "k", (T, H, dk), q.dtype, dev)
    _need(v, "v", (T, H, dv), q.dtype, dev)
    _need(g, "g", gshape, gdt, dev)
    _need(beta, "beta", (T, H), gdt, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if state_pool.dim() != 4:
        raise KdaArgumentError(2, f"state_pool must be [P, H, dk, dv], got {tuple(state_pool.shape)}")
    P = state_pool.shape[0]
    _need(state_pool, "state_pool", (P, H, dk, dv), torch.float32, dev)
    _need(state_slots, "state_slots", (N,), torch.int32, dev)
    out_dtype = v.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((T, H, dv), dtype=out_dtype, device=dev)
    _need(out, "out", (T, H, dv), out_dtype, dev)
    prob = _problem(T, N, H, dk, dv, q.dtype, out_dtype, scale, qk_l2norm, gph, state_layout)
    ws_bytes = chunk_fwd_workspace_bytes(prob)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.kda_chunk_fwd_pooled(ctypes.byref(prob), None if gate is None else ctypes.byref(gate), _ptr(q),
                                     _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(state_pool),
                                     P, _ptr(state_slots), _ptr(out), _ptr(workspace), ws_len, _stream(dev)))
    return out


def recurrent_verify(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                     beta: torch.Tensor, state_pool: torch.Tensor, state_indices: torch.Tensor,
                     num_accepted: Optional[torch.Tensor] = None, *, a_log: Optional[torch.Tensor] = None,
                     dt_bias: Optional[torch.Tensor] = None, lower_bound: Optional[float] = None,
                     scale: Optional[float] = None, state_layout: str = "dk_dv", qk_l2norm: bool = True,
                     out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                     out_gate: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
                     norm_eps: float = 1e-6) -> torch.Tensor:
    """Multi-token verify decode over a slot pool (``kda_recurrent_verify``).

    q, k [N, W, H, dk]; v [N, W, H, dv]; g, beta [N, W, H, dk], [N, W, H]
    (float32, or raw in q's dtype with a_log); state_pool [P, H, dk, dv]
    float32; state_indices [N, W] int32: sequence n starts from slot
    state_indices[n, a-1] (a = num_accepted[n] clamped to [1, W], 1 without
    num_accepted) and writes its state after token t to slot
    state_indices[n, t].  Returns out [N, W, H, dv].

    With out_gate [N, W, H, dv] (q's dtype) and norm_weight [dv] float32 the
    output epilogue is fused (``kda_recurrent_verify_normed``): the returned
    rows are o / sqrt(mean(o^2) + norm_eps) * norm_weight * sigmoid(out_gate).
    """
    if q.dim() != 4:
        raise KdaArgumentError(2, f"q must be [N, W, H, dk], got {tuple(q.shape)}")
    N, W, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise KdaArgumentError(2, "tensors must be on a GPU device")
    gph, gshape = _gate_shape(g, (N, W, H), dk)
    gate = _gate_or_none(a_log, dt_bias, H, dk, lower_bound, dev, gph)
    gdt = torch.float32 if gate is None else q.dtype
    _need(k, "k", (N, W, H, dk), q.dtype, dev)
    _need(v, "v", (N, W, H, dv), q.dtype, dev)
    _need(g, "g", gshape, gdt, dev)
    _need(beta, "beta", (N, W, H), gdt, dev)
    if state_pool.dim() != 4:
        raise KdaArgumentError(2, f"state_pool must be [P, H, dk, dv], got {tuple(state_pool.shape)}")
    P = state_pool.shape[0]
    _need(state_pool, "state_pool", (P, H, dk, dv), torch.float32, dev)
    _need(state_indices, "state_indices", (N, W), torch.int32, dev)
    if num_accepted is not None:
        _need(num_accepted, "num_accepted", (N,), torch.int32, dev)
    normed = out_gate is not None or norm_weight is not None
    if normed:
        if out_gate is None or norm_weight is None:
            raise KdaArgumentError(2, "out_gate and norm_weight go together")
        _need(out_gate, "out_gate", (N, W, H, dv), q.dtype, dev)
        _need(norm_weight, "norm_weight", (dv,), torch.float32, dev)
    out_dtype = v.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((N, W, H, dv), dtype=out_dtype, device=dev)
    _need(out, "out", (N, W, H, dv), out_dtype, dev)
    prob = _problem(N * W, N, H, dk, dv, q.dtype, out_dtype, scale, qk_l2norm, gph, state_layout)
    gp = None if gate is None else ctypes.byref(gate)
    if normed:
        _check(_lib.kda_recurrent_verify_normed(ctypes.byref(prob), W, gp, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                                _ptr(beta), _ptr(state_pool), P, _ptr(state_indices),
                                                _ptr(num_accepted), _ptr(out_gate), _ptr(norm_weight),
                                                float(norm_eps), _ptr(out), _stream(dev)))
    else:
        _check(_lib.kda_recurrent_verify(ctypes.byref(prob), W, gp, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                         _ptr(beta), _ptr(state_pool), P, _ptr(state_indices),
                                         _ptr(num_accepted), _ptr(out), _stream(dev)))
    return out


def recurrent_verify_normed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                            beta: torch.Tensor, state_pool: torch.Tensor, state_indices: torch.Tensor,
                            out_gate: torch.Tensor, norm_weight: torch.Tensor,
                            num_accepted: Optional[torch.Tensor] = None, *, norm_eps: float = 1e-6,
                            **kwargs) -> torch.Tensor:
    """Verify decode with the output epilogue fused (``kda_recurrent_verify_normed``).

    As ``recurrent_verify`` (same keyword arguments), but each returned row is
    o / sqrt(mean(o^2) + norm_eps) * norm_weight * sigmoid(out_gate), with
    out_gate [N, W, H, dv] in q's dtype and norm_weight [dv] float32.
    """
    return recurrent_verify(q, k, v, g, beta, state_pool, state_indices, num_accepted, out_gate=out_gate,
                            norm_weight=norm_weight, norm_eps=norm_eps, **kwargs)


def gated_rmsnorm(o: torch.Tensor, gate: torch.Tensor, weight: torch.Tensor, *, eps: float = 1e-6,
                  out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Output epilogue (``kda_gated_rmsnorm``): o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate).

    o, gate [..., dv] (float32 or bfloat16, one dtype, same shape); weight [dv]
    float32.  Returns out [..., dv] in ``out_dtype`` (default: o's dtype);
    ``out`` may be ``o`` itself when the dtypes match.
    """
    dev = o.device
    if dev.type != "cuda":
        raise KdaArgumentError(2, "tensors must be on a GPU device")
    if o.dim() < 1:
        raise KdaArgumentError(2, "o must have a trailing value dimension")
    dv = o.shape[-1]
    _need(o, "o", tuple(o.shape), None, dev)
    _need(gate, "gate", tuple(o.shape), o.dtype, dev)
    _need(weight, "weight", (dv,), torch.float32, dev)
    out_dtype = o.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(o.shape, dtype=out_dtype, device=dev)
    _need(out, "out", tuple(o.shape), out_dtype, dev)
    rows = o.numel() // dv if dv else 0
    _check(_lib.kda_gated_rmsnorm(rows, dv, _dtype_code(o.dtype), _dtype_code(out_dtype), _ptr(o), _ptr(gate),
                                  _ptr(weight), float(eps), _ptr(out), _stream(dev)))
    return out


def short_conv(x: torch.Tensor, weight: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
               state: Optional[torch.Tensor] = None, *, silu: bool = True, output_final_state: bool = True,
               out: Optional[torch.Tensor] = None,
               final_state: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Short causal convolution before the core (``kda_short_conv``).

    x [T, C] (float32 or bfloat16); weight [K, C] in x's dtype; cu_seqlens
    [N+1] int32 (None: one request of T tokens); state [N, K-1, C] in x's
    dtype or None (zeros).  Returns (y [T, C], final state [N, K-1, C] or
    None).  ``final_state`` may be ``state`` itself (in place: each request
    then runs on one thread per 8 channels, which suits decode and short
    requests).  ``cu_seqlens=None`` builds [0, T] on the device on every call
    (a host-to-device copy): not for graph capture or allocation-free loops.
    """
    dev = x.device
    if dev.type != "cuda":
        raise KdaArgumentError(2, "tensors must be on a GPU device")
    if x.dim() != 2 or weight.dim() != 2:
        raise KdaArgumentError(2, "x must be [T, C] and weight [K, C]")
    T, C = x.shape
    K = weight.shape[0]
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=dev)
    N = cu_seqlens.numel() - 1
    _need(x, "x", (T, C), None, dev)
    _need(weight, "weight", (K, C), x.dtype, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if state is not None:
        _need(state, "state", (N, K - 1, C), x.dtype, dev)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", (T, C), x.dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, K - 1, C), dtype=x.dtype, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", (N, K - 1, C), x.dtype, dev)
    _check(_lib.kda_short_conv(N, T, C, K, _dtype_code(x.dtype), int(bool(silu)), _ptr(x), _ptr(weight),
                               _ptr(cu_seqlens), _ptr(state), _ptr(final_state), _ptr(out), _stream(dev)))
    return out, final_state


def recurrent_step_normed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, state: torch.Tensor, out_gate: torch.Tensor,
                          norm_weight: torch.Tensor, *, norm_eps: float = 1e-6,
                          a_log: Optional[torch.Tensor] = None, dt_bias: Optional[torch.Tensor] = None,
                          lower_bound: Optional[float] = None, scale: Optional[float] = None,
                          state_layout: str = "dk_dv", qk_l2norm: bool = True,
                          out_dtype: Optional[torch.dtype] = None,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step with the output epilogue fused (``kda_recurrent_step_normed``).

    As ``recurrent_step`` (or ``recurrent_step_gated`` when ``a_log`` and
    ``dt_bias`` are given, g and beta then being the raw projections), but the
    returned rows are o / sqrt(mean(o^2) + norm_eps) * norm_weight *
    sigmoid(out_gate); out_gate [N, H, dv] in q's dtype, norm_weight [dv] float32.
    """
    if q.dim() != 3:
        raise KdaArgumentError(2, f"q must be [N, H, dk], got {tuple(q.shape)}")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise KdaArgumentError(2, "tensors must be on a GPU device")
    _need(k, "k", (N, H, dk), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    gph, gshape = _gate_shape(g, (N, H), dk)
    gate = _gate_or_none(a_log, dt_bias, H, dk, lower_bound, dev, gph)
    gdt = torch.float32 if gate is None else q.dtype
    _need(g, "g", gshape, gdt, dev)
    _need(beta, "beta", (N, H), gdt, dev)
    _need(state, "state", (N, H, dk, dv), torch.float32, dev)
    _need(out_gate, "out_gate", (N, H, dv), q.dtype, dev)
    _need(norm_weight, "norm_weight", (dv,), torch.float32, dev)
    out_dtype = v.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    _need(out, "out", (N, H, dv), out_dtype, dev)
    prob = _problem(N, N, H, dk, dv, q.dtype, out_dtype, scale, qk_l2norm, gph, state_layout)
    _check(_lib.kda_recurrent_step_normed(ctypes.byref(prob), None if gate is None else ctypes.byref(gate),
                                          _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                          _ptr(out_gate), _ptr(norm_weight), float(norm_eps), _ptr(out),
                                          _stream(dev)))
    return out

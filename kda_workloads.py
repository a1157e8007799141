"""Seeded synthetic inputs for the Kimi Delta Attention (KDA) core.

This module only draws random tensors.  It holds none of the method's
arithmetic, so both the CPU oracle and the HIP path may consume what it makes.

Shapes and distributions follow the Kimi-Linear model pages: per head the
queries, keys and values are ``head_dim`` wide, the decay ``g`` is one
log-decay per key channel (the nnterp Kimi-Linear page, kimi_linear family
description: the forget gate is [batch, seq, heads, key_dim]), ``beta`` is one scalar per
token and head in [0, 1] (the Ascend model file, ``_prefill_torch_kda``:
``beta = sigmoid(raw_beta)``), and states are fp32 ``[num_seqs, H, dk, dv]``
(the Ascend model file, ``_forward_core``: fp32 zero prefill state).

Recipe (one CPU ``torch.Generator`` per workload, seed 0 unless given):

* draw order is fixed: sequence lengths (varlen only), q, k, v, x_g, x_beta,
  initial state;
* q, k, v ~ N(0, 1), rounded to bf16 by round-to-nearest-even when the
  workload is bf16 (the exact stored values are what every consumer sees);
* g = logsigmoid(x_g), x_g ~ N(mu_g, 1), fp32 (so g <= 0);
* beta = sigmoid(x_beta), x_beta ~ N(0, 1), fp32;
* initial state ~ N(0, 0.01**2) (standard deviation 0.01), fp32, or absent.

Raw gate inputs for the fused-gate entry points (``make_gate``, its own
generator): raw gate ~ N(mu, 0.5**2) and raw beta ~ N(0, 1), both rounded to
the q/k/v dtype; a_log = log(U(1, 16)) per head (the Ascend model file's
``A_log`` initialisation); dt_bias ~ N(0, 0.5**2) per head and channel, fp32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch
import torch.nn.functional as F


@dataclasses.dataclass
class PrefillInputs:
    """One packed-varlen prefill problem, all tensors on the CPU.

    q, k: [T, H, dk]; v: [T, H, dv]; g: [T, H, dk] fp32; beta: [T, H] fp32;
    cu_seqlens: [N+1] int32; initial_state: [N, H, dk, dv] fp32 or None.
    """

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    cu_seqlens: torch.Tensor
    initial_state: Optional[torch.Tensor]
    scale: float

    @property
    def num_seqs(self) -> int:
        return self.cu_seqlens.numel() - 1

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_heads(self) -> int:
        return self.q.shape[1]

    @property
    def head_k(self) -> int:
        return self.q.shape[2]

    @property
    def head_v(self) -> int:
        return self.v.shape[2]


@dataclasses.dataclass
class DecodeInputs:
    """A batch of independent sequences advanced one token per step.

    q, k: [steps, N, H, dk]; v: [steps, N, H, dv]; g: [steps, N, H, dk] fp32;
    beta: [steps, N, H] fp32; initial_state: [N, H, dk, dv] fp32.
    """

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    initial_state: torch.Tensor
    scale: float

    @property
    def steps(self) -> int:
        return self.q.shape[0]


def _qkv(gen, shape_k, shape_v, dtype):
    q = torch.randn(shape_k, generator=gen, dtype=torch.float32)
    k = torch.randn(shape_k, generator=gen, dtype=torch.float32)
    v = torch.randn(shape_v, generator=gen, dtype=torch.float32)
    if dtype != torch.float32:
        q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    return q, k, v


def make_prefill(
    lengths: List[int],
    num_heads: int,
    head_dim: int,
    dtype: torch.dtype = torch.bfloat16,
    g_mu: float = 2.0,
    state_std: Optional[float] = 0.01,
    seed: int = 0,
    name: str = "prefill",
    head_v: Optional[int] = None,
    gen: Optional[torch.Generator] = None,
) -> PrefillInputs:
    """Packed varlen prefill with the given per-sequence lengths.

    ``gen`` continues an existing generator (the varlen workload draws its
    lengths from it first); otherwise a fresh one is seeded with ``seed``.
    """
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    dv = head_dim if head_v is None else head_v
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    q, k, v = _qkv(gen, (T, num_heads, head_dim), (T, num_heads, dv), dtype)
    x_g = torch.randn((T, num_heads, head_dim), generator=gen, dtype=torch.float32)
    x_b = torch.randn((T, num_heads), generator=gen, dtype=torch.float32)
    g = F.logsigmoid(x_g + g_mu)
    beta = torch.sigmoid(x_b)
    s0 = None
    if state_std is not None:
        s0 = torch.randn((len(lengths), num_heads, head_dim, dv), generator=gen,
                         dtype=torch.float32) * state_std
    return PrefillInputs(name, q, k, v, g, beta, cu, s0, 1.0 / math.sqrt(head_dim))


def varlen_lengths(n: int, lo: int, hi: int, gen: torch.Generator) -> List[int]:
    """n integer lengths uniform on [lo, hi] inclusive."""
    return torch.randint(lo, hi + 1, (n,), generator=gen).tolist()


def make_decode(
    num_seqs: int,
    steps: int,
    num_heads: int,
    head_dim: int,
    dtype: torch.dtype = torch.bfloat16,
    g_mu: float = 2.0,
    state_std: float = 0.01,
    seed: int = 0,
    name: str = "decode",
) -> DecodeInputs:
    gen = torch.Generator().manual_seed(seed)
    shp = (steps, num_seqs, num_heads, head_dim)
    q, k, v = _qkv(gen, shp, shp, dtype)
    x_g = torch.randn(shp, generator=gen, dtype=torch.float32)
    x_b = torch.randn((steps, num_seqs, num_heads), generator=gen, dtype=torch.float32)
    g = F.logsigmoid(x_g + g_mu)
    beta = torch.sigmoid(x_b)
    s0 = torch.randn((num_seqs, num_heads, head_dim, head_dim), generator=gen,
                     dtype=torch.float32) * state_std
    return DecodeInputs(name, q, k, v, g, beta, s0, 1.0 / math.sqrt(head_dim))


# The five named workloads.  Sizes and distributions are the Kimi-Linear-shaped
# shapes (H=32 heads of 128 channels) plus one tiny fp32 case.

def tiny_fp32() -> PrefillInputs:
    """B=1, T=256, H=2, dk=dv=64, fp32, g=logsigmoid(N(2,1)), zero initial state."""
    return make_prefill([256], 2, 64, torch.float32, g_mu=2.0, state_std=None,
                        name="tiny_fp32_T256_H2_d64")


def prefill_4k() -> PrefillInputs:
    """B=1, T=4096, H=32, d=128, bf16, g=logsigmoid(N(3,1)), S0 ~ N(0, 0.01^2)."""
    return make_prefill([4096], 32, 128, torch.bfloat16, g_mu=3.0, state_std=0.01,
                        name="prefill_T4096_H32_d128")


def varlen8(seed: int = 0) -> PrefillInputs:
    """8 sequences, lengths U{512..8192}, H=32, d=128, bf16, g=logsigmoid(N(2,1))."""
    gen = torch.Generator().manual_seed(seed)
    lengths = varlen_lengths(8, 512, 8192, gen)
    return make_prefill(lengths, 32, 128, torch.bfloat16, g_mu=2.0, state_std=0.01,
                        name="varlen8_H32_d128", gen=gen)


def long_128k() -> PrefillInputs:
    """B=1, T=131072, H=32, d=128, bf16, g=logsigmoid(N(4,1)), zero initial state."""
    return make_prefill([131072], 32, 128, torch.bfloat16, g_mu=4.0, state_std=None,
                        name="long_T131072_H32_d128")


def decode_256x64() -> DecodeInputs:
    """256 sequences x 64 decode steps, H=32, d=128, bf16 q/k/v, g=logsigmoid(N(2,1))."""
    return make_decode(256, 64, 32, 128, torch.bfloat16, g_mu=2.0, state_std=0.01,
                       name="decode_N256_steps64_H32_d128")


@dataclasses.dataclass
class GateInputs:
    """Raw gate inputs: raw_g [rows, H, dk] and raw_beta [rows, H] in the
    q/k/v dtype, a_log [H] fp32, dt_bias [H, dk] fp32, lower_bound (None for
    the softplus gate)."""

    raw_g: torch.Tensor
    raw_beta: torch.Tensor
    a_log: torch.Tensor
    dt_bias: torch.Tensor
    lower_bound: Optional[float]


def make_gate(rows: int, num_heads: int, head_k: int, dtype: torch.dtype, *, mu: float = -5.0,
              lower_bound: Optional[float] = None, seed: int = 0, lead: tuple = (),
              per_head: bool = False, std: float = 0.5, dt_std: float = 0.5,
              a_log_value: Optional[float] = None) -> GateInputs:
    """Draw raw gate inputs of ``lead + (rows, num_heads, head_k)`` (``lead + (rows,
    num_heads)`` and dt_bias [H] with ``per_head``: one decay per head).

    raw gate ~ N(mu, std**2); dt_bias ~ N(0, dt_std**2) (``dt_std=0`` gives the
    zero bias); ``a_log_value`` replaces every head's log(U(1, 16)) draw by one
    value (the draw still happens, so the other tensors do not change)."""
    gen = torch.Generator().manual_seed(seed)
    ch = () if per_head else (head_k,)
    raw_g = (torch.randn(*lead, rows, num_heads, *ch, generator=gen) * std + mu).to(dtype)
    raw_beta = torch.randn(*lead, rows, num_heads, generator=gen).to(dtype)
    a_log = torch.log(torch.empty(num_heads).uniform_(1.0, 16.0, generator=gen))
    if a_log_value is not None:
        a_log = torch.full((num_heads,), float(a_log_value))
    dt_bias = torch.randn(num_heads, *ch, generator=gen) * dt_std
    return GateInputs(raw_g, raw_beta, a_log, dt_bias, lower_bound)


def per_head_decay(shape: tuple, g_mu: float = 2.0, seed: int = 0) -> torch.Tensor:
    """One log-decay per (token, head): logsigmoid(N(g_mu, 1)) of the given shape, fp32."""
    gen = torch.Generator().manual_seed(seed)
    return F.logsigmoid(torch.randn(shape, generator=gen, dtype=torch.float32) + g_mu)


@dataclasses.dataclass
class VerifyInputs:
    """Verify decode over a state pool.

    q, k: [N, W, H, dk]; v: [N, W, H, dv]; g: [N, W, H, dk] fp32; beta:
    [N, W, H] fp32; pool: [P, H, dk, dv] fp32; indices: [N, W] int32 (one
    slot per token, distinct over the whole call, a few replaced by -1 when
    ``pad`` > 0); accepted: [N] int32 in [1, W].
    """

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    pool: torch.Tensor
    indices: torch.Tensor
    accepted: torch.Tensor
    scale: float


def make_verify(num_seqs: int, width: int, num_heads: int, head_dim: int,
                dtype: torch.dtype = torch.bfloat16, g_mu: float = 2.0, state_std: float = 0.01,
                extra_slots: int = 3, pad: int = 0, seed: int = 0, name: str = "verify") -> VerifyInputs:
    """Draw a verify-decode batch; the pool has N*W + extra_slots slots, the
    indices are a random injection of the N*W tokens into it."""
    gen = torch.Generator().manual_seed(seed)
    shp = (num_seqs, width, num_heads, head_dim)
    q, k, v = _qkv(gen, shp, shp, dtype)
    x_g = torch.randn(shp, generator=gen, dtype=torch.float32)
    x_b = torch.randn((num_seqs, width, num_heads), generator=gen, dtype=torch.float32)
    g = F.logsigmoid(x_g + g_mu)
    beta = torch.sigmoid(x_b)
    P = num_seqs * width + extra_slots
    pool = torch.randn((P, num_heads, head_dim, head_dim), generator=gen, dtype=torch.float32) * state_std
    indices = torch.randperm(P, generator=gen)[: num_seqs * width].to(torch.int32).view(num_seqs, width)
    if pad > 0:
        flat = indices.view(-1)
        flat[torch.randperm(flat.numel(), generator=gen)[:pad]] = -1
    accepted = torch.randint(1, width + 1, (num_seqs,), generator=gen, dtype=torch.int32)
    return VerifyInputs(name, q, k, v, g, beta, pool, indices, accepted, 1.0 / math.sqrt(head_dim))


@dataclasses.dataclass
class ConvPrefillInputs:
    """A prefill whose q, k, v come out of the short convolution: x is the fused
    projection before it, [T, 3, H, d] (q, k, v blocks); weight [K, 3 H d];
    conv_state [N, K - 1, 3 H d] or None; the rest as PrefillInputs."""

    name: str
    x: torch.Tensor
    weight: torch.Tensor
    conv_state: Optional[torch.Tensor]
    g: torch.Tensor
    beta: torch.Tensor
    cu_seqlens: torch.Tensor
    initial_state: Optional[torch.Tensor]
    scale: float


def make_conv_prefill(lengths: List[int], num_heads: int, head_dim: int, kernel_size: int = 4,
                      dtype: torch.dtype = torch.bfloat16, g_mu: float = 3.0, conv_state: bool = True,
                      state_std: Optional[float] = 0.01, seed: int = 0,
                      name: str = "conv_prefill") -> ConvPrefillInputs:
    """x ~ N(0, 1), conv weight ~ N(0, 0.5^2), conv state ~ N(0, 1) (in dtype);
    g = logsigmoid(N(g_mu, 1)), beta = sigmoid(N(0, 1)) (float32); S0 ~ N(0, state_std^2)."""
    base = make_prefill(lengths, num_heads, head_dim, dtype, g_mu=g_mu, state_std=state_std, seed=seed, name=name)
    gen = torch.Generator().manual_seed(seed + 1000)
    T, N, C = base.q.shape[0], len(lengths), 3 * num_heads * head_dim
    x = torch.randn((T, 3, num_heads, head_dim), generator=gen).to(dtype)
    w = (torch.randn((kernel_size, C), generator=gen) * 0.5).to(dtype)
    s = torch.randn((N, kernel_size - 1, C), generator=gen).to(dtype) if conv_state else None
    return ConvPrefillInputs(name, x, w, s, base.g, base.beta, base.cu_seqlens, base.initial_state, base.scale)

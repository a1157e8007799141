#!/usr/bin/env python3
"""Benchmark of the KDA core on one MI355X.

A step is one chunked prefill (kda_chunk_fwd) over the Kimi-Linear-shaped
workload: one sequence of T=4096 tokens, H=32 heads, dk=dv=128, bf16 q/k/v,
fp32 g/beta, fp32 initial state, bf16 output.  ``value`` is prefill tokens/s
with inputs resident in HBM.  Three copies of the inputs rotate from step to
step so that the 256 MB Infinity Cache cannot serve a step's reads from the
previous one.

The decode kernel (kda_recurrent_step) is timed on its own workload, 256
sequences x 64 steps, H=32, d=128, and reported under ``decode``.  The other
two bf16 prefill workloads are reported under ``varlen8`` (8 packed sequences
of U{512..8192} tokens) and ``long_128k`` (one sequence of 131,072 tokens),
each far larger than the Infinity Cache, so one input copy serves.  The same
prefill workload through the fused-gate entry point (kda_chunk_fwd_gated: raw
bf16 gate and beta activated in the kernel) is reported under ``gated_prefill``.

Kernel durations come from a pair of HIP events around each leg's K back-to-back
launches, on the stream the kernels run on; ``roofline.achieved`` divides the
algorithmic bytes of one launch by the mean launch duration (the events'
interval over K).  Before its timed launches every leg
runs its own step untimed for ``settle_s`` seconds, after its W warmup steps:
the GPU's clocks rise only after some tens of milliseconds of sustained load.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + decode steps/s (H=32,d=128) and % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
# Algorithmic flops of the chunked form per (token, head) at C = 64, d = 128:
# 5 C d + 6 d^2 + (2/3) C^2 with triangles counted at half.
PREFILL_FLOPS_PER_TOKEN_HEAD = round(5 * 64 * 128 + 6 * 128 * 128 + 2 * 64 * 64 / 3)  # 141,995
PREFILL_BYTES_PER_TOKEN_HEAD = 3 * 128 * 2 + 128 * 4 + 4 + 128 * 2   # q,k,v bf16; g fp32; beta; out bf16
STATE_BYTES = 128 * 128 * 4
DECODE_BYTES_PER_HEAD_STEP = 2 * STATE_BYTES + PREFILL_BYTES_PER_TOKEN_HEAD
# fused gate: raw gate [dk] and raw beta in bf16 replace fp32 g and beta
GATED_BYTES_PER_TOKEN_HEAD = 3 * 128 * 2 + 128 * 2 + 2 + 128 * 2
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "prefill": ["gated_delta_rule_53_amd/csrc/kda_prefill_split.hip", "gated_delta_rule_53_amd/csrc/kda_bf16_mfma.h",
                "gated_delta_rule_53_amd/csrc/kda_common.h"],
    "decode": ["gated_delta_rule_53_amd/csrc/kda_decode.hip", "gated_delta_rule_53_amd/csrc/kda_bf16_mfma.h",
               "gated_delta_rule_53_amd/csrc/kda_common.h"],
}
KERNEL_SOURCES["gated_prefill"] = KERNEL_SOURCES["prefill"]
KERNEL_SOURCES["prefill_varlen8"] = KERNEL_SOURCES["prefill"]
KERNEL_SOURCES["prefill_long128k"] = KERNEL_SOURCES["prefill"]
KERNEL_SOURCES["per_head_prefill"] = KERNEL_SOURCES["prefill"]
KERNEL_SOURCES["prefill_conv"] = KERNEL_SOURCES["prefill"] + ["gated_delta_rule_53_amd/csrc/kda_conv.hip"]
KERNEL_SOURCES["verify_decode"] = KERNEL_SOURCES["decode"]
KERNEL_SOURCES["verify_normed"] = KERNEL_SOURCES["decode"]
KERNEL_SOURCES["decode_dv_dk"] = KERNEL_SOURCES["decode"]
KERNEL_SOURCES["prologue"] = ["gated_delta_rule_53_amd/csrc/kda_conv.hip", "gated_delta_rule_53_amd/csrc/kda_common.h"]
KERNEL_SOURCES["epilogue"] = ["gated_delta_rule_53_amd/csrc/kda_epilogue.hip", "gated_delta_rule_53_amd/csrc/kda_common.h"]
# kernels launched by one kda_chunk_fwd call on the bf16, d=128 path
# one chain per (sequence, head, 16-column tile): chain_kernel while every tile
# has a compute unit, scan_kernel (two tiles per workgroup) beyond that
# one sequence, every chain on compute units of its own: prep and the chain pass find the
# chunks themselves (no chunk-map launch)
PREFILL_KERNELS = ["prep_kernel", "chain_kernel"]
PREFILL_KERNELS_MANY = ["chunk_map_kernel", "prep_kernel", "scan_kernel"]


def source_digest(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kind: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[kind]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_digest") != source_digest(kind):
        return None
    return rec.get("bytes_per_launch")


# The GPU raises its clocks only after some tens of milliseconds of sustained load:
# on a 4096-token prefill the first ~100 calls after idle ran at 160-180 us, the
# following ones at ~150 us.  Each leg therefore runs its own step untimed for at
# least this long before its K timed launches (after its W warmup steps), so that
# the timed launches see the clocks that a caller issuing work back to back sees.
SETTLE_S = 0.2


def settle(fn, seconds: float = SETTLE_S) -> int:
    """Call fn(i) untimed until `seconds` of wall time have passed; returns the call count."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return i


def time_launches(fn, n: int, stream):
    """Run fn() n times back to back; returns (wall seconds, mean per-launch seconds).

    The leg's step is first run untimed for SETTLE_S seconds (settle()).  One
    pair of HIP events on the kernels' stream brackets the n launches, and the
    mean launch duration is their interval over n: it includes whatever gaps the
    GPU leaves between launches, and no event markers are placed between them
    (a marker per launch left the GPU idle about 5 us per launch)."""
    import torch
    settle(fn)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(n):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = start.elapsed_time(end) / n / 1e3
    return wall, per


PER_HEAD_BYTES_PER_TOKEN_HEAD = 3 * 128 * 2 + 4 + 4 + 128 * 2   # g is one fp32 per (token, head)


def bench_prefill(steps: int, warmup: int, per_head: bool = False):
    """kda_chunk_fwd on the T=4096, H=32, d=128 workload; per_head: g [T, H] (one decay per head)."""
    import torch

    import gated_delta_rule_53_amd as kda
    import kda_workloads as w

    x = w.prefill_4k()
    g_in = w.per_head_decay((x.total_tokens, x.num_heads), 3.0, seed=1) if per_head else x.g
    dev = "cuda:0"
    copies = []
    for _ in range(3):
        copies.append(dict(q=x.q.to(dev), k=x.k.to(dev), v=x.v.to(dev), g=g_in.to(dev),
                           beta=x.beta.to(dev), cu=x.cu_seqlens.to(dev),
                           s0=x.initial_state.to(dev),
                           out=torch.empty_like(x.v, device=dev),
                           fs=torch.empty_like(x.initial_state, device=dev)))
    prob = kda.Problem(total_tokens=x.total_tokens, num_seqs=x.num_seqs, num_heads=x.num_heads,
                       head_k=x.head_k, head_v=x.head_v, qkv_dtype=1, out_dtype=1,
                       scale=x.scale, qk_l2norm=1, chunk_size=64, gate_per_head=int(per_head))
    workspace = torch.empty(max(kda.chunk_fwd_workspace_bytes(prob), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        c = copies[i % 3]
        kda.chunk_fwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["cu"], c["s0"],
                      scale=x.scale, out=c["out"], final_state=c["fs"], workspace=workspace)

    for i in range(warmup):
        step(i)
    wall, per = time_launches(step, steps, stream)
    T, H = x.total_tokens, x.num_heads
    per_token = PER_HEAD_BYTES_PER_TOKEN_HEAD if per_head else PREFILL_BYTES_PER_TOKEN_HEAD
    alg_bytes = T * H * per_token + x.num_seqs * H * 2 * STATE_BYTES
    return dict(x=x, wall=wall, per_launch=per, alg_bytes=alg_bytes, tokens=T,
                workspace_bytes=workspace.numel())


def bench_prefill_workload(x, steps: int, warmup: int):
    """kda_chunk_fwd on one of the larger bf16 workloads (one input copy: each
    is several GB, far beyond the 256 MB Infinity Cache)."""
    import torch

    import gated_delta_rule_53_amd as kda

    dev = "cuda:0"
    q, k, v, g, b, cu = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens))
    s0 = None if x.initial_state is None else x.initial_state.to(dev)
    out = torch.empty_like(v)
    fs = torch.empty((x.num_seqs, x.num_heads, x.head_k, x.head_v), device=dev)
    prob = kda.Problem(total_tokens=x.total_tokens, num_seqs=x.num_seqs, num_heads=x.num_heads,
                       head_k=x.head_k, head_v=x.head_v, qkv_dtype=1, out_dtype=1,
                       scale=x.scale, qk_l2norm=1, chunk_size=64)
    workspace = torch.empty(max(kda.chunk_fwd_workspace_bytes(prob), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        kda.chunk_fwd(q, k, v, g, b, cu, s0, scale=x.scale, out=out, final_state=fs, workspace=workspace)

    for i in range(warmup):
        step(i)
    wall, per = time_launches(step, steps, stream)
    T, H, N = x.total_tokens, x.num_heads, x.num_seqs
    states = (2 if s0 is not None else 1) * N * H * STATE_BYTES
    alg_bytes = T * H * PREFILL_BYTES_PER_TOKEN_HEAD + states
    res = dict(x=x, wall=wall, per_launch=per, alg_bytes=alg_bytes, tokens=T,
               flops=T * H * PREFILL_FLOPS_PER_TOKEN_HEAD)
    del q, k, v, g, b, out, fs, workspace
    torch.cuda.empty_cache()
    return res


def prefill_roofline(kernel: str, r, traffic):
    """HBM roofline of one prefill call, with the MFMA fraction of the same call beside it."""
    achieved = r["alg_bytes"] / r["per_launch"] / 1e9
    tflops = r["flops"] / r["per_launch"] / 1e12
    return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic / r["per_launch"] / 1e9, 2),
            "traffic_bytes_per_launch": traffic, "alg_bytes_per_launch": r["alg_bytes"],
            "launch_us": round(r["per_launch"] * 1e6, 2),
            "mfma_achieved_tflops": round(tflops, 2), "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "alg_flops_per_launch": r["flops"]}


CONV_K = 4


def bench_prefill_conv(steps: int, warmup: int):
    """kda_chunk_fwd_conv (short convolution fused into the prefill's loads) on
    the T=4096, H=32, d=128 prefill with K=4 and SiLU, beside the unfused pair
    (kda_short_conv on the fused projection, then kda_chunk_fwd on its split
    output).  Three input copies in turn, as for the plain prefill."""
    import torch

    import gated_delta_rule_53_amd as kda
    import kda_workloads as w

    x = w.make_conv_prefill([4096], 32, 128, CONV_K, seed=0, name="conv_prefill_T4096_H32_d128_K4")
    dev = "cuda:0"
    T, _, H, d = x.x.shape
    C = 3 * H * d
    copies = []
    for _ in range(3):
        copies.append(dict(x=x.x.to(dev), g=x.g.to(dev), b=x.beta.to(dev), s0=x.initial_state.to(dev),
                           cs=x.conv_state.to(dev), cs_out=torch.empty_like(x.conv_state, device=dev),
                           out=torch.empty((T, H, d), dtype=torch.bfloat16, device=dev),
                           fs=torch.empty_like(x.initial_state, device=dev)))
    w_, cu = x.weight.to(dev), x.cu_seqlens.to(dev)
    prob = kda.Problem(total_tokens=T, num_seqs=1, num_heads=H, head_k=d, head_v=d, qkv_dtype=1, out_dtype=1,
                       scale=x.scale, qk_l2norm=1, chunk_size=64)
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    y = torch.empty((T, C), dtype=torch.bfloat16, device=dev)
    # the convolved q, k, v of each input copy (three copies in turn, as for the fused call)
    qkv = [[torch.empty((T, H, d), dtype=torch.bfloat16, device=dev) for _ in range(3)] for _ in range(3)]
    stream = torch.cuda.current_stream()

    def fused(i):
        c = copies[i % 3]
        kda.chunk_fwd_conv(c["x"], c["g"], c["b"], w_, cu, c["s0"], c["cs"], conv_state_out=c["cs_out"],
                           scale=x.scale, out=c["out"], final_state=c["fs"], workspace=ws)

    # the unfused pair, timed launch by launch (the split of y into contiguous
    # q, k, v that kda_chunk_fwd takes is left out: done once, outside)
    def conv_only(i):
        c = copies[i % 3]
        kda.short_conv(c["x"].view(T, C), w_, cu, c["cs"], silu=True, out=y, final_state=c["cs_out"])

    def core_only(i):
        c, q3 = copies[i % 3], qkv[i % 3]
        kda.chunk_fwd(q3[0], q3[1], q3[2], c["g"], c["b"], cu, c["s0"], scale=x.scale, out=c["out"],
                      final_state=c["fs"], workspace=ws)

    for i in range(warmup):
        fused(i)
    wall, per = time_launches(fused, steps, stream)
    yv = y.view(T, 3, H, d)
    for i in range(3):
        conv_only(i)
        for j in range(3):
            qkv[i][j].copy_(yv[:, j])
    for i in range(warmup):
        conv_only(i)
        core_only(i)
    _, per_c = time_launches(conv_only, steps, stream)
    _, per_p = time_launches(core_only, steps, stream)
    per_u = per_c + per_p
    states = 2 * H * STATE_BYTES + 2 * (CONV_K - 1) * C * 2
    alg_bytes = T * H * PREFILL_BYTES_PER_TOKEN_HEAD + states
    # the unfused pair also writes the convolved q/k/v and reads them back (the split copy aside)
    alg_bytes_unfused = alg_bytes + 2 * T * C * 2
    return dict(x=x, wall=wall, per_launch=per, per_launch_unfused=per_u, alg_bytes=alg_bytes,
                alg_bytes_unfused=alg_bytes_unfused, tokens=T, flops=T * H * PREFILL_FLOPS_PER_TOKEN_HEAD)


def bench_prefill_gated(steps: int, warmup: int):
    import torch

    import gated_delta_rule_53_amd as kda
    import kda_workloads as w

    x = w.prefill_4k()
    T, H = x.total_tokens, x.num_heads
    gi = w.make_gate(T, H, x.head_k, torch.bfloat16, seed=1)
    dev = "cuda:0"
    copies = []
    for _ in range(3):
        copies.append(dict(q=x.q.to(dev), k=x.k.to(dev), v=x.v.to(dev), rg=gi.raw_g.to(dev),
                           rb=gi.raw_beta.to(dev), cu=x.cu_seqlens.to(dev), s0=x.initial_state.to(dev),
                           out=torch.empty_like(x.v, device=dev),
                           fs=torch.empty_like(x.initial_state, device=dev)))
    a_log, dt_bias = gi.a_log.to(dev), gi.dt_bias.to(dev)
    prob = kda.Problem(total_tokens=T, num_seqs=x.num_seqs, num_heads=H, head_k=x.head_k, head_v=x.head_v,
                       qkv_dtype=1, out_dtype=1, scale=x.scale, qk_l2norm=1, chunk_size=64)
    workspace = torch.empty(max(kda.chunk_fwd_workspace_bytes(prob), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        c = copies[i % 3]
        kda.chunk_fwd_gated(c["q"], c["k"], c["v"], c["rg"], c["rb"], a_log, dt_bias, c["cu"], c["s0"],
                            scale=x.scale, out=c["out"], final_state=c["fs"], workspace=workspace)

    for i in range(warmup):
        step(i)
    wall, per = time_launches(step, steps, stream)
    alg_bytes = T * H * GATED_BYTES_PER_TOKEN_HEAD + x.num_seqs * H * 2 * STATE_BYTES
    return dict(x=x, wall=wall, per_launch=per, alg_bytes=alg_bytes, tokens=T)


def bench_decode(loops: int, state_layout: str = "dk_dv"):
    """kda_recurrent_step, 256 sequences x 64 steps; state_layout "dv_dk" keeps the states transposed."""
    import torch

    import gated_delta_rule_53_amd as kda
    import kda_workloads as w

    x = w.decode_256x64()
    dev = "cuda:0"
    q, k, v, g, b = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.beta))
    st = x.initial_state.to(dev)
    if state_layout == "dv_dk":
        st = st.transpose(-1, -2).contiguous()
    out = torch.empty_like(v[0])
    stream = torch.cuda.current_stream()

    def one(i):
        t = i % x.steps
        kda.recurrent_step(q[t], k[t], v[t], g[t], b[t], st, scale=x.scale, out=out, state_layout=state_layout)

    for i in range(x.steps):  # warm-up pass over all 64 steps
        one(i)
    n = loops * x.steps
    wall, per = time_launches(one, n, stream)
    N, H = x.q.shape[1], x.q.shape[2]
    alg_bytes = N * H * DECODE_BYTES_PER_HEAD_STEP
    return dict(x=x, wall=wall, per_launch=per, launches=n, alg_bytes=alg_bytes, num_seqs=N)


EPILOGUE_BYTES_PER_ROW = 3 * 128 * 2   # o and gate read, y written, bf16


def bench_epilogue(steps: int, warmup: int):
    """kda_gated_rmsnorm on the core's output shape: T=4096, H=32, dv=128, bf16 in and out."""
    import torch

    import gated_delta_rule_53_amd as kda

    T, H, dv = 4096, 32, 128
    gen = torch.Generator().manual_seed(3)
    dev = "cuda:0"
    copies = []
    for _ in range(3):
        copies.append(dict(o=torch.randn((T, H, dv), generator=gen).to(torch.bfloat16).to(dev),
                           g=torch.randn((T, H, dv), generator=gen).to(torch.bfloat16).to(dev),
                           y=torch.empty((T, H, dv), dtype=torch.bfloat16, device=dev)))
    w = torch.ones(dv, device=dev)
    stream = torch.cuda.current_stream()

    def one(i):
        c = copies[i % 3]
        kda.gated_rmsnorm(c["o"], c["g"], w, eps=1e-6, out=c["y"])

    for i in range(warmup):
        one(i)
    wall, per = time_launches(one, steps, stream)
    return dict(wall=wall, per_launch=per, alg_bytes=T * H * EPILOGUE_BYTES_PER_ROW, tokens=T)


def bench_conv(steps: int, warmup: int):
    """kda_short_conv on the fused q/k/v projection of the prefill workload: T=4096,
    C = 3 * 32 * 128, 4 taps, bf16, SiLU, one request with a starting state."""
    import torch

    import gated_delta_rule_53_amd as kda

    T, C, K = 4096, 3 * 32 * 128, 4
    gen = torch.Generator().manual_seed(4)
    dev = "cuda:0"
    copies = [dict(x=torch.randn((T, C), generator=gen).to(torch.bfloat16).to(dev),
                   y=torch.empty((T, C), dtype=torch.bfloat16, device=dev)) for _ in range(3)]
    w = (torch.randn((K, C), generator=gen) * 0.5).to(torch.bfloat16).to(dev)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    s0 = torch.zeros((1, K - 1, C), dtype=torch.bfloat16, device=dev)
    s1 = torch.empty_like(s0)
    stream = torch.cuda.current_stream()

    def one(i):
        c = copies[i % 3]
        kda.short_conv(c["x"], w, cu, s0, out=c["y"], final_state=s1)

    for i in range(warmup):
        one(i)
    wall, per = time_launches(one, steps, stream)
    # x read and y written once; weights and states are negligible
    return dict(wall=wall, per_launch=per, alg_bytes=2 * T * C * 2, tokens=T)


VERIFY_WIDTH = 4


def bench_verify(steps: int, warmup: int, normed: bool = False):
    """Verify decode over a state pool: 256 sequences x 4 tokens, H=32, d=128, bf16.

    normed: kda_recurrent_verify_normed (gated RMSNorm fused); the unfused pair
    (kda_recurrent_verify, then kda_gated_rmsnorm on its bf16 output) is timed
    beside it."""
    import torch

    import gated_delta_rule_53_amd as kda
    import kda_workloads as w

    x = w.make_verify(256, VERIFY_WIDTH, 32, 128, torch.bfloat16, g_mu=2.0, extra_slots=0, seed=7,
                      name="verify_N256_W4_H32_d128")
    dev = "cuda:0"
    q, k, v, g, b, idx, acc = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.beta, x.indices, x.accepted))
    pool = x.pool.to(dev)
    out = torch.empty_like(v)
    stream = torch.cuda.current_stream()
    gen = torch.Generator().manual_seed(8)
    og = torch.randn(tuple(v.shape), generator=gen).to(torch.bfloat16).to(dev)
    nw = (1.0 + 0.1 * torch.randn((v.shape[-1],), generator=gen)).to(dev)
    y = torch.empty_like(v)

    def one(i):
        if normed:
            kda.recurrent_verify_normed(q, k, v, g, b, pool, idx, og, nw, acc, scale=x.scale, out=out)
        else:
            kda.recurrent_verify(q, k, v, g, b, pool, idx, acc, scale=x.scale, out=out)

    def unfused(i):
        kda.recurrent_verify(q, k, v, g, b, pool, idx, acc, scale=x.scale, out=out)
        kda.gated_rmsnorm(out, og, nw, eps=1e-6, out=y)

    for i in range(warmup):
        one(i)
    wall, per = time_launches(one, steps, stream)
    N, W, H = x.q.shape[:3]
    dv = x.v.shape[-1]
    # per (sequence, head): the starting state read, one state written per token, the token I/O
    # (normed: plus the output-gate row each token reads)
    alg_bytes = N * H * ((1 + W) * STATE_BYTES + W * PREFILL_BYTES_PER_TOKEN_HEAD + (W * dv * 2 if normed else 0))
    res = dict(x=x, wall=wall, per_launch=per, alg_bytes=alg_bytes, tokens=N * W)
    if normed:
        for i in range(warmup):
            unfused(i)
        _, per_u = time_launches(unfused, steps, stream)
        # the unfused pair also writes o and reads it back: two more bf16 rows per token-head
        res.update(per_launch_unfused=per_u, alg_bytes_unfused=alg_bytes + 2 * N * W * H * dv * 2)
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(min_seconds: float = 8.0, heads: int = 0, threads: int = 0):
    """The fp64 oracle on the host cores, over whole passes of the same prefill workload
    (``heads``: only the first so many heads, for a bounded single-core sample;
    ``threads``: the oracle's OpenMP thread count, 0 for its default)."""
    import kda_workloads as w
    import oracle
    if threads > 0:
        oracle.set_threads(threads)
    x = w.prefill_4k()
    H = x.num_heads if heads <= 0 else heads
    sl = lambda t: t[:, :H].contiguous()
    s0 = x.initial_state[:, :H].contiguous()
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), x.cu_seqlens, s0, scale=x.scale)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or passes >= 50:
            break
    # tokens/s of the whole workload (all 32 heads): heads are independent and equal in work
    value = passes * x.total_tokens * H / x.num_heads / el
    # the oracle's threads each take whole (sequence, head) pairs: at most that many work
    return dict(value=value, unit="tokens/s", cores=min(oracle.threads(), x.num_seqs * H), kind="oracle",
                sample=f"{passes} pass(es) of prefill_T4096_H32_d128 over {H} of {x.num_heads} heads "
                       f"(fp64 recurrence, {el:.1f} s wall), scaled to all heads")


def cpu_baseline_single_core():
    """The same oracle on one core: one head, so one (sequence, head) pair and
    one busy thread whatever the OpenMP thread count (set to 16 on the GPU
    hosts), scaled to all heads."""
    return cpu_baseline(min_seconds=6.0, heads=1)


def hbm_copy_bandwidth(gib: int = 2, reps: int = 10):
    """A plain device-to-device copy: the practical HBM rate beside the 8 TB/s peak."""
    import torch
    n = gib * (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    wall, per = time_launches(lambda i: dst.copy_(src), reps, torch.cuda.current_stream())
    del src, dst
    torch.cuda.empty_cache()
    gbs = 2 * n * 4 / per / 1e9
    # write-only: the rate a store-dominated kernel (verify writes 4 states per read) can reach
    dst = torch.empty(n, dtype=torch.float32, device="cuda:0")
    for _ in range(2):
        dst.zero_()
    _, per_w = time_launches(lambda i: dst.zero_(), reps, torch.cuda.current_stream())
    del dst
    torch.cuda.empty_cache()
    wgbs = n * 4 / per_w / 1e9
    return {"kernel": "torch copy_ (read + write)", "bytes_per_launch": 2 * n * 4, "gbs": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "write_only": {"kernel": "torch zero_ (write)", "bytes_per_launch": n * 4, "gbs": round(wgbs, 1),
                           "frac_of_peak": round(wgbs / HBM_PEAK_GBS, 4)}}


def copy_calibration(gib: int = 1, reps: int = 4):
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = gib * (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n * 4,
                                           "bytes_written_per_launch": n * 4, "launches": reps}}))


def _wl(name):
    import kda_workloads as w
    return getattr(w, name)()


# One leg at a time (--leg), for profiler runs that must see one workload.
LEGS = {
    "prefill": lambda a: bench_prefill(a.steps, a.warmup),
    "prefill_varlen8": lambda a: bench_prefill_workload(_wl("varlen8"), min(a.steps, 10), 1),
    "prefill_long128k": lambda a: bench_prefill_workload(_wl("long_128k"), min(a.steps, 5), 1),
    "per_head_prefill": lambda a: bench_prefill(a.steps, a.warmup, per_head=True),
    "gated_prefill": lambda a: bench_prefill_gated(a.steps, a.warmup),
    "prefill_conv": lambda a: bench_prefill_conv(a.steps, a.warmup),
    "decode": lambda a: bench_decode(a.decode_loops),
    "decode_dv_dk": lambda a: bench_decode(1, state_layout="dv_dk"),
    "verify_decode": lambda a: bench_verify(a.steps, a.warmup),
    "verify_normed": lambda a: bench_verify(a.steps, a.warmup, normed=True),
    "prologue": lambda a: bench_conv(a.steps, a.warmup),
    "epilogue": lambda a: bench_epilogue(a.steps, a.warmup),
}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-loops", type=int, default=4, help="timed passes over the 64 decode steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--leg", choices=sorted(LEGS),
                    help="only run this leg (for per-workload profiler runs); prints its launch time")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the KDA core "
              "shards heads and sequences with no exchange, so more GPUs would only repeat this "
              "measurement per GPU).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.leg:
        r = LEGS[args.leg](args)
        print(json.dumps({"leg": args.leg, "launch_us": round(r["per_launch"] * 1e6, 2),
                          "alg_bytes_per_launch": r.get("alg_bytes")}), flush=True)
        return

    pf = bench_prefill(args.steps, args.warmup)
    pf["flops"] = pf["tokens"] * 32 * PREFILL_FLOPS_PER_TOKEN_HEAD
    print(f"prefill: {pf['per_launch'] * 1e6:.1f} us per launch (events), "
          f"{pf['wall'] / args.steps * 1e6:.1f} us per step (wall)", file=sys.stderr, flush=True)
    import kda_workloads as w
    v8 = bench_prefill_workload(w.varlen8(), min(args.steps, 10), 1)
    print(f"varlen8 prefill: {v8['per_launch'] * 1e3:.3f} ms per launch (events)", file=sys.stderr, flush=True)
    lg = bench_prefill_workload(w.long_128k(), min(args.steps, 5), 1)
    print(f"long_128k prefill: {lg['per_launch'] * 1e3:.3f} ms per launch (events)", file=sys.stderr, flush=True)
    cp = hbm_copy_bandwidth()
    print(f"device copy: {cp['gbs']} GB/s", file=sys.stderr, flush=True)
    dc = bench_decode(args.decode_loops)
    dt = bench_decode(1, state_layout="dv_dk")
    print(f"decode, transposed states: {dt['per_launch'] * 1e6:.1f} us per launch (events)", file=sys.stderr,
          flush=True)
    dt_achieved = dt["alg_bytes"] / dt["per_launch"] / 1e9
    dt_tr = measured_traffic("decode_dv_dk")
    vf = bench_verify(args.steps, args.warmup)
    ph = bench_prefill(args.steps, args.warmup, per_head=True)
    print(f"per-head prefill: {ph['per_launch'] * 1e6:.1f} us per launch (events)", file=sys.stderr, flush=True)
    ph_achieved = ph["alg_bytes"] / ph["per_launch"] / 1e9
    ph_tr = measured_traffic("per_head_prefill")
    print(f"verify decode: {vf['per_launch'] * 1e6:.1f} us per launch (events)", file=sys.stderr, flush=True)
    v_achieved = vf["alg_bytes"] / vf["per_launch"] / 1e9
    v_tr = measured_traffic("verify_decode")
    vn = bench_verify(args.steps, args.warmup, normed=True)
    print(f"verify decode + fused gated rmsnorm: {vn['per_launch'] * 1e6:.1f} us per launch; unfused pair "
          f"{vn['per_launch_unfused'] * 1e6:.1f} us (events)", file=sys.stderr, flush=True)
    vn_achieved = vn["alg_bytes"] / vn["per_launch"] / 1e9
    vn_tr = measured_traffic("verify_normed")
    print(f"decode: {dc['per_launch'] * 1e6:.1f} us per launch (events)", file=sys.stderr, flush=True)
    cv = bench_conv(args.steps, args.warmup)
    print(f"short conv prologue: {cv['per_launch'] * 1e6:.1f} us per launch (events)", file=sys.stderr, flush=True)
    cv_achieved = cv["alg_bytes"] / cv["per_launch"] / 1e9
    cv_tr = measured_traffic("prologue")
    ep = bench_epilogue(args.steps, args.warmup)
    print(f"gated rmsnorm epilogue: {ep['per_launch'] * 1e6:.1f} us per launch (events)", file=sys.stderr, flush=True)
    ep_achieved = ep["alg_bytes"] / ep["per_launch"] / 1e9
    ep_tr = measured_traffic("epilogue")
    gp = bench_prefill_gated(args.steps, args.warmup)
    print(f"gated prefill: {gp['per_launch'] * 1e6:.1f} us per launch (events)", file=sys.stderr, flush=True)
    g_achieved = gp["alg_bytes"] / gp["per_launch"] / 1e9
    g_tr = measured_traffic("gated_prefill")
    pc = bench_prefill_conv(args.steps, args.warmup)
    print(f"prefill with fused conv: {pc['per_launch'] * 1e6:.1f} us per launch; unfused conv + prefill "
          f"{pc['per_launch_unfused'] * 1e6:.1f} us (events)", file=sys.stderr, flush=True)
    pc_tr = measured_traffic("prefill_conv")

    ms_per_step = pf["wall"] / args.steps * 1e3
    tokens_per_s = pf["tokens"] * args.steps / pf["wall"]
    achieved = pf["alg_bytes"] / pf["per_launch"] / 1e9
    tr = measured_traffic("prefill")
    d_achieved = dc["alg_bytes"] / dc["per_launch"] / 1e9
    d_tr = measured_traffic("decode")
    decode_steps_per_s = dc["launches"] / dc["wall"]

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_note": "MFMA on fp16/bf16 operands (fp16 hi/lo pairs for the state side, bf16 hi/lo "
                      "where fp32 accuracy is needed in the chunk pass), fp32 accumulation and fp32 state",
        "data": "synthetic",
        "config": {"workload": pf["x"].name, "num_seqs": 1, "seq_len": pf["tokens"],
                   "heads": 32, "head_dim": 128, "chunk": 64, "qkv": "bf16", "g_beta": "f32",
                   "state": "f32", "out": "bf16", "input_copies_rotated": 3},
        "roofline": {**prefill_roofline("kda_chunk_fwd = " + " + ".join(PREFILL_KERNELS), pf, tr),
                     "workspace_bytes": pf["workspace_bytes"]},
        "hbm_copy": cp,
        "varlen8": {"workload": v8["x"].name, "tokens": v8["tokens"], "num_seqs": v8["x"].num_seqs,
                    "tokens_per_s": round(v8["tokens"] / v8["per_launch"], 1),
                    "ms_per_call": round(v8["per_launch"] * 1e3, 4),
                    "roofline": prefill_roofline("kda_chunk_fwd = " + " + ".join(PREFILL_KERNELS_MANY), v8,
                                                 measured_traffic("prefill_varlen8"))},
        "long_128k": {"workload": lg["x"].name, "tokens": lg["tokens"],
                      "tokens_per_s": round(lg["tokens"] / lg["per_launch"], 1),
                      "ms_per_call": round(lg["per_launch"] * 1e3, 4), "target_ms": 2.0,
                      "roofline": prefill_roofline("kda_chunk_fwd = " + " + ".join(PREFILL_KERNELS), lg,
                                                   measured_traffic("prefill_long128k"))},
        "decode": {"workload": dc["x"].name, "steps_per_s": round(decode_steps_per_s, 1),
                   "tokens_per_s": round(decode_steps_per_s * dc["num_seqs"], 1),
                   "roofline": {"kernel": "decode_step_kernel", "bound": "hbm",
                                "achieved": round(d_achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(d_achieved / HBM_PEAK_GBS, 4),
                                "traffic": None if d_tr is None else round(d_tr / dc["per_launch"] / 1e9, 2), "traffic_bytes_per_launch": d_tr,
                                "alg_bytes_per_launch": dc["alg_bytes"],
                                "launch_us": round(dc["per_launch"] * 1e6, 2)}},
        "decode_dv_dk": {"workload": dt["x"].name + "_state_dv_dk",
                         "steps_per_s": round(dt["launches"] / dt["wall"], 1),
                         "roofline": {"kernel": "decode_step_kernel (state_layout dv_dk)", "bound": "hbm",
                                      "achieved": round(dt_achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(dt_achieved / HBM_PEAK_GBS, 4),
                                      "traffic": None if dt_tr is None else round(dt_tr / dt["per_launch"] / 1e9, 2),
                                      "traffic_bytes_per_launch": dt_tr,
                                      "alg_bytes_per_launch": dt["alg_bytes"],
                                      "launch_us": round(dt["per_launch"] * 1e6, 2)}},
        "prologue": {"workload": "short_conv_T4096_C12288_K4_bf16_silu",
                     "tokens_per_s": round(cv["tokens"] * args.steps / cv["wall"], 1),
                     "roofline": {"kernel": "short_conv_kernel", "bound": "hbm",
                                  "achieved": round(cv_achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(cv_achieved / HBM_PEAK_GBS, 4),
                                  "traffic": None if cv_tr is None else round(cv_tr / cv["per_launch"] / 1e9, 2),
                                  "traffic_bytes_per_launch": cv_tr,
                                  "alg_bytes_per_launch": cv["alg_bytes"],
                                  "launch_us": round(cv["per_launch"] * 1e6, 2)}},
        "epilogue": {"workload": "gated_rmsnorm_T4096_H32_dv128_bf16",
                     "tokens_per_s": round(ep["tokens"] * args.steps / ep["wall"], 1),
                     "roofline": {"kernel": "gated_rmsnorm_kernel", "bound": "hbm",
                                  "achieved": round(ep_achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(ep_achieved / HBM_PEAK_GBS, 4),
                                  "traffic": None if ep_tr is None else round(ep_tr / ep["per_launch"] / 1e9, 2),
                                  "traffic_bytes_per_launch": ep_tr,
                                  "alg_bytes_per_launch": ep["alg_bytes"],
                                  "launch_us": round(ep["per_launch"] * 1e6, 2)}},
        "prefill_conv": {"workload": pc["x"].name + "_silu",
                         "tokens_per_s": round(pc["tokens"] * args.steps / pc["wall"], 1),
                         "unfused_us": round(pc["per_launch_unfused"] * 1e6, 2),
                         "unfused_alg_bytes": pc["alg_bytes_unfused"],
                         "roofline": prefill_roofline("kda_chunk_fwd_conv = prep_kernel (CONV) + "
                                                      "chain_kernel (CONV, writes the conv state)", pc, pc_tr)},
        "gated_prefill": {"workload": gp["x"].name + "_raw_bf16_gate",
                          "tokens_per_s": round(gp["tokens"] * args.steps / gp["wall"], 1),
                          "roofline": {"kernel": "kda_chunk_fwd_gated = " + " + ".join(PREFILL_KERNELS),
                                       "bound": "hbm", "achieved": round(g_achieved, 2), "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": round(g_achieved / HBM_PEAK_GBS, 4),
                                       "traffic": None if g_tr is None else round(g_tr / gp["per_launch"] / 1e9, 2), "traffic_bytes_per_launch": g_tr,
                                       "alg_bytes_per_launch": gp["alg_bytes"],
                                       "launch_us": round(gp["per_launch"] * 1e6, 2)}},
        "per_head_prefill": {"workload": ph["x"].name + "_g_per_head",
                             "tokens_per_s": round(ph["tokens"] * args.steps / ph["wall"], 1),
                             "roofline": {"kernel": "kda_chunk_fwd (gate_per_head) = " + " + ".join(PREFILL_KERNELS),
                                          "bound": "hbm", "achieved": round(ph_achieved, 2), "peak": HBM_PEAK_GBS,
                                          "unit": "GB/s", "frac": round(ph_achieved / HBM_PEAK_GBS, 4),
                                          "traffic": None if ph_tr is None else round(ph_tr / ph["per_launch"] / 1e9, 2),
                                          "traffic_bytes_per_launch": ph_tr, "alg_bytes_per_launch": ph["alg_bytes"],
                                          "launch_us": round(ph["per_launch"] * 1e6, 2)}},
        "verify_decode": {"workload": vf["x"].name, "tokens_per_s": round(vf["tokens"] * args.steps / vf["wall"], 1),
                          "roofline": {"kernel": "verify_kernel", "bound": "hbm",
                                       "achieved": round(v_achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(v_achieved / HBM_PEAK_GBS, 4),
                                       "traffic": None if v_tr is None else round(v_tr / vf["per_launch"] / 1e9, 2), "traffic_bytes_per_launch": v_tr,
                                       "alg_bytes_per_launch": vf["alg_bytes"],
                                       "launch_us": round(vf["per_launch"] * 1e6, 2)}},
        "verify_normed": {"workload": vn["x"].name + "_gated_rmsnorm",
                          "tokens_per_s": round(vn["tokens"] * args.steps / vn["wall"], 1),
                          "unfused_us": round(vn["per_launch_unfused"] * 1e6, 2),
                          "unfused_alg_bytes": vn["alg_bytes_unfused"],
                          "roofline": {"kernel": "verify_kernel (NORM)", "bound": "hbm",
                                       "achieved": round(vn_achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(vn_achieved / HBM_PEAK_GBS, 4),
                                       "traffic": None if vn_tr is None else round(vn_tr / vn["per_launch"] / 1e9, 2),
                                       "traffic_bytes_per_launch": vn_tr, "alg_bytes_per_launch": vn["alg_bytes"],
                                       "launch_us": round(vn["per_launch"] * 1e6, 2)}},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
        line["cpu_baseline"]["model"] = cpu_model()
        line["cpu_baseline"]["single_core"] = cpu_baseline_single_core()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

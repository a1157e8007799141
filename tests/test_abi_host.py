"""The C-ABI library without a GPU: load, exported symbols, argument validation.

Every call here is rejected (or is a no-op) on the host before any HIP call,
so it runs on a machine without a GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_53_amd as kda
from gated_delta_rule_53_amd._binding import Problem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def exported_symbols(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "kda_abi_version", "kda_status_string", "kda_last_error",
        "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd", "kda_recurrent_step",
        "kda_chunk_fwd_gated", "kda_recurrent_step_gated", "kda_chunk_fwd_pooled",
        "kda_recurrent_verify", "kda_gated_rmsnorm", "kda_short_conv", "kda_recurrent_step_normed",
        "kda_chunk_fwd_noalloc", "kda_recurrent_verify_normed", "kda_chunk_fwd_conv"])


def test_library_exports_every_declared_symbol():
    syms = exported_symbols(kda.library_path())
    missing = [f for f in declared_functions() if f not in syms]
    assert not missing, f"not exported: {missing}"


def test_abi_version_matches_header():
    m = re.search(r"#define KDA_ABI_VERSION (\d+)", open(HEADER).read())
    assert kda.abi_version() == int(m.group(1))


def test_gate_struct_layout():
    assert ctypes.sizeof(kda.Gate) == 24
    assert kda.Gate.has_lower_bound.offset == 16 and kda.Gate.lower_bound.offset == 20


def _c_layout(struct: str, fields):
    """sizeof and offsetof of the header's struct, as the C compiler lays it out."""
    import shutil
    import subprocess
    import tempfile
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "kda.h"', "int main(void) {",
             f'    printf("%zu\\n", sizeof({struct}));']
    lines += [f'    printf("%zu\\n", offsetof({struct}, {f}));' for f in fields]
    lines += ["    return 0;", "}"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        open(src, "w").write("\n".join(lines) + "\n")
        subprocess.run([cc, "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()]
    return vals[0], dict(zip(fields, vals[1:]))


@pytest.mark.parametrize("cls,struct", [(Problem, "kda_problem_t"), (kda.Gate, "kda_gate_t"),
                                        (kda.Conv, "kda_conv_t")])
def test_struct_layout_matches_header(cls, struct):
    """The ctypes mirrors match the C compiler's layout of include/kda.h, field by field."""
    fields = [f for f, _ in cls._fields_]
    size, offs = _c_layout(struct, fields)
    assert ctypes.sizeof(cls) == size
    for f in fields:
        assert getattr(cls, f).offset == offs[f], f


def test_status_strings():
    lib = kda.raw_library()
    names = {i: lib.kda_status_string(i).decode() for i in range(6)}
    assert names[0] == "ok" and names[5] == "HIP error"
    assert lib.kda_status_string(99).decode() == "unknown status"


def _prob(**kw):
    base = dict(total_tokens=128, num_seqs=1, num_heads=2, head_k=128, head_v=128, qkv_dtype=1,
                out_dtype=0, scale=0.088, qk_l2norm=1, chunk_size=64)
    base.update(kw)
    return Problem(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


def _chunk(prob, **ptrs):
    lib = kda.raw_library()
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, s0=None, out=FAKE, fs=None, ws=None,
             ws_bytes=0)
    p.update(ptrs)
    st = lib.kda_chunk_fwd(None if prob is None else ctypes.byref(prob), p["q"], p["k"], p["v"],
                           p["g"], p["beta"], p["cu"], p["s0"], p["out"], p["fs"], p["ws"],
                           p["ws_bytes"], None)
    return st, lib.kda_last_error().decode()


def _step(prob, **ptrs):
    lib = kda.raw_library()
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, out=FAKE)
    p.update(ptrs)
    st = lib.kda_recurrent_step(None if prob is None else ctypes.byref(prob), p["q"], p["k"],
                                p["v"], p["g"], p["beta"], p["state"], p["out"], None)
    return st, lib.kda_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(num_seqs=-1), 2, "num_seqs"),
    (dict(total_tokens=-5), 2, "total_tokens"),
    (dict(num_heads=0), 2, "num_heads"),
    (dict(head_k=96, head_v=96), 3, "head size 96"),
    (dict(head_k=128, head_v=64), 3, "head_k"),
    (dict(head_k=0), 2, "head sizes"),
    (dict(qkv_dtype=7), 3, "qkv_dtype"),
    (dict(out_dtype=2), 3, "out_dtype"),
    (dict(qk_l2norm=3), 2, "qk_l2norm"),
    (dict(chunk_size=32), 3, "chunk_size"),
    (dict(gate_per_head=2), 2, "gate_per_head"),
    (dict(state_layout=2), 2, "state_layout"),
    (dict(state_layout=-1), 2, "state_layout"),
])
def test_chunk_fwd_rejects_bad_problem(kw, status, needle):
    st, msg = _chunk(_prob(**kw))
    assert st == status and needle in msg, (st, msg)


def test_chunk_fwd_null_pointers():
    assert _chunk(None)[0] == 1
    st, msg = _chunk(_prob(), cu=None)
    assert st == 1 and "cu_seqlens" in msg
    for name in ("q", "k", "v", "g", "beta", "out"):
        st, msg = _chunk(_prob(), **{name: None})
        assert st == 1, name


def test_chunk_fwd_empty_batch_is_a_noop():
    st, msg = _chunk(_prob(num_seqs=0, total_tokens=0), q=None, k=None, v=None, g=None, beta=None,
                     cu=None, out=None)
    assert st == 0 and msg == ""


# bytes of one (chunk, head) record of the two-pass bf16 path
REC_BYTES = 61952


def test_workspace_query():
    lib = kda.raw_library()
    q = lambda **kw: lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(_prob(**kw)))
    # bf16, 128-wide heads: chunk offsets [N+1] and scan order [N] (int32) padded
    # to 256 bytes, then one record per (chunk, head) for up to ceil(T/64) + N chunks.
    assert q() == 256 + (2 + 1) * 2 * REC_BYTES
    assert q(total_tokens=4096, num_seqs=1, num_heads=32) == 256 + (64 + 1) * 32 * REC_BYTES
    assert q(total_tokens=100, num_seqs=70, num_heads=1) == 768 + (2 + 70) * REC_BYTES
    assert q(total_tokens=100, num_seqs=63, num_heads=1) == 512 + (2 + 63) * REC_BYTES
    # every other configuration needs none
    assert q(qkv_dtype=0) == 0
    assert q(head_k=64, head_v=64) == 0
    assert q(num_seqs=0, total_tokens=0) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(None) == 0


def test_workspace_is_checked():
    need = 256 + 3 * 2 * REC_BYTES
    st, msg = _chunk(_prob(), ws=FAKE, ws_bytes=need - 1)
    assert st == 4 and "workspace" in msg, (st, msg)
    st, msg = _chunk(_prob(), ws=None, ws_bytes=need)
    assert st == 1 and "workspace" in msg, (st, msg)


def _noalloc(prob, **ptrs):
    lib = kda.raw_library()
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, s0=None, out=FAKE, fs=None)
    p.update(ptrs)
    st = lib.kda_chunk_fwd_noalloc(None if prob is None else ctypes.byref(prob), p["q"], p["k"], p["v"],
                                   p["g"], p["beta"], p["cu"], p["s0"], p["out"], p["fs"], None)
    return st, lib.kda_last_error().decode()


MISALIGNED = ctypes.c_void_p(0x1008)  # 8-byte aligned, not 16
MISALIGNED4 = ctypes.c_void_p(0x1002)  # 2-byte aligned, not 4


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "out", "s0", "fs", "ws"])
def test_chunk_fwd_rejects_misaligned_vector_operands(name):
    prob = _prob()
    need = kda.raw_library().kda_chunk_fwd_workspace_bytes(ctypes.byref(prob))
    ptrs = dict(ws=FAKE, ws_bytes=need)
    ptrs[name] = MISALIGNED
    st, msg = _chunk(prob, **ptrs)
    assert st == 2 and "16-byte aligned" in msg, (name, st, msg)


@pytest.mark.parametrize("name", ["beta", "cu"])
def test_chunk_fwd_rejects_misaligned_elements(name):
    prob = _prob()
    need = kda.raw_library().kda_chunk_fwd_workspace_bytes(ctypes.byref(prob))
    st, msg = _chunk(prob, ws=FAKE, ws_bytes=need, **{name: MISALIGNED4})
    assert st == 2 and "aligned" in msg, (name, st, msg)


def test_per_head_g_needs_only_element_alignment():
    """g [T, H] (one decay per head) is read element by element: a 4-byte aligned g
    passes the alignment check (and the call then fails later, on the host, for
    want of a workspace)."""
    prob = _prob(gate_per_head=1)
    st, msg = _chunk(prob, g=ctypes.c_void_p(0x1004))
    assert st == 4 and "workspace" in msg, (st, msg)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "state", "out"])
def test_recurrent_step_rejects_misaligned_vector_operands(name):
    st, msg = _step(_prob(total_tokens=2, num_seqs=2), **{name: MISALIGNED})
    assert st == 2 and "16-byte aligned" in msg, (name, st, msg)


def test_noalloc_checks_like_chunk_fwd():
    assert _noalloc(None)[0] == 1
    for kw, status, needle in [(dict(num_seqs=-1), 2, "num_seqs"), (dict(head_k=96, head_v=96), 3, "head size"),
                               (dict(chunk_size=32), 3, "chunk_size")]:
        st, msg = _noalloc(_prob(**kw))
        assert st == status and needle in msg and "noalloc" in msg, (st, msg)
    for name in ("q", "k", "v", "g", "beta", "out", "cu"):
        st, msg = _noalloc(_prob(), **{name: None})
        assert st == 1, name
    st, msg = _noalloc(_prob(num_seqs=0, total_tokens=0), q=None, k=None, v=None, g=None, beta=None, cu=None,
                       out=None)
    assert st == 0 and msg == ""


def test_noalloc_rejects_problems_beyond_its_scratch():
    """The library's array holds 128 MiB: one sequence of 4,224 tokens at H = 32
    fits, 4,225 does not (before any HIP call, so this runs without a GPU)."""
    lib = kda.raw_library()
    limit = 128 << 20
    fits = _prob(total_tokens=4224, num_seqs=1, num_heads=32)
    over = _prob(total_tokens=4225, num_seqs=1, num_heads=32)
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(fits)) <= limit
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(over)) > limit
    st, msg = _noalloc(over)
    assert st == 3 and "scratch" in msg, (st, msg)
    assert kda._binding.NOALLOC_SCRATCH_BYTES == limit
    m = re.search(r"#define KDA_NOALLOC_SCRATCH_BYTES \(\(size_t\)128 << 20\)", open(HEADER).read())
    assert m is not None


@pytest.mark.parametrize("kw,status,needle", [
    (dict(total_tokens=3, num_seqs=2), 2, "one token each"),
    (dict(total_tokens=2, num_seqs=2, head_k=32, head_v=32), 3, "head size 32"),
    (dict(total_tokens=2, num_seqs=2, num_heads=-1), 2, "num_heads"),
])
def test_recurrent_step_rejects_bad_problem(kw, status, needle):
    st, msg = _step(_prob(**kw))
    assert st == status and needle in msg, (st, msg)


def test_recurrent_step_null_pointers_and_empty():
    assert _step(None)[0] == 1
    for name in ("q", "k", "v", "g", "beta", "state", "out"):
        st, _ = _step(_prob(total_tokens=2, num_seqs=2), **{name: None})
        assert st == 1, name
    st, msg = _step(_prob(total_tokens=0, num_seqs=0), q=None, state=None)
    assert st == 0


def _gate(**kw):
    base = dict(a_log=0x2000, dt_bias=0x3000, has_lower_bound=0, lower_bound=0.0)
    base.update(kw)
    return kda.Gate(**base)


def _chunk_gated(prob, gate, **ptrs):
    lib = kda.raw_library()
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, s0=None, out=FAKE, fs=None, ws=None,
             ws_bytes=0)
    p.update(ptrs)
    st = lib.kda_chunk_fwd_gated(ctypes.byref(prob), None if gate is None else ctypes.byref(gate), p["q"],
                                 p["k"], p["v"], p["g"], p["beta"], p["cu"], p["s0"], p["out"], p["fs"],
                                 p["ws"], p["ws_bytes"], None)
    return st, lib.kda_last_error().decode()


def _step_gated(prob, gate, **ptrs):
    lib = kda.raw_library()
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, out=FAKE)
    p.update(ptrs)
    st = lib.kda_recurrent_step_gated(ctypes.byref(prob), None if gate is None else ctypes.byref(gate),
                                      p["q"], p["k"], p["v"], p["g"], p["beta"], p["state"], p["out"], None)
    return st, lib.kda_last_error().decode()


@pytest.mark.parametrize("gate,status,needle", [
    (None, 1, "gate is NULL"),
    (dict(a_log=None), 1, "a_log"),
    (dict(dt_bias=None), 1, "dt_bias"),
    (dict(has_lower_bound=2), 2, "has_lower_bound"),
    (dict(has_lower_bound=1, lower_bound=0.5), 2, "lower_bound"),
    (dict(has_lower_bound=1, lower_bound=float("nan")), 2, "lower_bound"),
    (dict(has_lower_bound=1, lower_bound=float("-inf")), 2, "lower_bound"),
])
def test_gated_entry_points_check_the_gate(gate, status, needle):
    g = None if gate is None else _gate(**gate)
    st, msg = _chunk_gated(_prob(), g)
    assert st == status and needle in msg, (st, msg)
    st, msg = _step_gated(_prob(total_tokens=2, num_seqs=2), g)
    assert st == status and needle in msg, (st, msg)


def test_gated_entry_points_check_problem_and_pointers():
    st, msg = _chunk_gated(_prob(head_k=96, head_v=96), _gate())
    assert st == 3 and "head size 96" in msg
    for name in ("q", "k", "v", "g", "beta", "out"):
        st, _ = _chunk_gated(_prob(), _gate(), **{name: None})
        assert st == 1, name
    st, msg = _chunk_gated(_prob(), _gate(), ws=FAKE, ws_bytes=16)
    assert st == 4 and "workspace" in msg
    for name in ("q", "k", "v", "g", "beta", "state", "out"):
        st, _ = _step_gated(_prob(total_tokens=2, num_seqs=2), _gate(), **{name: None})
        assert st == 1, name
    st, msg = _step_gated(_prob(total_tokens=3, num_seqs=2), _gate())
    assert st == 2 and "one token each" in msg


def _verify(prob, width, gate=None, **ptrs):
    lib = kda.raw_library()
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, pool=FAKE, num_slots=4, idx=FAKE, acc=None, out=FAKE)
    p.update(ptrs)
    st = lib.kda_recurrent_verify(ctypes.byref(prob), width, None if gate is None else ctypes.byref(gate),
                                  p["q"], p["k"], p["v"], p["g"], p["beta"], p["pool"], p["num_slots"],
                                  p["idx"], p["acc"], p["out"], None)
    return st, lib.kda_last_error().decode()


def _pooled(prob, gate=None, **ptrs):
    lib = kda.raw_library()
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, pool=FAKE, num_slots=4, slots=FAKE, out=FAKE,
             ws=None, ws_bytes=0)
    p.update(ptrs)
    st = lib.kda_chunk_fwd_pooled(ctypes.byref(prob), None if gate is None else ctypes.byref(gate), p["q"],
                                  p["k"], p["v"], p["g"], p["beta"], p["cu"], p["pool"], p["num_slots"],
                                  p["slots"], p["out"], p["ws"], p["ws_bytes"], None)
    return st, lib.kda_last_error().decode()


def test_verify_checks_its_arguments():
    vp = lambda **kw: _prob(**{**dict(total_tokens=12, num_seqs=3), **kw})
    assert _verify(vp(), 0)[0] == 2 and "width" in _verify(vp(), 0)[1]
    st, msg = _verify(vp(), 3)
    assert st == 2 and "num_seqs * width" in msg, (st, msg)
    st, msg = _verify(vp(), 4, num_slots=-1)
    assert st == 2 and "num_slots" in msg
    for name in ("q", "k", "v", "g", "beta", "pool", "idx", "out"):
        st, _ = _verify(vp(), 4, **{name: None})
        assert st == 1, name
    st, msg = _verify(vp(), 4, gate=_gate(has_lower_bound=3))
    assert st == 2 and "has_lower_bound" in msg
    st, msg = _verify(vp(head_k=96, head_v=96), 4)
    assert st == 3 and "head size 96" in msg
    assert _verify(vp(total_tokens=0, num_seqs=0), 5, q=None, pool=None)[0] == 0
    for name in ("q", "pool", "out"):
        st, msg = _verify(vp(), 4, **{name: MISALIGNED})
        assert st == 2 and "16-byte aligned" in msg, (name, st, msg)
    st, msg = _verify(vp(), 4, idx=MISALIGNED4)
    assert st == 2 and "4-byte aligned" in msg, (st, msg)


def test_pooled_prefill_checks_its_arguments():
    st, msg = _pooled(_prob(), num_slots=-2)
    assert st == 2 and "num_slots" in msg
    for name in ("pool", "slots"):
        st, msg = _pooled(_prob(), **{name: None})
        assert st == 1 and "state_pool" in msg, (name, msg)
    for name in ("q", "k", "v", "g", "beta", "out"):
        st, _ = _pooled(_prob(), **{name: None})
        assert st == 1, name
    st, msg = _pooled(_prob(), gate=_gate(a_log=None))
    assert st == 1 and "a_log" in msg
    st, msg = _pooled(_prob(), ws=FAKE, ws_bytes=8)
    assert st == 4 and "workspace" in msg


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 2, 64)
    with pytest.raises(kda.KdaError):
        kda.chunk_fwd(x, x, x, x, torch.zeros(4, 2))
    with pytest.raises(kda.KdaError):
        kda.recurrent_step(x, x, x, x, torch.zeros(4, 2), torch.zeros(4, 2, 64, 64))


def test_product_package_does_not_reference_the_oracle():
    pkg = os.path.dirname(kda.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"


def test_binding_rejects_unknown_state_layout():
    from gated_delta_rule_53_amd._binding import KdaArgumentError, _layout_code
    assert _layout_code("dk_dv") == 0 and _layout_code("dv_dk") == 1
    with pytest.raises(KdaArgumentError):
        _layout_code("transposed")


def _norm(rows=8, head_v=128, in_dtype=1, out_dtype=0, o=FAKE, gate=FAKE, weight=FAKE, eps=1e-6, out=None):
    lib = kda.raw_library()
    out = ctypes.c_void_p(0x2000) if out is None else out
    st = lib.kda_gated_rmsnorm(rows, head_v, in_dtype, out_dtype, o, gate, weight, eps, out, None)
    return st, lib.kda_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(rows=-1), 2, "rows"),
    (dict(head_v=96), 3, "head_v 96"),
    (dict(in_dtype=5), 3, "in_dtype"),
    (dict(out_dtype=5), 3, "out_dtype"),
    (dict(eps=-1.0), 2, "eps"),
    (dict(eps=float("nan")), 2, "eps"),
    (dict(gate=None), 1, "required"),
    (dict(weight=None), 1, "required"),
    (dict(out=FAKE, in_dtype=1, out_dtype=0), 2, "out may be o"),
    (dict(gate=ctypes.c_void_p(0x1004)), 2, "16-byte aligned"),
])
def test_gated_rmsnorm_rejects_before_launch(kw, status, needle):
    st, msg = _norm(**kw)
    assert st == status and needle in msg, (st, msg)


def test_gated_rmsnorm_zero_rows_is_a_noop():
    st, msg = _norm(rows=0, o=None, gate=None, weight=None, out=None)
    assert st == 0 and msg == ""


def _conv(num_seqs=2, total_tokens=10, channels=64, kernel_size=4, dtype=1, silu=1, x=FAKE, weight=FAKE, cu=FAKE,
          state_in=None, state_out=None, y=FAKE):
    lib = kda.raw_library()
    st = lib.kda_short_conv(num_seqs, total_tokens, channels, kernel_size, dtype, silu, x, weight, cu, state_in,
                            state_out, y, None)
    return st, lib.kda_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(num_seqs=-1), 2, "num_seqs"),
    (dict(total_tokens=-1), 2, "total_tokens"),
    (dict(channels=12), 3, "channels"),
    (dict(channels=0), 3, "channels"),
    (dict(kernel_size=5), 3, "kernel_size"),
    (dict(kernel_size=0), 3, "kernel_size"),
    (dict(dtype=4), 3, "dtype"),
    (dict(silu=2), 2, "silu"),
    (dict(weight=None), 1, "required"),
    (dict(cu=None), 1, "required"),
    (dict(y=None), 1, "required"),
    (dict(x=ctypes.c_void_p(0x1008)), 2, "16-byte aligned"),
    # the launch's work-items along x (256 per 8 tokens) stay below 2^32
    (dict(total_tokens=(1 << 27) - 1023), 3, "too large"),
    (dict(num_seqs=(1 << 23) + 1), 3, "too large"),
])
def test_short_conv_rejects_before_launch(kw, status, needle):
    st, msg = _conv(**kw)
    assert st == status and needle in msg, (st, msg)


def test_short_conv_empty_batch_is_a_noop():
    st, msg = _conv(num_seqs=0, total_tokens=0, x=None, weight=None, cu=None, y=None)
    assert st == 0 and msg == ""


def test_recurrent_step_normed_rejects_before_launch():
    lib = kda.raw_library()
    p = _prob(total_tokens=4, num_seqs=4)
    st = lib.kda_recurrent_step_normed(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                       1e-6, FAKE, None)
    assert st == 1 and "out_gate" in lib.kda_last_error().decode()
    st = lib.kda_recurrent_step_normed(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       -1.0, FAKE, None)
    assert st == 2 and "norm_eps" in lib.kda_last_error().decode()
    p = _prob(total_tokens=5, num_seqs=4)
    st = lib.kda_recurrent_step_normed(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       1e-6, FAKE, None)
    assert st == 2 and "one token each" in lib.kda_last_error().decode()


def test_recurrent_verify_normed_rejects_before_launch():
    lib = kda.raw_library()
    p = _prob(total_tokens=12, num_seqs=3)
    call = lambda prob, width, og, nw, eps: lib.kda_recurrent_verify_normed(
        ctypes.byref(prob), width, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, None, og, nw, eps, FAKE, None)
    assert call(p, 4, None, FAKE, 1e-6) == 1 and "out_gate" in lib.kda_last_error().decode()
    assert call(p, 4, FAKE, None, 1e-6) == 1 and "norm_weight" in lib.kda_last_error().decode()
    assert call(p, 4, FAKE, FAKE, -1.0) == 2 and "norm_eps" in lib.kda_last_error().decode()
    assert call(p, 4, FAKE, FAKE, float("nan")) == 2 and "norm_eps" in lib.kda_last_error().decode()
    # the checks of kda_recurrent_verify apply as well
    assert call(p, 3, FAKE, FAKE, 1e-6) == 2 and "num_seqs * width" in lib.kda_last_error().decode()
    st = call(p, 4, MISALIGNED, FAKE, 1e-6)
    assert st == 2 and "16-byte aligned" in lib.kda_last_error().decode()
    st = call(p, 4, FAKE, MISALIGNED, 1e-6)
    assert st == 2 and "16-byte aligned" in lib.kda_last_error().decode()
    # an empty batch needs no epilogue operands
    assert call(_prob(total_tokens=0, num_seqs=0), 4, None, None, 1e-6) == 0


def _conv_call(prob, conv, **ptrs):
    lib = kda.raw_library()
    p = dict(gate=None, qkv=FAKE, g=FAKE, beta=FAKE, cu=FAKE, s0=None, out=FAKE, fs=None, ws=FAKE,
             ws_bytes=1 << 40)
    p.update(ptrs)
    st = lib.kda_chunk_fwd_conv(ctypes.byref(prob), p["gate"], None if conv is None else ctypes.byref(conv),
                                p["qkv"], p["g"], p["beta"], p["cu"], p["s0"], p["out"], p["fs"], p["ws"],
                                p["ws_bytes"], None)
    return st, lib.kda_last_error().decode()


def test_chunk_fwd_conv_rejects_before_launch():
    ok = lambda **kw: kda.Conv(**{**dict(kernel_size=4, silu=1, weight=0x1000, state_in=None, state_out=None), **kw})
    st, msg = _conv_call(_prob(), None)
    assert st == 1 and "conv is NULL" in msg
    for K in (0, 5):
        st, msg = _conv_call(_prob(), ok(kernel_size=K))
        assert st == 3 and "kernel_size" in msg, (K, st, msg)
    st, msg = _conv_call(_prob(), ok(silu=2))
    assert st == 2 and "silu" in msg
    # only the bf16, d = 128 path has the convolution fused
    for kw in (dict(qkv_dtype=0), dict(head_k=64, head_v=64)):
        st, msg = _conv_call(_prob(**kw), ok())
        assert st == 3 and "bf16, d = 128" in msg, (kw, st, msg)
    for name in ("weight", "state_in", "state_out"):
        st, msg = _conv_call(_prob(), ok(**{name: 0x1008}))
        assert st == 2 and "16-byte aligned" in msg, (name, st, msg)
    st, msg = _conv_call(_prob(), ok(weight=None))
    assert st == 1 and "weight" in msg
    st, msg = _conv_call(_prob(), ok(), qkv=None)
    assert st == 1 and "qkv" in msg
    st, msg = _conv_call(_prob(), ok(), qkv=MISALIGNED)
    assert st == 2 and "16-byte aligned" in msg, (st, msg)
    # the checks of kda_chunk_fwd apply as well
    st, msg = _conv_call(_prob(), ok(), ws_bytes=16)
    assert st == 4 and "workspace" in msg, (st, msg)
    st, msg = _conv_call(_prob(), ok(), gate=ctypes.byref(_gate(has_lower_bound=3)))
    assert st == 2 and "has_lower_bound" in msg
    assert _conv_call(_prob(total_tokens=0, num_seqs=0), ok(weight=None), qkv=None)[0] == 0

"""Plant plausible mistakes in copies of the C oracle; the pins must catch each.

Every mutant is the oracle source with one textual edit, compiled with gcc
into a temporary directory.  The pins in oracle_pins.py run against it and at
least one must fail.  This shows that the pins constrain every step of the
recurrence: decay, recall, delta sign, update, read-out order, normalisation,
scale placement, state indexing.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")


def _swap_blocks(src: str, first: str, second: str, end: str) -> str:
    """Swap the code block starting at marker ``first`` with the one at ``second``
    (which runs up to marker ``end``)."""
    a = src.index(first)
    b = src.index(second)
    c = src.index(end, b)
    return src[:a] + src[b:c] + src[a:b] + src[c:]


MUTANTS = {
    "decay_dropped": lambda s: s.replace("row[j] *= a;", "row[j] *= 1.0;"),
    "decay_sign": lambda s: s.replace("exp((double)gt[c])", "exp(-(double)gt[c])"),
    "delta_sign": lambda s: s.replace("b * ((double)vt[j] - u[j])", "b * ((double)vt[j] + u[j])"),
    "beta_dropped": lambda s: s.replace("b * ((double)vt[j] - u[j])", "((double)vt[j] - u[j])"),
    "recall_transposed": lambda s: s.replace("u[j] += kc * row[j];", "u[j] += kc * S[j * dv + c];"),
    "update_uses_query": lambda s: s.replace(
        "const double kc = kf[c];\n            double *row = S + c * dv;\n            for (int64_t j = 0; j < dv; ++j) row[j] += kc * u[j];",
        "const double kc = qf[c];\n            double *row = S + c * dv;\n            for (int64_t j = 0; j < dv; ++j) row[j] += kc * u[j];"),
    "read_before_update": lambda s: _swap_blocks(s, "/* S += k_hat delta^T */", "/* o_t = S^T q_hat */",
                                                 "    }\n}\n"),
    "eps_outside_root": lambda s: s.replace("rq = 1.0 / sqrt(sq + 1e-6);", "rq = 1.0 / fmax(sqrt(sq), 1e-6);")
                                   .replace("rk = 1.0 / sqrt(sk + 1e-6);", "rk = 1.0 / fmax(sqrt(sk), 1e-6);"),
    "scale_on_key": lambda s: s.replace("qf[c] = qf[c] * rq * scale;", "qf[c] = qf[c] * rq;")
                               .replace("kf[c] = kf[c] * rk;", "kf[c] = kf[c] * rk * scale;"),
    "state_index_swapped": lambda s: s.replace(
        "const size_t state_off = (size_t)((n * H + h) * dk * dv);",
        "const size_t state_off = (size_t)((h * num_seqs + n) * dk * dv);"),
    "varlen_offset": lambda s: s.replace("run_pair(cu_seqlens[n], cu_seqlens[n + 1],",
                                         "run_pair(cu_seqlens[n], cu_seqlens[n + 1] - (cu_seqlens[n + 1] > cu_seqlens[n] + 1),"),
}


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, workdir):
    src = open(SRC).read()
    mutated = MUTANTS[name](src)
    assert mutated != src, f"mutation {name} did not apply"
    cpath = os.path.join(workdir, f"{name}.c")
    lpath = os.path.join(workdir, f"lib{name}.so")
    open(cpath, "w").write(mutated)
    subprocess.run(["gcc", *oracle.CFLAGS, cpath, "-o", lpath, "-lm"], check=True,
                   stderr=subprocess.DEVNULL)
    lib = oracle.load(lpath)

    def fwd(*args, **kw):
        return oracle.forward(*args, lib=lib, **kw)

    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(fwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"

"""Planted mistakes in the oracle: every one must make the pin suite fail.

The pins of test_oracle_pins.py are only worth something if a plausible slip in
the oracle's arithmetic breaks at least one of them.  Each case below is such a
slip, written as a text edit of oracle/ssd_oracle.c (the recurrence of section
"Mamba-2 架构" on dbyun.net's "基于 NVIDIA CUDA Tile 加速 Mamba-2 高性能前向传播内核",
and the chunk cumsum of its section "Kernel 1：计算累积和"): the edited copy is
compiled with the same flags into a temporary library, the pin suite runs against
it in a subprocess (SSD_ORACLE_LIBRARY), and the test requires that run to fail.
The unedited source, built the same way, must pass.  CPU only.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
PINS = os.path.join(HERE, "test_oracle_pins.py")

UPDATE = "        /* state update: h <- exp(A dt) h + dt * x (outer) B */"
OUTPUT = "        /* output: y = h . C + D x */"


def _output_before_update(src):
    """y_t read from the state before token t's update (h_{t-1} instead of h_t)."""
    a, b = src.index(UPDATE), src.index(OUTPUT)
    end = src.index("    if (jb->hT) memcpy")
    end = src.rindex("    }\n", b, end)       # closes the token loop
    return src[:a] + src[b:end] + src[a:b] + src[end:]


# (name, edit): an edit is (old, new) -- `old` must occur exactly once -- or a function
MUTANTS = [
    ("decay sign flipped", ("exp(A * dt)", "exp(-A * dt)")),
    ("decay without dt", ("exp(A * dt)", "exp(A)")),
    ("input term without dt", ("const double coef = dt * xrow[p];", "const double coef = xrow[p];")),
    ("C in the state update", ("coef * brow[n]", "coef * crow[n]")),
    ("B in the read-out", ("acc += Sp[n] * crow[n];", "acc += Sp[n] * brow[n];")),
    ("skip term dropped", ("yrow[p] = acc + Dh * xrow[p];", "yrow[p] = acc;")),
    ("skip term on the output", ("yrow[p] = acc + Dh * xrow[p];", "yrow[p] = acc + Dh * acc;")),
    ("interleaved head-to-group map", ("const int64_t g = h / (H / G);", "const int64_t g = h % G;")),
    ("initial state ignored", ("if (jb->h0) memcpy", "if (0) memcpy")),
    ("output from the previous state", _output_before_update),
    ("snapshot one token early", ("t % jb->chunk == 0 && jb->snaps", "(t + 1) % jb->chunk == 0 && jb->snaps")),
    ("cumsum not restarted per chunk", ("if (t % chunk == 0) run = 0.0;", "if (t == 0) run = 0.0;")),
    ("cumsum scaled by ln 2", ("run * M_LOG2E", "run * M_LN2")),
    ("exclusive cumsum", ("                run += A[h] * d;\n"
                          "                G2[(b * nheads + h) * seqlen + t] = run * M_LOG2E;\n",
                          "                G2[(b * nheads + h) * seqlen + t] = run * M_LOG2E;\n"
                          "                run += A[h] * d;\n")),
]


def _apply(src, edit):
    if callable(edit):
        return edit(src)
    old, new = edit
    assert src.count(old) == 1, f"edit target not found exactly once: {old!r}"
    return src.replace(old, new)


def _pins_pass(library):
    """Run the pin suite against `library`; True when every pin passes."""
    env = dict(os.environ, SSD_ORACLE_LIBRARY=library)
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       env=env, capture_output=True, text=True, timeout=300)
    return r.returncode == 0, r.stdout[-2000:]


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = str(tmp_path / f"lib{name}.so")
    oracle.compile_oracle(str(src), lib)
    return lib


def test_planted_mistakes_fail_the_pins(tmp_path):
    with open(oracle.SOURCE) as fh:
        base = fh.read()
    libs = [("unedited", _build(tmp_path, "unedited", base))]
    for i, (name, edit) in enumerate(MUTANTS):
        text = _apply(base, edit)
        assert text != base, name
        libs.append((name, _build(tmp_path, f"mutant{i}", text)))
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda nl: _pins_pass(nl[1]), libs))
    ok, out = results[0]
    assert ok, f"the unedited oracle failed its pins:\n{out}"
    survivors = [name for (name, _), (ok, _) in zip(libs[1:], results[1:]) if ok]
    for (name, _), (ok, _) in zip(libs[1:], results[1:]):
        print(f"  {name}: {'SURVIVED' if ok else 'caught'}")
    assert not survivors, f"planted mistakes that no pin catches: {survivors}"


@pytest.mark.parametrize("name,edit", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_each_edit_changes_the_source(name, edit):
    with open(oracle.SOURCE) as fh:
        base = fh.read()
    assert _apply(base, edit) != base

"""The CPU oracle reads no memory before writing it.

Both oracle libraries are built a second time with tests/oracle_poison.h,
which makes every malloc'd block start as 0xFF bytes (NaN as a float or a
double, 0xFFFFFFFF as an index).  Every entry point then runs on small seeded
inputs in a child process (an out-of-range index read ends the child, not the
test run), and its results must equal the normal build's bit for bit.  A
planted mistake, the suffix recurrence's carry left unset, must be caught.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
POISON = os.path.join(HERE, "oracle_poison.h")
SRC = os.path.join(ROOT, "oracle", "laplex_oracle.c")
SRC_PAR = os.path.join(ROOT, "oracle", "laplex_oracle_par.c")

# child: run every entry point with the given library (or the normal build)
# and save the results
CHILD = r'''
import sys, ctypes
import numpy as np
sys.path.insert(0, sys.argv[1])
import oracle
seq_path, par_path, out = sys.argv[2], sys.argv[3], sys.argv[4]
lib = oracle.load(seq_path) if seq_path != "-" else oracle.load()
r = np.random.default_rng(7)
res = {}
for n, m, k in ((1, 1, 1), (2, 3, 1), (37, 8, 23), (300, 16, 170), (1001, 5, 999)):
    a = r.uniform(0, n / 4.0 + 1.0, n).astype(np.float32)
    a[r.integers(0, n, n // 5)] = a[0]          # ties
    b = r.uniform(0, n / 4.0 + 1.0, k).astype(np.float32)
    x = r.normal(size=(n, m)).astype(np.float32)
    xb = r.normal(size=(k, m)).astype(np.float32)
    g = r.normal(size=(n, m)).astype(np.float32)
    phi = r.uniform(0, 6.2831853, n).astype(np.float32)
    psi = r.uniform(0, 6.2831853, k).astype(np.float32)
    rows = np.unique(r.integers(0, n, min(n, 7)))
    t = "%d_%d_%d_" % (n, m, k)
    res[t + "perm"] = oracle.stable_argsort(a, lib=lib)
    res[t + "sym"] = oracle.sym_apply(a, x, lib=lib)
    res[t + "gen"] = oracle.general_apply(a, b, xb, lib=lib)
    res[t + "phs"] = oracle.phased_apply(a, phi, x, lib=lib)
    res[t + "phg"] = oracle.phased_apply(a, phi, xb, b=b, psi=psi, lib=lib)
    dx, da = oracle.sym_backward(a, x, g, lib=lib)
    res[t + "bdx"], res[t + "bda"] = dx, da
    gdx, gda, gdb = oracle.general_backward(a, b, xb, g, lib=lib)
    res[t + "gdx"], res[t + "gda"], res[t + "gdb"] = gdx, gda, gdb
    rda, renv = oracle.backward_rows(rows, a, x, g, lib=lib)
    res[t + "rda"], res[t + "renv"] = rda, renv
    yr, er = oracle.dense_rows_c(rows, a, x, lib=lib)
    res[t + "dry"], res[t + "dre"] = yr, er
    if par_path != "-":
        oracle._par_handle = None
        oracle._SO_PAR = par_path
    res[t + "pperm"] = oracle.stable_argsort_par(a)
    res[t + "psym"] = oracle.sym_apply_par(a, x)
np.savez(out, **res)
'''


def _build(src: str, out: str, extra: list[str]) -> None:
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-include", POISON, *extra, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)


def _run(seq: str, par: str, out: str) -> subprocess.CompletedProcess:
    return subprocess.run([sys.executable, "-c", CHILD, ROOT, seq, par, out], capture_output=True, text=True, timeout=600)


def _compare(ref_npz: str, got_npz: str) -> list[str]:
    ref, got = np.load(ref_npz), np.load(got_npz)
    bad = []
    for key in ref.files:
        r, g = ref[key], got[key]
        if r.dtype.kind == "f" and not np.isfinite(g).all():
            bad.append("%s: non-finite" % key)
        elif r.tobytes() != g.tobytes():
            bad.append("%s: bits differ" % key)
    return bad


@pytest.fixture(scope="module")
def normal_results(tmp_path_factory):
    oracle.build()
    oracle.build_par()
    out = str(tmp_path_factory.mktemp("normal") / "normal.npz")
    p = _run("-", "-", out)
    assert p.returncode == 0, p.stderr[-2000:]
    return out


def test_oracle_results_do_not_depend_on_unwritten_memory(normal_results, tmp_path):
    seq, par = str(tmp_path / "seq.so"), str(tmp_path / "par.so")
    _build(SRC, seq, [])
    _build(SRC_PAR, par, ["-fopenmp"])
    out = str(tmp_path / "poisoned.npz")
    p = _run(seq, par, out)
    assert p.returncode == 0, "poisoned oracle run failed:\n" + p.stderr[-2000:]
    bad = _compare(normal_results, out)
    assert not bad, "results depend on memory read before written: %s" % bad[:8]


def test_planted_unset_carry_is_caught(normal_results, tmp_path):
    # the suffix recurrence of the symmetric apply without its zero carry
    src = open(SRC).read()
    line = "for (int64_t c = 0; c < m; ++c) u[c] = 0.0;"
    assert src.count(line) == 1
    planted = str(tmp_path / "planted.c")
    with open(planted, "w") as f:
        f.write(src.replace(line, ""))
    seq, par = str(tmp_path / "seq.so"), str(tmp_path / "par.so")
    _build(planted, seq, [])
    _build(SRC_PAR, par, ["-fopenmp"])
    out = str(tmp_path / "planted.npz")
    p = _run(seq, par, out)
    assert p.returncode == 0, p.stderr[-2000:]
    bad = _compare(normal_results, out)
    assert any(k.endswith("_sym: non-finite") or "_sym:" in k for k in bad), bad

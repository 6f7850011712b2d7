"""The symmetric operator's index path (m > 4 columns: rows gathered by the
permutation, tile reduce, tile carries, apply with scatter) executed on the
CPU from the library's own device code, by the SIMT emulation in
tests/simt/simt.hpp.

- A ThreadSanitizer build reports any communication between GPU threads
  through memory that no barrier or wave exchange orders (a missing
  __syncthreads, a shared array reused across column chunks too early).
- Two runs whose workspaces, output and shared memory start filled with
  different poison values (a NaN and the largest finite float) must give the
  same output bits, finite and within the parity bar of a float64 reference:
  then no word the kernels read was left unwritten, and every output row was
  written.
- Guard zones around every buffer must come back untouched (no write out of
  bounds); an AddressSanitizer build catches accesses further out.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SIMT = os.path.join(HERE, "simt")
CSRC = os.path.join(os.path.dirname(HERE), "laplace_prefix_scans_amd", "csrc")
SRC = os.path.join(SIMT, "sim_sym_index.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _build(tmp, name, extra):
    out = os.path.join(tmp, name)
    cmd = ["g++", "-std=c++17", "-pthread", "-Wno-attributes", "-I", SIMT, "-I", CSRC, SRC, "-o", out] + extra
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


@pytest.fixture(scope="module")
def sims(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("simt"))
    return {
        "plain": _build(tmp, "sim", ["-O2"]),
        "tsan": _build(tmp, "sim_tsan", ["-O1", "-g", "-fsanitize=thread"]),
        "asan": _build(tmp, "sim_asan", ["-O1", "-g", "-fsanitize=address"]),
    }


def _run(exe, n, m, ties, seed, poison, stride=1, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe, str(n), str(m), str(ties), str(seed), poison, str(stride)], capture_output=True,
                       text=True, timeout=timeout, env=env)
    assert r.returncode == 0, r.stderr[-6000:]
    assert "ThreadSanitizer" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-6000:]
    out = dict(line.split("=", 1) for line in r.stdout.split())
    return out


CASES = [(5000, 8, 1), (3001, 16, 0), (4097, 5, 0)]


@pytest.mark.parametrize("n,m,ties", CASES)
def test_index_path_reads_only_written_words(sims, n, m, ties):
    a = _run(sims["plain"], n, m, ties, 7, "7fc0dead")
    b = _run(sims["plain"], n, m, ties, 7, "7f7fffff")
    for o in (a, b):
        assert o["nonfinite_rows"] == "0" and o["guards_ok"] == "1", o
        assert float(o["err"]) <= 1e-6, o
    assert a["y_hash"] == b["y_hash"], "the output depends on unwritten memory: %s vs %s" % (a, b)


@pytest.mark.parametrize("n,m,ties", CASES[:2])
def test_index_path_has_no_race(sims, n, m, ties):
    o = _run(sims["tsan"], n, m, ties, 11, "7fc0dead")
    assert o["nonfinite_rows"] == "0" and o["guards_ok"] == "1" and float(o["err"]) <= 1e-6, o


def test_index_path_in_bounds(sims):
    o = _run(sims["asan"], 3001, 16, 1, 13, "7fc0dead")
    assert o["nonfinite_rows"] == "0" and o["guards_ok"] == "1" and float(o["err"]) <= 1e-6, o

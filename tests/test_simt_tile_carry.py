"""The tile-carry scan (k_tile_carry) executed on the CPU from the library's
own device code by the SIMT emulation in tests/simt/simt.hpp, at tile counts
that select each of its load widths (1, 2, 4, 8 and 16 tiles per thread; the
last two serve the middle level of the three-level path and are reached on
the GPU only by inputs of billions of elements).

The carries from the left and from the right must match the plain recurrence
in float64 to 1e-5 of the same recurrence over the absolute aggregates, with
the kernel's decay in one column and the tie decay (weight 1 between equal
anchors, else 0) in the other; tile boundaries carry ties.  A ThreadSanitizer
build reports any communication between GPU threads that no barrier or wave
exchange orders.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SIMT = os.path.join(HERE, "simt")
CSRC = os.path.join(os.path.dirname(HERE), "laplace_prefix_scans_amd", "csrc")
SRC = os.path.join(SIMT, "sim_tile_carry.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")

# tile counts around each load width's limits: 1024 q tiles for q loads per thread
COUNTS = [1, 2, 700, 1024, 1025, 2049, 4096, 4097, 8192, 9000, 16384]


def _build(tmp, name, extra):
    out = os.path.join(tmp, name)
    cmd = ["g++", "-std=c++17", "-pthread", "-Wno-attributes", "-I", SIMT, "-I", CSRC, SRC, "-o", out] + extra
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


@pytest.fixture(scope="module")
def sims(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("simt_carry"))
    return {"plain": _build(tmp, "sim", ["-O2"]), "tsan": _build(tmp, "sim_tsan", ["-O1", "-g", "-fsanitize=thread"])}


def _run(exe, T, M, tie_from, seed, timeout=600):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe, str(T), str(M), str(tie_from), str(seed)], capture_output=True, text=True, timeout=timeout,
                       env=env)
    assert r.returncode == 0, r.stderr[-6000:]
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-6000:]
    return dict(line.split("=", 1) for line in r.stdout.split())


@pytest.mark.parametrize("T", COUNTS)
def test_tile_carry_matches_recurrence(sims, T):
    out = _run(sims["plain"], T, 2, 1, 11 + T)
    assert int(out["nonfinite"]) == 0
    assert float(out["err_f"]) <= 1e-5, out
    assert float(out["err_b"]) <= 1e-5, out


@pytest.mark.parametrize("T", [1025, 9000])
def test_tile_carry_no_unordered_communication(sims, T):
    out = _run(sims["tsan"], T, 1, 1, 5 + T)
    assert float(out["err_f"]) <= 1e-5 and float(out["err_b"]) <= 1e-5, out

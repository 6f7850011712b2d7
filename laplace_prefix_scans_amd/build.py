"""Build liblaplex.so (HIP, gfx950) in-tree with hipcc, and beside it
liblaplex_probe.so, the memory-system probes the benchmark measures the
operator's kernels against.

    python -m laplace_prefix_scans_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblaplex.so")
SOURCES = ["laplex_sort.hip", "laplex_route.hip", "laplex_apply.hip", "laplex_api.hip"]
PROBE_LIB = os.path.join(HERE, "liblaplex_probe.so")
PROBE_SOURCES = ["laplex_probe.hip"]
ARCH = "gfx950"
FLAGS = [
    "-O3",
    "-std=c++17",
    "--offload-arch=" + ARCH,
    "-fPIC",
    # no implicit multiply-add contraction: every fused multiply-add is an
    # explicit fmaf, so results do not depend on code generation
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link liblaplex.so and liblaplex_probe.so
    (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)

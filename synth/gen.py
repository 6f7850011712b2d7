"""Seeded generators for anchors, phases and right-hand sides.

Every array is drawn in chunks of ``CHUNK`` elements; chunk ``c`` of stream
``s`` of workload ``w`` uses its own PCG64 generator seeded with
``SeedSequence([ROOT, w, s, c])``.  The bytes of an array therefore do not
depend on how much memory the caller has, and a large array can be produced
straight into a preallocated (e.g. pinned) buffer.

Anchors are drawn in float64 and rounded to the nearest float32, which gives
finer values than drawing float32 uniforms directly (whose 24-bit grid would
make every anchor of the largest workload a multiple of 8).

The five named workloads are synthetic stand-ins for the settings the LAPLEX
pages describe (the operator of "2.1 The Operator", sizes from the scaling
experiments of "4.1 Scaling and Performance", the flattened-image Gram model
of "4.2", and the abstract's matvec at dimension up to 10^9).  No dataset is
used: the flattened 3x1024x1024 image workload only takes its shape and the
raster structure of its coordinates.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Optional

import numpy as np

ROOT = 0x1A91E
CHUNK = 1 << 22

# stream ids
S_A, S_B, S_X, S_PHI, S_PSI, S_JIT, S_D = 1, 2, 3, 4, 5, 6, 7


def _fill(out: np.ndarray, wid: int, sid: int, draw: Callable[[np.random.Generator, int, int], np.ndarray]) -> np.ndarray:
    """Fill ``out`` (1-D view over the leading axis) chunk by chunk."""
    n = out.shape[0]
    for c, lo in enumerate(range(0, n, CHUNK)):
        hi = min(n, lo + CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT, wid, sid, c])))
        out[lo:hi] = draw(rng, lo, hi)
    return out


def anchors_uniform(n: int, lo: float, hi: float, wid: int, sid: int = S_A, out: Optional[np.ndarray] = None) -> np.ndarray:
    """float32 anchors, iid Uniform(lo, hi) drawn in float64 and rounded to float32."""
    if out is None:
        out = np.empty(n, np.float32)
    return _fill(out, wid, sid, lambda r, a, b: r.uniform(lo, hi, b - a).astype(np.float32))


def anchors_normal(n: int, mean: float, var: float, wid: int, sid: int = S_A, out: Optional[np.ndarray] = None) -> np.ndarray:
    """float32 anchors, iid Normal(mean, variance=var) drawn in float64."""
    if out is None:
        out = np.empty(n, np.float32)
    sd = math.sqrt(var)
    return _fill(out, wid, sid, lambda r, a, b: r.normal(mean, sd, b - a).astype(np.float32))


def anchors_grid_jitter(channels: int, height: int, width: int, var: float, wid: int,
                        sid: int = S_JIT, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Pixel-coordinate anchors of a flattened CxHxW image plus Normal(0, var) jitter.

    Element ``i = c*H*W + r*W + col`` gets the raster index ``r*W + col`` of its
    pixel (shared by the channels) plus its own jitter, rounded to float32.
    """
    n = channels * height * width
    hw = height * width
    if out is None:
        out = np.empty(n, np.float32)
    sd = math.sqrt(var)

    def draw(r, a, b):
        base = (np.arange(a, b, dtype=np.int64) % hw).astype(np.float64)
        return (base + r.normal(0.0, sd, b - a)).astype(np.float32)

    return _fill(out, wid, sid, draw)


def columns_normal(n: int, m: int, wid: int, sid: int = S_X, out: Optional[np.ndarray] = None) -> np.ndarray:
    """float32 right-hand sides, row-major n x m, iid N(0, 1)."""
    if out is None:
        out = np.empty((n, m), np.float32)
    return _fill(out, wid, sid, lambda r, a, b: r.standard_normal((b - a, m), dtype=np.float32))


def phases_uniform(n: int, wid: int, sid: int = S_PHI, out: Optional[np.ndarray] = None) -> np.ndarray:
    """float32 phases, iid Uniform(0, 2*pi) drawn in float64."""
    if out is None:
        out = np.empty(n, np.float32)
    return _fill(out, wid, sid, lambda r, a, b: r.uniform(0.0, 2.0 * math.pi, b - a).astype(np.float32))


@dataclasses.dataclass
class Workload:
    """One synthetic workload: anchors ``a`` (n), optional ``b`` (k), phases, and x."""
    name: str
    kind: str              # "sym" | "general" | "phased" | "gram"
    n: int
    m: int
    k: int
    a: np.ndarray
    x: np.ndarray
    b: Optional[np.ndarray] = None
    phi: Optional[np.ndarray] = None
    psi: Optional[np.ndarray] = None
    D: Optional[np.ndarray] = None   # Gram weights (k)
    recipe: str = ""


# name -> (workload id, kind, description)
WORKLOADS = {
    "sym4096": (1, "sym", "symmetric, n=4096, m=1, a~U(0,512), x~N(0,1)"),
    "sym2p20m16": (2, "sym", "symmetric Gram-style apply, n=2^20, m=16, a~U(0,2^17), X~N(0,1)"),
    "gen2p24k2p16": (3, "general", "general, n=2^24 a~N(0,var 2^12), k=2^16 b~N(0,var 2^12), x~N(0,1), m=1"),
    "phased3x1024x1024m8": (4, "phased", "phased symmetric, n=3*2^20 flattened 3x1024x1024, a=raster index + N(0,var 0.1), phi~U(0,2pi), m=8"),
    "sym2p30": (5, "sym", "symmetric, n=2^30, m=1, a~U(0,2^27), x~N(0,1)"),
    "gram2p16k2p16": (6, "gram", "weighted Gram A diag(D) A^T, n=2^16 a~U(0,2^13), k=2^16 b~U(0,2^13), D~U(0,1)"),
}


def make_workload(name: str, scale: int = 0) -> Workload:
    """Build a named workload.  ``scale > 0`` divides n (and k) by 2**scale,
    keeping the distributions (the anchor range is scaled with n so that the
    density of anchors, and hence the tie structure, is preserved)."""
    wid, kind, desc = WORKLOADS[name]
    s = 1 << scale
    if name == "sym4096":
        n, m = 4096 // s, 1
        a = anchors_uniform(n, 0.0, 512.0 / s, wid)
        return Workload(name, kind, n, m, n, a, columns_normal(n, m, wid), recipe=desc)
    if name == "sym2p20m16":
        n, m = (1 << 20) // s, 16
        a = anchors_uniform(n, 0.0, float(1 << 17) / s, wid)
        return Workload(name, kind, n, m, n, a, columns_normal(n, m, wid), recipe=desc)
    if name == "gen2p24k2p16":
        n, k, m = (1 << 24) // s, (1 << 16) // s, 1
        a = anchors_normal(n, 0.0, float(1 << 12), wid, S_A)
        b = anchors_normal(k, 0.0, float(1 << 12), wid, S_B)
        return Workload(name, kind, n, m, k, a, columns_normal(k, m, wid), b=b, recipe=desc)
    if name == "phased3x1024x1024m8":
        side = 1024 // (1 << (scale // 2)) if scale else 1024
        n, m = 3 * side * side, 8
        a = anchors_grid_jitter(3, side, side, 0.1, wid)
        phi = phases_uniform(n, wid)
        return Workload(name, kind, n, m, n, a, columns_normal(n, m, wid), phi=phi, psi=phi, recipe=desc)
    if name == "sym2p30":
        n, m = (1 << 30) // s, 1
        a = anchors_uniform(n, 0.0, float(1 << 27) / s, wid)
        return Workload(name, kind, n, m, n, a, columns_normal(n, m, wid), recipe=desc)
    if name == "gram2p16k2p16":
        n, k = (1 << 16) // s, (1 << 16) // s
        a = anchors_uniform(n, 0.0, float(1 << 13) / s, wid, S_A)
        b = anchors_uniform(k, 0.0, float(1 << 13) / s, wid, S_B)
        D = anchors_uniform(k, 0.0, 1.0, wid, S_D)
        return Workload(name, kind, n, 1, k, a, np.zeros((0, 1), np.float32), b=b, D=D, recipe=desc)
    raise KeyError(name)

"""Helpers for the GPU parity tests: move seeded host inputs to the device,
call the library through its C-ABI binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np

TOL = 1e-5  # normwise: ||y - y_ref||_inf / ||K0 |x| ||_inf, per column


def have_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def dev(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_sort(a: np.ndarray):
    import laplace_prefix_scans_amd as lp
    a_d = dev(a)
    a_s, perm = lp.laplex_sort_anchors(a_d, check=True)
    return a_d, a_s, perm


def assert_perm_is_stable_argsort(a: np.ndarray, perm: np.ndarray, a_sorted: np.ndarray):
    """Properties that together pin the stable ascending argsort uniquely, for
    sizes where a second sort on the host would be too slow: a permutation;
    a_sorted == a[perm] bit for bit; nondecreasing; equal anchors in input order."""
    n = a.size
    assert perm.dtype == np.uint32 and perm.size == n
    seen = np.zeros(n, dtype=bool)
    assert int(perm.max()) < n
    seen[perm] = True
    assert seen.all(), "perm is not a permutation"
    del seen
    g = a[perm]
    assert np.array_equal(g.view(np.uint32), a_sorted.view(np.uint32)), "a_sorted != a[perm]"
    del g
    assert np.all(a_sorted[1:] >= a_sorted[:-1]), "not ascending"
    ties = a_sorted[1:] == a_sorted[:-1]
    assert np.all(perm[1:][ties] > perm[:-1][ties]), "equal anchors out of input order"


def describe_nonfinite(y: np.ndarray, perm: np.ndarray, tile_rows: int = 0) -> str:
    """Where the non-finite rows of y (original order) sit in sorted order:
    their sorted positions, the tiles those fall in (tile_rows rows per tile,
    when given) and the columns involved, so that a failure names its rows."""
    y2 = y.reshape(y.shape[0], -1)
    bad = np.nonzero(~np.isfinite(y2).all(axis=1))[0]
    if bad.size == 0:
        return "all finite"
    pinv = np.empty(perm.size, np.int64)
    pinv[perm.astype(np.int64)] = np.arange(perm.size)
    pos = np.sort(pinv[bad])
    msg = "%d non-finite rows; sorted positions %s; columns %s" % (
        bad.size, pos[:8].tolist(), np.unique(np.nonzero(~np.isfinite(y2[bad]))[1]).tolist()[:8])
    if tile_rows:
        msg += "; tiles %s" % np.unique(pos // tile_rows)[:8].tolist()
    return msg

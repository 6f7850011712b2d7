"""GPU parity of the general backward (dx = K^T g, anchor gradients da, db)
with the float64 oracle, through the C-ABI.

Error measure, per output: ||y - y_ref||_inf / ||envelope||_inf with the
envelope K^T|g| for dx, sum_c |g_c| K|x_c| for da and sum_c |x_c| K^T|g_c| for
db (the sizes of the summands the fp32 scans add up)."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([0x6B4C, seed]))


def _case(n, k, m, seed, ties):
    """a and b over the same range; with ties both are rounded to integers so
    that a and b share anchors (and repeat their own)."""
    r = _rng(seed)
    span = (n + k) / 8.0 + 1.0
    a = r.uniform(0, span, n).astype(np.float32)
    b = r.uniform(0, span, k).astype(np.float32)
    if ties:
        a, b = np.round(a).astype(np.float32), np.round(b).astype(np.float32)
    x = r.standard_normal((k, m)).astype(np.float32)
    g = r.standard_normal((n, m)).astype(np.float32)
    return a, b, x, g


def _errors(a, b, x, g, dx, da, db):
    dx_ref, da_ref, db_ref = oracle.general_backward(a, b, x, g)
    env_dx = oracle.general_apply(b, a, np.abs(g))
    env_da = (np.abs(g) * oracle.general_apply(a, b, np.abs(x))).sum(axis=1)
    env_db = (np.abs(x) * env_dx).sum(axis=1)
    e_dx = oracle.normwise_error(dx.reshape(dx_ref.shape), dx_ref, env_dx)
    e_da = float(np.max(np.abs(da - da_ref)) / max(np.max(env_da), 1e-300))
    e_db = float(np.max(np.abs(db - db_ref)) / max(np.max(env_db), 1e-300))
    return e_dx, e_da, e_db


def _run(a, b, x, g, route):
    import laplace_prefix_scans_amd as lp
    ra = lp.route_buffer(a.size) if route else None
    rb = lp.route_buffer(b.size) if route else None
    a_s, pa = lp.laplex_sort_anchors(dev(a), route=ra, check=True)
    b_s, pb = lp.laplex_sort_anchors(dev(b), route=rb, check=True)
    dx, da, db = lp.laplex_backward_general(a_s, pa, b_s, pb, dev(x), dev(g), route_a=ra, route_b=rb)
    return host(dx), host(da), host(db)


CASES = [(1, 1, 1), (1, 5, 1), (5, 1, 2), (1000, 37, 1), (2048, 2048, 1), (3000, 1100, 1), (70001, 4097, 1),
         (4097, 70001, 2), (65536, 256, 4), (12345, 999, 8), (300000, 65536, 1), (20000, 20000, 3)]


@pytest.mark.parametrize("n,k,m", CASES)
@pytest.mark.parametrize("ties", [False, True])
def test_backward_general_parity(n, k, m, ties):
    a, b, x, g = _case(n, k, m, 100 + n + 3 * k + 7 * m, ties)
    for route in ((False, True) if m <= 4 else (False,)):
        dx, da, db = _run(a, b, x, g, route)
        assert np.isfinite(dx).all() and np.isfinite(da).all() and np.isfinite(db).all()
        e_dx, e_da, e_db = _errors(a, b, x, g, dx, da, db)
        assert max(e_dx, e_da, e_db) <= TOL, "n=%d k=%d m=%d ties=%s route=%s: dx %.2e da %.2e db %.2e" % (
            n, k, m, ties, route, e_dx, e_da, e_db)


@pytest.mark.parametrize("n,k,m", [(5000, 700, 1), (7001, 7001, 2), (999, 9999, 4), (140001, 131073, 1)])
def test_backward_general_route_bitwise(n, k, m):
    """Moving rows along the routes or by index gives the same bits."""
    a, b, x, g = _case(n, k, m, 7 + n + k, True)
    r0 = _run(a, b, x, g, False)
    r1 = _run(a, b, x, g, True)
    for u, v in zip(r0, r1):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))


def test_backward_general_all_tied_is_exactly_zero():
    """Every anchor of a and b equal: no pair has a sign, so da and db are
    exactly 0, and dx is the column sums of g on every row."""
    n, k, m = 9000, 3000, 2
    r = _rng(3)
    a = np.full(n, -1.25, np.float32)
    b = np.full(k, -1.25, np.float32)
    x = r.standard_normal((k, m)).astype(np.float32)
    g = r.standard_normal((n, m)).astype(np.float32)
    dx, da, db = _run(a, b, x, g, True)
    assert np.all(da == 0.0) and np.all(db == 0.0)
    e_dx, _, _ = _errors(a, b, x, g, dx, da, db)
    assert e_dx <= TOL


def test_backward_general_matches_symmetric_when_b_is_a():
    """b = a (as a separate array): dx equals the symmetric backward's dx and
    da + db equals its anchor gradient (each pair's two terms, split between
    the row and the column copy of the anchor)."""
    import laplace_prefix_scans_amd as lp
    n, m = 40000, 1
    r = _rng(5)
    a = r.uniform(0, 5000, n).astype(np.float32)
    x = r.standard_normal((n, m)).astype(np.float32)
    g = r.standard_normal((n, m)).astype(np.float32)
    dx, da, db = _run(a, a.copy(), x, g, True)
    a_s, pa = lp.laplex_sort_anchors(dev(a))
    dxs, das = lp.laplex_backward_sym(a_s, pa, dev(x), dev(g))
    env = oracle.sym_apply(a, np.abs(g))
    assert oracle.normwise_error(dx, host(dxs).astype(np.float64), env) <= 2 * TOL
    kx, kg = oracle.sym_apply(a, np.abs(x)), oracle.sym_apply(a, np.abs(g))
    env_da = (np.abs(g) * kx + np.abs(x) * kg).sum(axis=1)
    assert np.max(np.abs((da + db) - host(das))) / np.max(env_da) <= 2 * TOL


def test_backward_general_empty_sides():
    """k = 0: da is zero (no columns); n = 0: dx and db are zero (no rows)."""
    import torch
    import laplace_prefix_scans_amd as lp
    a = dev(np.linspace(0, 9, 10, dtype=np.float32))
    a_s, pa = lp.laplex_sort_anchors(a)
    e = torch.empty(0, device="cuda")
    e_perm = torch.empty(0, dtype=torch.uint32, device="cuda")
    da = torch.full((10,), 7.0, device="cuda")
    lp.laplex_backward_general(a_s, pa, e, e_perm, torch.empty(0, 1, device="cuda"), torch.ones(10, 1, device="cuda"),
                               da=da)
    assert np.all(host(da) == 0.0)
    dx = torch.full((10, 1), 7.0, device="cuda")
    db = torch.full((10,), 7.0, device="cuda")
    lp.laplex_backward_general(e, e_perm, a_s, pa, torch.ones(10, 1, device="cuda"), torch.empty(0, 1, device="cuda"),
                               dx=dx, db=db)
    assert np.all(host(dx) == 0.0) and np.all(host(db) == 0.0)


def test_backward_general_rejects_bad_arguments():
    import torch
    import laplace_prefix_scans_amd as lp
    a_s, pa = lp.laplex_sort_anchors(dev(np.arange(100, dtype=np.float32)))
    b_s, pb = lp.laplex_sort_anchors(dev(np.arange(30, dtype=np.float32)))
    x = torch.zeros(30, 2, device="cuda")
    g = torch.zeros(100, 2, device="cuda")
    with pytest.raises(ValueError):
        lp.laplex_backward_general(a_s, pa, b_s, pb, x, torch.zeros(100, 3, device="cuda"))
    with pytest.raises(ValueError):
        lp.laplex_backward_general(a_s, pa, b_s, pb, x, torch.zeros(99, 2, device="cuda"))
    with pytest.raises(lp.LaplexError):
        lp.laplex_backward_general(a_s, pa, b_s, pb, x, g, dx=x)  # output on top of an input
    with pytest.raises(lp.LaplexError):
        lp.laplex_backward_general(a_s, pa, b_s, pb, x, g, db=a_s[:30])


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_backward_general_full_workload():
    """The general workload at full size (n = 2^24, k = 2^16, m = 1, routes):
    every element of dx, da and db against the oracle."""
    from synth import make_workload
    w = make_workload("gen2p24k2p16")
    r = _rng(24)
    g = r.standard_normal((w.n, 1)).astype(np.float32)
    x = w.x.reshape(w.k, 1)
    dx, da, db = _run(w.a, w.b, x, g, True)
    print("gpu done", flush=True)
    assert np.isfinite(dx).all() and np.isfinite(da).all() and np.isfinite(db).all()
    e_dx, e_da, e_db = _errors(w.a, w.b, x, g, dx, da, db)
    print("errors dx %.3e da %.3e db %.3e" % (e_dx, e_da, e_db), flush=True)
    assert max(e_dx, e_da, e_db) <= TOL

"""GPU parity of the symmetric backward (dx = K g, anchor gradient da) with
the float64 oracle, through the C-ABI.

Error measure, per output: ||y - y_ref||_inf / ||envelope||_inf with the
envelope K|g| for dx and  sum_c |g_c| K|x_c| + |x_c| K|g_c|  for da (the sizes
of the summands the fp32 scans add up)."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([0xBAC4, seed]))


def _case(n, m, seed, ties):
    r = _rng(seed)
    a = r.uniform(0, n / 8.0 + 1.0, n).astype(np.float32)
    if ties:
        a = np.round(a).astype(np.float32)
    x = r.standard_normal((n, m)).astype(np.float32)
    g = r.standard_normal((n, m)).astype(np.float32)
    return a, x, g


def _errors(a, x, g, dx, da):
    dx_ref, da_ref = oracle.sym_backward(a, x, g)
    env_dx = oracle.sym_apply(a, np.abs(g))
    kx, kg = oracle.sym_apply(a, np.abs(x)), oracle.sym_apply(a, np.abs(g))
    env_da = (np.abs(g) * kx + np.abs(x) * kg).sum(axis=1)
    e_dx = oracle.normwise_error(dx.reshape(dx_ref.shape), dx_ref, env_dx)
    e_da = float(np.max(np.abs(da - da_ref)) / np.max(env_da))
    return e_dx, e_da


def _run(a, x, g, route):
    import laplace_prefix_scans_amd as lp
    ra = lp.route_buffer(a.size) if route else None
    a_s, perm = lp.laplex_sort_anchors(dev(a), route=ra, check=True)
    dx, da = lp.laplex_backward_sym(a_s, perm, dev(x), dev(g), route=ra)
    return host(dx), host(da)


CASES = [(1, 1), (2, 1), (7, 2), (1000, 1), (2048, 1), (2049, 1), (4097, 3), (70001, 1), (70001, 2), (65536, 4),
         (12345, 8), (300000, 1)]


@pytest.mark.parametrize("n,m", CASES)
@pytest.mark.parametrize("ties", [False, True])
def test_backward_sym_parity(n, m, ties):
    a, x, g = _case(n, m, 100 + n + 7 * m, ties)
    for route in ((False, True) if m <= 4 else (False,)):
        dx, da = _run(a, x, g, route)
        assert np.isfinite(dx).all() and np.isfinite(da).all()
        e_dx, e_da = _errors(a, x, g, dx, da)
        assert e_dx <= TOL and e_da <= TOL, "n=%d m=%d ties=%s route=%s: dx %.2e da %.2e" % (n, m, ties, route, e_dx, e_da)


@pytest.mark.parametrize("n,m", [(5000, 1), (70001, 2), (9999, 4), (140001, 1), ((1 << 17) + 1, 3)])
def test_backward_route_bitwise(n, m):
    """Moving rows along the route or by index gives the same bits."""
    a, x, g = _case(n, m, 7 + n, True)
    dx0, da0 = _run(a, x, g, False)
    dx1, da1 = _run(a, x, g, True)
    assert np.array_equal(dx0.view(np.uint32), dx1.view(np.uint32))
    assert np.array_equal(da0.view(np.uint32), da1.view(np.uint32))


def test_backward_all_tied_is_exactly_zero():
    """With every anchor equal no pair has a sign: da is exactly 0 and dx is
    the column sums of g."""
    n, m = 20000, 2
    r = _rng(3)
    a = np.full(n, 3.5, np.float32)
    x = r.standard_normal((n, m)).astype(np.float32)
    g = r.standard_normal((n, m)).astype(np.float32)
    dx, da = _run(a, x, g, True)
    assert np.all(da == 0.0)
    e_dx, _ = _errors(a, x, g, dx, da)
    assert e_dx <= TOL


def test_backward_two_far_clusters():
    """Two clusters 400 apart (exp(-400) underflows in fp32): each cluster's
    gradient is its own, the other cluster contributes exactly nothing."""
    r = _rng(4)
    n1, n2, m = 3000, 5000, 1
    a1 = r.uniform(0, 20, n1).astype(np.float32)
    a2 = r.uniform(500, 520, n2).astype(np.float32)
    a = np.concatenate([a1, a2])
    x = r.standard_normal((n1 + n2, m)).astype(np.float32)
    g = r.standard_normal((n1 + n2, m)).astype(np.float32)
    dx, da = _run(a, x, g, True)
    dx1, da1 = _run(a1, x[:n1], g[:n1], True)
    dx2, da2 = _run(a2, x[n1:], g[n1:], True)
    e1 = np.max(np.abs(da[:n1] - da1)) / max(1e-30, np.max(np.abs(da1)))
    e2 = np.max(np.abs(da[n1:] - da2)) / max(1e-30, np.max(np.abs(da2)))
    assert e1 <= TOL and e2 <= TOL


def _run_one_call(a, x, g):
    """Forward in one call (laplex_sort_matvec_sym with a kept workspace),
    then the backward from that workspace."""
    import laplace_prefix_scans_amd as lp
    n, m = x.shape
    ws = lp.workspace(lp.LAPLEX_OP_SORT_SYM, n, 0, m)
    y = lp.laplex_sort_matvec_sym(dev(a), dev(x), ws=ws, check=True)
    dx, da = lp.laplex_sort_matvec_sym_backward(ws, dev(g))
    return host(y), host(dx), host(da)


@pytest.mark.parametrize("n,m", [(1, 1), (2, 1), (7, 2), (2049, 1), (4097, 3), (70001, 1), (65536, 4), (12345, 8),
                                 (600001, 1)])
@pytest.mark.parametrize("ties", [False, True])
def test_backward_from_one_call_forward(n, m, ties):
    """The backward from a one-call forward's workspace (x kept in sorted
    order, only g moved): the oracle's gradients, and the same bits as the
    backward given the sort handle (routed when m <= 4, by index above)."""
    a, x, g = _case(n, m, 500 + n + 7 * m, ties)
    y, dx, da = _run_one_call(a, x, g)
    e_dx, e_da = _errors(a, x, g, dx, da)
    assert e_dx <= TOL and e_da <= TOL, "n=%d m=%d ties=%s: dx %.2e da %.2e" % (n, m, ties, e_dx, e_da)
    dx2, da2 = _run(a, x, g, m <= 4)
    assert np.array_equal(dx.view(np.uint32), dx2.reshape(dx.shape).view(np.uint32))
    assert np.array_equal(da.view(np.uint32), da2.view(np.uint32))


def test_backward_from_one_call_rejects_bad_arguments():
    import torch
    import laplace_prefix_scans_amd as lp
    n = 1000
    a, x, g = _case(n, 1, 9, False)
    ws = lp.workspace(lp.LAPLEX_OP_SORT_SYM, n, 0, 1)
    lp.laplex_sort_matvec_sym(dev(a), dev(x), ws=ws)
    with pytest.raises(lp.LaplexError):  # forward workspace of fewer anchors
        lp.laplex_sort_matvec_sym_backward(ws[:1024], dev(g))
    gd = dev(g)
    with pytest.raises(lp.LaplexError):  # dx on top of g
        lp.laplex_sort_matvec_sym_backward(ws, gd, dx=gd)
    with pytest.raises(ValueError):
        lp.laplex_sort_matvec_sym_backward(ws, gd, da=torch.empty(n - 1, device="cuda"))


def test_backward_rejects_bad_arguments():
    import torch
    import laplace_prefix_scans_amd as lp
    a = dev(np.arange(100, dtype=np.float32))
    a_s, perm = lp.laplex_sort_anchors(a)
    x = torch.zeros(100, 2, device="cuda")
    with pytest.raises(ValueError):
        lp.laplex_backward_sym(a_s, perm, x, torch.zeros(100, 3, device="cuda"))
    with pytest.raises(lp.LaplexError):
        lp.laplex_backward_sym(a_s, perm, x, x, dx=x)  # output on top of an input


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_backward_sym2p30_sampled():
    """The n = 2^30 workload (m = 1, routes): da at spot rows (extreme anchors,
    tile boundaries, random rows) against the plain definition, and dx = K g
    through the symmetry <u, dx(g)> = <K u, g>; the backward from a one-call
    forward's workspace gives the same bits."""
    import torch
    import laplace_prefix_scans_amd as lp
    from synth import make_workload
    w = make_workload("sym2p30")
    print("generated n=%d" % w.n, flush=True)
    r = _rng(30)
    g = r.standard_normal(w.n).astype(np.float32)
    route = lp.route_buffer(w.n)
    a_s, pa = lp.laplex_sort_anchors(dev(w.a), route=route, check=True)
    dx, da = lp.laplex_backward_sym(a_s, pa, dev(w.x), dev(g), route=route)
    torch.cuda.synchronize()
    print("gpu done", flush=True)
    perm = host(pa)
    rows = np.unique(np.concatenate([perm[[0, 1, 2047, 2048, w.n // 2, w.n - 2048, w.n - 1]].astype(np.int64),
                                     r.integers(0, w.n, 9)]))
    da_ref, env = oracle.backward_rows(rows, w.a, w.x, g)
    err = float(np.max(np.abs(host(da)[rows] - da_ref)) / np.max(env))
    print("sampled da error %.3e over %d rows" % (err, rows.size), flush=True)
    assert err <= TOL
    u = torch.randn(w.n, device="cuda", generator=torch.Generator(device="cuda").manual_seed(8))
    ku = lp.laplex_matvec_sym(a_s, pa, u, route=route)
    lhs = float(torch.dot(u.double(), dx.double()))
    rhs = float(torch.dot(ku.double(), dev(g).double()))
    kabs = lp.laplex_matvec_sym(a_s, pa, dev(np.abs(g)), route=route)
    scale = float(torch.dot(u.abs().double(), kabs.double()))
    print("dx symmetry |lhs-rhs|/scale = %.3e" % (abs(lhs - rhs) / scale), flush=True)
    assert abs(lhs - rhs) <= TOL * scale
    # the backward the benchmark times: from a one-call forward's workspace
    del ku, kabs, u, a_s, pa, route
    torch.cuda.empty_cache()
    ws = lp.workspace(lp.LAPLEX_OP_SORT_SYM, w.n, 0, 1)
    lp.laplex_sort_matvec_sym(dev(w.a), dev(w.x), ws=ws, check=True)
    dx1, da1 = lp.laplex_sort_matvec_sym_backward(ws, dev(g))
    assert torch.equal(dx1.view(torch.int32), dx.view(torch.int32)), "one-call backward dx differs"
    assert torch.equal(da1.view(torch.int32), da.view(torch.int32)), "one-call backward da differs"
    print("one-call backward: same bits", flush=True)

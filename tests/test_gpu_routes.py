"""Applies that move x and y along the sort's route.

The route path reads and writes the same values in the same arithmetic order
as the index path (gather through perm, scatter through perm), so the two must
agree bit for bit; both are also checked against the oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([0x50E7, seed]))


def _sorted_with_route(a):
    import laplace_prefix_scans_amd as lp
    route = lp.route_buffer(a.size)
    a_s, perm = lp.laplex_sort_anchors(dev(a), route=route, check=True)
    return a_s, perm, route


@pytest.mark.parametrize("n,m", [(1, 1), (5, 2), (4095, 1), (4096, 3), (4097, 4), (70001, 1), (300000, 2), (123457, 4),
                                 (1 << 17, 3), ((1 << 17) + 1, 2),
                                 (20000, 8)])
def test_sym_route_bitwise(n, m):
    import laplace_prefix_scans_amd as lp
    r = _rng(n * 10 + m)
    a = r.uniform(0, n / 6.0 + 1.0, n).astype(np.float32)
    a[::11] = a[0]
    x = r.standard_normal((n, m)).astype(np.float32)
    a_s, perm, route = _sorted_with_route(a)
    y_route = host(lp.laplex_matvec_sym(a_s, perm, dev(x), route=route))
    y_index = host(lp.laplex_matvec_sym(a_s, perm, dev(x)))
    assert np.array_equal(y_route.view(np.uint32), y_index.view(np.uint32)), "route and index paths differ"
    err = oracle.normwise_error(y_route, oracle.sym_apply(a, x), oracle.sym_apply(a, np.abs(x)))
    assert err <= TOL


@pytest.mark.timeout(300)
@pytest.mark.parametrize("n,m", [((1 << 25) + 12345, 1), ((1 << 25) + 777, 2), ((1 << 25) + 3, 4)])
def test_sym_route_bitwise_large(n, m):
    """Past 4096 sort tiles (three-level carries, many workgroups per XCD in
    every route pass): the route path gives the same bits as the index path,
    and the one-call path (m = 1) the same bits as both; every column is
    within the parity bar of the float64 oracle."""
    import laplace_prefix_scans_amd as lp
    r = _rng(n * 10 + m)
    a = r.uniform(0, n / 6.0 + 1.0, n).astype(np.float32)
    a[::11] = a[0]
    x = r.standard_normal((n, m)).astype(np.float32)
    a_s, perm, route = _sorted_with_route(a)
    x_d = dev(x)
    y_route = lp.laplex_matvec_sym(a_s, perm, x_d, route=route)
    y_index = lp.laplex_matvec_sym(a_s, perm, x_d)
    assert np.array_equal(host(y_route).view(np.uint32), host(y_index).view(np.uint32)), "route and index paths differ"
    if m == 1:
        y_one = lp.laplex_sort_matvec_sym(dev(a), x_d, check=True)
        assert np.array_equal(host(y_one).view(np.uint32), host(y_route).view(np.uint32)), "one-call path differs"
    err = oracle.normwise_error(host(y_route), oracle.sym_apply(a, x), oracle.sym_apply(a, np.abs(x)))
    print("n=%d m=%d normwise error %.3e" % (n, m, err), flush=True)
    assert err <= TOL


@pytest.mark.parametrize("n,m", [(4096, 1), (70001, 2), (9999, 4), (140001, 2)])
def test_phased_route_bitwise(n, m):
    import laplace_prefix_scans_amd as lp
    r = _rng(7 + n + m)
    a = r.uniform(0, n / 6.0, n).astype(np.float32)
    phi = r.uniform(0, 2 * np.pi, n).astype(np.float32)
    x = r.standard_normal((n, m)).astype(np.float32)
    a_s, perm, route = _sorted_with_route(a)
    y_route = host(lp.laplex_matvec_phased(a_s, perm, dev(phi), dev(x), route_a=route))
    y_index = host(lp.laplex_matvec_phased(a_s, perm, dev(phi), dev(x)))
    assert np.array_equal(y_route.view(np.uint32), y_index.view(np.uint32))
    err = oracle.normwise_error(y_route, oracle.phased_apply(a, phi, x), oracle.sym_apply(a, np.abs(x)))
    assert err <= TOL


@pytest.mark.parametrize("n,k,m", [(5000, 300, 1), (200000, 70000, 2), (3000, 90000, 3), (100000, 1, 1), (9000, 140001, 1)])
@pytest.mark.parametrize("which", ["a", "b", "both"])
def test_general_route_bitwise(n, k, m, which):
    import laplace_prefix_scans_amd as lp
    r = _rng(11 + n + k + m)
    a = r.normal(0, 40, n).astype(np.float32)
    b = r.normal(0, 40, k).astype(np.float32)
    xb = r.standard_normal((k, m)).astype(np.float32)
    a_s, pa, ra = _sorted_with_route(a)
    b_s, pb, rb = _sorted_with_route(b)
    kw = {"route_a": ra if which in ("a", "both") else None, "route_b": rb if which in ("b", "both") else None}
    y_route = host(lp.laplex_matvec_general(a_s, pa, b_s, pb, dev(xb), **kw))
    y_index = host(lp.laplex_matvec_general(a_s, pa, b_s, pb, dev(xb)))
    assert np.array_equal(y_route.view(np.uint32), y_index.view(np.uint32))
    err = oracle.normwise_error(y_route, oracle.general_apply(a, b, xb), oracle.general_apply(a, b, np.abs(xb)))
    assert err <= TOL


def test_phased_general_route_bitwise():
    import laplace_prefix_scans_amd as lp
    r = _rng(99)
    n, k, m = 60000, 20000, 2
    a = r.normal(0, 30, n).astype(np.float32)
    b = r.normal(0, 30, k).astype(np.float32)
    phi = r.uniform(0, 2 * np.pi, n).astype(np.float32)
    psi = r.uniform(0, 2 * np.pi, k).astype(np.float32)
    xb = r.standard_normal((k, m)).astype(np.float32)
    a_s, pa, ra = _sorted_with_route(a)
    b_s, pb, rb = _sorted_with_route(b)
    y_route = host(lp.laplex_matvec_phased(a_s, pa, dev(phi), dev(xb), b_sorted=b_s, perm_b=pb, psi=dev(psi), route_a=ra,
                                           route_b=rb))
    y_index = host(lp.laplex_matvec_phased(a_s, pa, dev(phi), dev(xb), b_sorted=b_s, perm_b=pb, psi=dev(psi)))
    assert np.array_equal(y_route.view(np.uint32), y_index.view(np.uint32))
    err = oracle.normwise_error(y_route, oracle.phased_apply(a, phi, xb, b=b, psi=psi), oracle.general_apply(a, b, np.abs(xb)))
    assert err <= TOL


def test_sort_with_route_same_permutation():
    """Recording the route does not change the sort's outputs."""
    import laplace_prefix_scans_amd as lp
    r = _rng(5)
    a = r.uniform(0, 1000, 1 << 20).astype(np.float32)
    a_s1, p1 = lp.laplex_sort_anchors(dev(a), check=True)
    a_s2, p2, _ = _sorted_with_route(a)
    assert np.array_equal(host(p1), host(p2))
    assert np.array_equal(host(a_s1).view(np.uint32), host(a_s2).view(np.uint32))
    assert np.array_equal(host(p1), oracle.stable_argsort(a))

"""GPU parity of the general phased backward (dx = W^T g, gradients of the
row anchors and phases a, phi and of the column anchors and phases b, psi)
with the float64 oracle, through the C-ABI.

Error measure, per output: ||y - y_ref||_inf / ||envelope||_inf with the
unphased envelopes K^T|g| for dx, sum_c |g_c| K|x_c| for da and dphi, and
sum_c |x_c| K^T|g_c| for db and dpsi."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([0x6B4D, seed]))


def _case(n, k, m, seed, ties):
    r = _rng(seed)
    span = (n + k) / 8.0 + 1.0
    a = r.uniform(0, span, n).astype(np.float32)
    b = r.uniform(0, span, k).astype(np.float32)
    if ties:
        a, b = np.round(a).astype(np.float32), np.round(b).astype(np.float32)
    phi = r.uniform(0, 2 * np.pi, n).astype(np.float32)
    psi = r.uniform(0, 2 * np.pi, k).astype(np.float32)
    x = r.standard_normal((k, m)).astype(np.float32)
    g = r.standard_normal((n, m)).astype(np.float32)
    return a, phi, b, psi, x, g


def _errors(a, phi, b, psi, x, g, got):
    dx, da, db, dphi, dpsi = got
    ref = oracle.dense_phased_backward(a, phi, x, g, b=b, psi=psi)
    env_dx = oracle.general_apply(b, a, np.abs(g))
    env_a = (np.abs(g) * oracle.general_apply(a, b, np.abs(x))).sum(axis=1)
    env_b = (np.abs(x) * env_dx).sum(axis=1)
    e = [oracle.normwise_error(dx.reshape(ref[0].shape), ref[0], env_dx)]
    for u, v, env in ((da, ref[1], env_a), (db, ref[2], env_b), (dphi, ref[3], env_a), (dpsi, ref[4], env_b)):
        e.append(float(np.max(np.abs(u - v)) / max(np.max(env), 1e-300)))
    return e


def _run(a, phi, b, psi, x, g, route):
    import laplace_prefix_scans_amd as lp
    ra = lp.route_buffer(a.size) if route else None
    rb = lp.route_buffer(b.size) if route else None
    a_s, pa = lp.laplex_sort_anchors(dev(a), route=ra, check=True)
    b_s, pb = lp.laplex_sort_anchors(dev(b), route=rb, check=True)
    out = lp.laplex_backward_phased_general(a_s, pa, dev(phi), b_s, pb, dev(psi), dev(x), dev(g), route_a=ra, route_b=rb)
    return [host(t) for t in out]


CASES = [(1, 1, 1), (1, 5, 1), (5, 1, 2), (1000, 37, 1), (1024, 1024, 1), (3000, 1100, 3), (4097, 2000, 4),
         (2500, 3500, 8), (6000, 600, 2)]


@pytest.mark.parametrize("n,k,m", CASES)
@pytest.mark.parametrize("ties", [False, True])
def test_backward_phased_general_parity(n, k, m, ties):
    a, phi, b, psi, x, g = _case(n, k, m, 300 + n + 3 * k + 7 * m, ties)
    for route in ((False, True) if m <= 4 else (False,)):
        got = _run(a, phi, b, psi, x, g, route)
        assert all(np.isfinite(t).all() for t in got)
        e = _errors(a, phi, b, psi, x, g, got)
        assert max(e) <= TOL, "n=%d k=%d m=%d ties=%s route=%s: %s" % (n, k, m, ties, route, ["%.2e" % v for v in e])


@pytest.mark.parametrize("n,k,m", [(5000, 900, 2), (140001, 131073, 1)])
def test_backward_phased_general_route_bitwise(n, k, m):
    a, phi, b, psi, x, g = _case(n, k, m, 11, True)
    r0 = _run(a, phi, b, psi, x, g, False)
    r1 = _run(a, phi, b, psi, x, g, True)
    for u, v in zip(r0, r1):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))


def test_backward_phased_general_matches_symmetric_when_b_is_a():
    """b = a and psi = phi as separate arrays: dx is the symmetric phased dx,
    and the row and column gradients add up to the symmetric ones."""
    import laplace_prefix_scans_amd as lp
    n, m = 30000, 1
    a, phi, _, _, _, g = _case(n, 1, m, 5, False)
    x = _rng(6).standard_normal((n, m)).astype(np.float32)
    dx, da, db, dphi, dpsi = _run(a, phi, a.copy(), phi.copy(), x, g, True)
    a_s, perm = lp.laplex_sort_anchors(dev(a))
    sx, sa, sp = (host(t) for t in lp.laplex_backward_phased(a_s, perm, dev(phi), dev(x), dev(g)))
    kx, kg = oracle.sym_apply(a, np.abs(x)), oracle.sym_apply(a, np.abs(g))
    env = (np.abs(g) * kx + np.abs(x) * kg).sum(axis=1)
    assert oracle.normwise_error(dx, sx.astype(np.float64), kg) <= 2 * TOL
    assert np.max(np.abs((da + db) - sa)) / np.max(env) <= 2 * TOL
    assert np.max(np.abs((dphi + dpsi) - sp)) / np.max(env) <= 2 * TOL


def test_backward_phased_general_empty_sides():
    import torch
    import laplace_prefix_scans_amd as lp
    a_s, pa = lp.laplex_sort_anchors(dev(np.linspace(0, 9, 10, dtype=np.float32)))
    e = torch.empty(0, device="cuda")
    ep = torch.empty(0, dtype=torch.uint32, device="cuda")
    ph = torch.ones(10, device="cuda")
    f = lambda: torch.full((10,), 7.0, device="cuda")
    da, dphi = f(), f()
    lp.laplex_backward_phased_general(a_s, pa, ph, e, ep, e, torch.empty(0, 1, device="cuda"), torch.ones(10, 1, device="cuda"),
                                      out=(torch.empty(0, 1, device="cuda"), da, e.clone(), dphi, e.clone()))
    assert np.all(host(da) == 0.0) and np.all(host(dphi) == 0.0)
    dx, db, dpsi = torch.full((10, 1), 7.0, device="cuda"), f(), f()
    lp.laplex_backward_phased_general(e, ep, e, a_s, pa, ph, torch.ones(10, 1, device="cuda"), torch.empty(0, 1, device="cuda"),
                                      out=(dx, e.clone(), db, e.clone(), dpsi))
    assert np.all(host(dx) == 0.0) and np.all(host(db) == 0.0) and np.all(host(dpsi) == 0.0)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_backward_phased_general_workload_shape():
    """The general workload's anchors (n = 2^24, k = 2^16, m = 1) with seeded
    phases: every element of the five outputs against the oracle is too slow
    densely, so rows and columns are sampled: da, dphi at rows and db, dpsi at
    columns by the plain definition (dense slices of W)."""
    from synth import make_workload
    w = make_workload("gen2p24k2p16")
    r = _rng(24)
    phi = r.uniform(0, 2 * np.pi, w.n).astype(np.float32)
    psi = r.uniform(0, 2 * np.pi, w.k).astype(np.float32)
    x = w.x.reshape(w.k, 1)
    g = r.standard_normal((w.n, 1)).astype(np.float32)
    dx, da, db, dphi, dpsi = _run(w.a, phi, w.b, psi, x, g, True)
    print("gpu done", flush=True)
    rows = np.unique(r.integers(0, w.n, 24))
    cols = np.unique(r.integers(0, w.k, 24))
    a64, b64 = w.a.astype(np.float64), w.b.astype(np.float64)
    # rows: sums over all k columns
    D = a64[rows, None] - b64[None, :]
    P = phi[rows, None].astype(np.float64) - psi[None, :].astype(np.float64)
    K = np.exp(-np.abs(D))
    gx = g[rows].astype(np.float64) @ x.astype(np.float64).T
    da_ref = -(np.sign(D) * K * np.cos(P) * gx).sum(axis=1)
    dphi_ref = -(K * np.sin(P) * gx).sum(axis=1)
    env_r = (K * (np.abs(g[rows]).astype(np.float64) @ np.abs(x).astype(np.float64).T)).sum(axis=1)
    # columns: sums over all n rows, in chunks
    db_ref = np.zeros(cols.size)
    dpsi_ref = np.zeros(cols.size)
    dx_ref = np.zeros(cols.size)
    env_c = np.zeros(cols.size)
    for lo in range(0, w.n, 1 << 22):
        hi = min(w.n, lo + (1 << 22))
        D = a64[lo:hi, None] - b64[None, cols]
        P = phi[lo:hi, None].astype(np.float64) - psi[None, cols].astype(np.float64)
        K = np.exp(-np.abs(D))
        gc = g[lo:hi, 0].astype(np.float64)
        xc = x[cols, 0].astype(np.float64)
        db_ref += (np.sign(D) * K * np.cos(P) * gc[:, None]).sum(axis=0) * xc
        dpsi_ref += (K * np.sin(P) * gc[:, None]).sum(axis=0) * xc
        dx_ref += (K * np.cos(P) * gc[:, None]).sum(axis=0)
        env_c += (K * np.abs(gc)[:, None]).sum(axis=0)
    e = [float(np.max(np.abs(da[rows] - da_ref)) / np.max(env_r)),
         float(np.max(np.abs(dphi[rows] - dphi_ref)) / np.max(env_r)),
         float(np.max(np.abs(db[cols] - db_ref)) / np.max(env_c * np.abs(x[cols, 0]))),
         float(np.max(np.abs(dpsi[cols] - dpsi_ref)) / np.max(env_c * np.abs(x[cols, 0]))),
         float(np.max(np.abs(dx[cols, 0] - dx_ref)) / np.max(env_c))]
    print("sampled errors %s" % ["%.2e" % v for v in e], flush=True)
    assert max(e) <= TOL

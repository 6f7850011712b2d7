"""GPU parity of the symmetric phased backward (dx = W g, anchor gradient da,
phase gradient dphi; W_ij = exp(-|a_i - a_j|) cos(phi_i - phi_j)) with the
float64 oracle, through the C-ABI.

Error measure, per output: ||y - y_ref||_inf / ||envelope||_inf with the
unphased envelopes K|g| for dx and  sum_c |g_c| K|x_c| + |x_c| K|g_c|  for da
and dphi (the sizes of the summands the fp32 scans add up)."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([0xBAC5, seed]))


def _case(n, m, seed, ties):
    r = _rng(seed)
    a = r.uniform(0, n / 8.0 + 1.0, n).astype(np.float32)
    if ties:
        a = np.round(a).astype(np.float32)
    phi = r.uniform(0, 2 * np.pi, n).astype(np.float32)
    x = r.standard_normal((n, m)).astype(np.float32)
    g = r.standard_normal((n, m)).astype(np.float32)
    return a, phi, x, g


def _envelopes(a, x, g):
    kx, kg = oracle.sym_apply(a, np.abs(x)), oracle.sym_apply(a, np.abs(g))
    return kg, (np.abs(g) * kx + np.abs(x) * kg).sum(axis=1)


def _errors(a, phi, x, g, dx, da, dphi):
    dx_ref, da_ref, dp_ref = oracle.dense_phased_backward(a, phi, x, g)
    env_dx, env_v = _envelopes(a, x, g)
    e_dx = oracle.normwise_error(dx.reshape(dx_ref.shape), dx_ref, env_dx)
    e_da = float(np.max(np.abs(da - da_ref)) / np.max(env_v))
    e_dp = float(np.max(np.abs(dphi - dp_ref)) / np.max(env_v))
    return e_dx, e_da, e_dp


def _run(a, phi, x, g, route):
    import laplace_prefix_scans_amd as lp
    ra = lp.route_buffer(a.size) if route else None
    a_s, perm = lp.laplex_sort_anchors(dev(a), route=ra, check=True)
    dx, da, dphi = lp.laplex_backward_phased(a_s, perm, dev(phi), dev(x), dev(g), route=ra)
    return host(dx), host(da), host(dphi)


CASES = [(1, 1), (2, 1), (7, 2), (1000, 1), (1024, 1), (1025, 3), (4097, 4), (5000, 8), (3001, 6), (6000, 2)]


@pytest.mark.parametrize("n,m", CASES)
@pytest.mark.parametrize("ties", [False, True])
def test_backward_phased_parity(n, m, ties):
    a, phi, x, g = _case(n, m, 200 + n + 7 * m, ties)
    for route in ((False, True) if m <= 4 else (False,)):
        dx, da, dphi = _run(a, phi, x, g, route)
        assert np.isfinite(dx).all() and np.isfinite(da).all() and np.isfinite(dphi).all()
        errs = _errors(a, phi, x, g, dx, da, dphi)
        assert max(errs) <= TOL, "n=%d m=%d ties=%s route=%s: dx %.2e da %.2e dphi %.2e" % ((n, m, ties, route) + errs)


@pytest.mark.parametrize("n,m", [(5000, 1), (7001, 2), (999, 4), ((1 << 17) + 1, 2)])
def test_backward_phased_route_bitwise(n, m):
    """Moving rows along the route or by index gives the same bits."""
    a, phi, x, g = _case(n, m, 9 + n, True)
    r0 = _run(a, phi, x, g, False)
    r1 = _run(a, phi, x, g, True)
    for u, v in zip(r0, r1):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))


def test_backward_phased_zero_phase_is_the_symmetric_backward():
    """With every phase zero the phased operator is the plain one: dx and da
    match the symmetric backward and the phase gradient is zero."""
    import laplace_prefix_scans_amd as lp
    n, m = 20000, 2
    a, _, x, g = _case(n, m, 5, True)
    phi = np.zeros(n, np.float32)
    dx, da, dphi = _run(a, phi, x, g, True)
    a_s, perm = lp.laplex_sort_anchors(dev(a))
    dxs, das = lp.laplex_backward_sym(a_s, perm, dev(x), dev(g))
    env_dx, env_v = _envelopes(a, x, g)
    assert oracle.normwise_error(dx, host(dxs).astype(np.float64), env_dx) <= 2 * TOL
    assert np.max(np.abs(da - host(das))) / np.max(env_v) <= 2 * TOL
    assert np.max(np.abs(dphi)) / np.max(env_v) <= TOL


def test_backward_phased_rejects_bad_arguments():
    import torch
    import laplace_prefix_scans_amd as lp
    a_s, perm = lp.laplex_sort_anchors(dev(np.arange(100, dtype=np.float32)))
    phi = torch.zeros(100, device="cuda")
    x = torch.zeros(100, 2, device="cuda")
    with pytest.raises(ValueError):
        lp.laplex_backward_phased(a_s, perm, phi, x, torch.zeros(100, 3, device="cuda"))
    with pytest.raises(ValueError):
        lp.laplex_backward_phased(a_s, perm, torch.zeros(99, device="cuda"), x, x)
    with pytest.raises(lp.LaplexError):
        lp.laplex_backward_phased(a_s, perm, phi, x, x.clone(), dx=x)  # output on top of an input
    with pytest.raises(lp.LaplexError):
        lp.laplex_backward_phased(a_s, perm, phi, x, x.clone(), dphi=phi)  # phase gradient on top of the phases


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_backward_phased_full_workload():
    """The phased workload at full size (n = 3 * 2^20 flattened-image anchors,
    m = 8): da and dphi at spot rows against the plain definition, and dx = W g
    through the symmetry <u, dx(g)> = <W u, g> with the GPU's phased apply."""
    import torch
    import laplace_prefix_scans_amd as lp
    from synth import make_workload
    w = make_workload("phased3x1024x1024m8")
    r = _rng(31)
    g = r.standard_normal((w.n, w.m)).astype(np.float32)
    a_s, perm = lp.laplex_sort_anchors(dev(w.a), check=True)
    phi_d, g_d = dev(w.phi), dev(g)
    dx, da, dphi = lp.laplex_backward_phased(a_s, perm, phi_d, dev(w.x), g_d)
    torch.cuda.synchronize()
    print("gpu done", flush=True)
    p = host(perm)
    rows = np.unique(np.concatenate([p[[0, 1, 1023, 1024, w.n // 2, w.n - 1]].astype(np.int64), r.integers(0, w.n, 10)]))
    da_ref, dp_ref, env = oracle.phased_backward_rows(rows, w.a, w.phi, w.x, g)
    e_da = float(np.max(np.abs(host(da)[rows] - da_ref)) / np.max(env))
    e_dp = float(np.max(np.abs(host(dphi)[rows] - dp_ref)) / np.max(env))
    print("sampled errors da %.3e dphi %.3e over %d rows" % (e_da, e_dp, rows.size), flush=True)
    assert e_da <= TOL and e_dp <= TOL
    u = torch.randn(w.n, w.m, device="cuda", generator=torch.Generator(device="cuda").manual_seed(3))
    wu = lp.laplex_matvec_phased(a_s, perm, phi_d, u)
    lhs = float(torch.sum(u.double() * dx.double()))
    rhs = float(torch.sum(wu.double() * g_d.double()))
    ka = lp.laplex_matvec_sym(a_s, perm, g_d.abs())
    scale = float(torch.sum(u.abs().double() * ka.double()))
    print("dx symmetry |lhs-rhs|/scale = %.3e" % (abs(lhs - rhs) / scale), flush=True)
    assert abs(lhs - rhs) <= TOL * scale

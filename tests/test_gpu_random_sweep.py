"""GPU parity over seeded random cases: every entry point of the forward
operator (sort handle + symmetric, general and phased applies, with and
without the sort's route; the one-call symmetric and general paths) at
random sizes, column counts and anchor distributions (uniform, normal,
integer ties, tight clusters far apart, a wide range of magnitudes), each
case new (no case is run twice).  Permutations bit for bit against the
oracle's stable argsort; outputs finite and within the normwise bar of the
float64 oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, describe_nonfinite, dev, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

KINDS = ["sym", "sym_one_call", "general", "general_one_call", "phased", "phased_general"]
NCASES = 48


def _anchors(r, n, dist):
    if dist == "uniform":
        return r.uniform(0, n / 8.0 + 1.0, n)
    if dist == "normal":
        return r.normal(0, max(1.0, n / 50.0), n)
    if dist == "int_ties":
        return r.integers(-max(1, n // 20), max(2, n // 20), n).astype(np.float64)
    if dist == "clusters":  # a few tight groups, 300 apart (couplings between groups underflow)
        return r.integers(0, 7, n) * 300.0 + r.normal(0, 0.5, n)
    return r.standard_normal(n) * 10.0 ** r.uniform(-3, 4, n)  # "wide"


def _case(i):
    r = np.random.default_rng(np.random.SeedSequence([0x5EE9, i]))
    kind = KINDS[i % len(KINDS)]
    n = int(r.choice([1, 2, 3, 31, 4095, 4097, 8193]) if r.random() < 0.25 else r.integers(1, 150001))
    k = int(r.integers(1, 80001))
    m_choices = [1, 2, 3, 4, 8] if kind.startswith("phased") else [1, 2, 3, 4, 5, 8, 12, 16]
    m = int(r.choice(m_choices))
    dist = str(r.choice(["uniform", "normal", "int_ties", "clusters", "wide"]))
    routed = bool(r.random() < 0.5)
    a = _anchors(r, n, dist).astype(np.float32)
    b = _anchors(r, k, dist).astype(np.float32)
    if kind.startswith("general") or kind == "phased_general":
        b[: min(k, n, 3)] = a[: min(k, n, 3)]  # exact coincidences a_i == b_j
    rows = k if kind in ("general", "general_one_call", "phased_general") else n
    x = r.standard_normal((rows, m)).astype(np.float32)
    phi = r.uniform(0, 2 * np.pi, n).astype(np.float32)
    psi = r.uniform(0, 2 * np.pi, k).astype(np.float32)
    return kind, n, k, m, dist, routed, a, b, x, phi, psi


def _sorted(lp, arr, routed):
    route = lp.route_buffer(arr.size) if routed else None
    a_s, perm = lp.laplex_sort_anchors(dev(arr), route=route, check=True)
    assert np.array_equal(host(perm), oracle.stable_argsort(arr)), "permutation differs from the stable argsort"
    return a_s, perm, route


@pytest.mark.parametrize("i", range(NCASES))
def test_random_case(i):
    import laplace_prefix_scans_amd as lp
    kind, n, k, m, dist, routed, a, b, x, phi, psi = _case(i)
    print("case %d: %s n=%d k=%d m=%d anchors=%s routed=%s" % (i, kind, n, k, m, dist, routed), flush=True)
    perm_h = None
    if kind == "sym":
        a_s, pa, ra = _sorted(lp, a, routed)
        perm_h = host(pa)
        y = host(lp.laplex_matvec_sym(a_s, pa, dev(x), route=ra))
        ref, env = oracle.sym_apply(a, x), oracle.sym_apply(a, np.abs(x))
    elif kind == "sym_one_call":
        y = host(lp.laplex_sort_matvec_sym(dev(a), dev(x), check=True))
        ref, env = oracle.sym_apply(a, x), oracle.sym_apply(a, np.abs(x))
    elif kind == "general":
        a_s, pa, ra = _sorted(lp, a, routed)
        b_s, pb, rb = _sorted(lp, b, routed)
        y = host(lp.laplex_matvec_general(a_s, pa, b_s, pb, dev(x), route_a=ra, route_b=rb))
        ref, env = oracle.general_apply(a, b, x), oracle.general_apply(a, b, np.abs(x))
    elif kind == "general_one_call":
        y = host(lp.laplex_sort_matvec_general(dev(a), dev(b), dev(x), check=True))
        ref, env = oracle.general_apply(a, b, x), oracle.general_apply(a, b, np.abs(x))
    elif kind == "phased":
        a_s, pa, ra = _sorted(lp, a, routed)
        perm_h = host(pa)
        y = host(lp.laplex_matvec_phased(a_s, pa, dev(phi), dev(x), route_a=ra))
        ref, env = oracle.phased_apply(a, phi, x), oracle.sym_apply(a, np.abs(x))
    else:
        a_s, pa, ra = _sorted(lp, a, routed)
        b_s, pb, rb = _sorted(lp, b, routed)
        y = host(lp.laplex_matvec_phased(a_s, pa, dev(phi), dev(x), b_sorted=b_s, perm_b=pb, psi=dev(psi), route_a=ra,
                                         route_b=rb))
        ref, env = oracle.phased_apply(a, phi, x, b=b, psi=psi), oracle.general_apply(a, b, np.abs(x))
    if not np.isfinite(y).all():
        where = describe_nonfinite(y, perm_h) if perm_h is not None else "non-finite output"
        pytest.fail("case %d (%s n=%d m=%d): %s" % (i, kind, n, m, where))
    err = oracle.normwise_error(y, ref, env)
    assert err <= TOL, "case %d (%s n=%d k=%d m=%d %s routed=%s): err=%.3e" % (i, kind, n, k, m, dist, routed, err)

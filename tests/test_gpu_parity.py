"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Sort: permutation bit-exact against the oracle's stable argsort, sorted
anchors bit-exact.  Operator applies: normwise error
||y - y_ref||_inf / ||K0|x|||_inf <= 1e-5 per column (fp32 against float64),
with exact checks where the arithmetic is exact.
"""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, assert_perm_is_stable_argsort, describe_nonfinite, dev, gpu_sort, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([0x6B0, seed]))


def _anchor_cases():
    r = _rng(1)
    return {
        "n1": np.array([3.5], np.float32),
        "n2_tie": np.array([1.0, 1.0], np.float32),
        "signed_zero": np.array([0.0, -0.0, 1.0, -0.0, 0.0, -1.0, -0.0], np.float32),
        "uniform_4095": r.uniform(0, 512, 4095).astype(np.float32),
        "uniform_4096": r.uniform(0, 512, 4096).astype(np.float32),
        "uniform_4097": r.uniform(0, 512, 4097).astype(np.float32),
        "ints_ties_20000": r.integers(-50, 50, 20000).astype(np.float32),
        "all_equal_9000": np.full(9000, -7.25, np.float32),
        "sorted_10000": np.sort(r.standard_normal(10000).astype(np.float32)),
        "reversed_10000": np.sort(r.standard_normal(10000).astype(np.float32))[::-1].copy(),
        "wide_range_30000": (r.standard_normal(30000) * 1e30).astype(np.float32),
        "dense_ties_2p20": r.uniform(0, 2 ** 17, 1 << 20).astype(np.float32),
        "ragged_300001": r.uniform(-1e4, 1e4, 300001).astype(np.float32),
        # around the size (64 tiles of 8192) from which the first pass takes
        # its offsets from the histogram's per-tile tables
        "tiles63_ties": r.integers(-3000, 3000, 63 * 8192).astype(np.float32),
        "tiles64_ragged": r.uniform(0, 1e5, 64 * 8192 - 5).astype(np.float32),
        "signed_zero_600000": r.choice(np.array([0.0, -0.0, 2.0, -2.0], np.float32), 600000),
        # 257 histogram chunks: two chunks per histogram block, some blocks empty
        "chunks257_int_ties": r.integers(0, 1 << 12, 16384 * 257 + 3).astype(np.float32),
        # sorts of up to 2^17 keys run on 2048-key tiles, larger ones on 8192:
        # both sides of the switch, and the small cases' patterns on the
        # large tiles
        "switch_131072_ties": r.integers(-500, 500, 1 << 17).astype(np.float32),
        "switch_131073_ties": r.integers(-500, 500, (1 << 17) + 1).astype(np.float32),
        "all_equal_140000": np.full(140000, 2.5, np.float32),
        "sorted_140001": np.sort(r.standard_normal(140001).astype(np.float32)),
        "reversed_140001": np.sort(r.standard_normal(140001).astype(np.float32))[::-1].copy(),
        "signed_zero_131075": r.choice(np.array([0.0, -0.0, 3.0, -3.0], np.float32), 131075),
        "wide_range_140000": (r.standard_normal(140000) * 1e30).astype(np.float32),
    }


@pytest.mark.parametrize("name", sorted(_anchor_cases()))
def test_sort_bit_exact(name):
    a = _anchor_cases()[name]
    _, a_s, perm = gpu_sort(a)
    perm_h, a_s_h = host(perm), host(a_s)
    ref = oracle.stable_argsort(a)
    assert np.array_equal(perm_h, ref), "perm differs from the stable argsort"
    assert np.array_equal(a_s_h.view(np.uint32), a[ref].view(np.uint32)), "a_sorted differs from a[perm] bitwise"


def test_sort_rejects_nonfinite():
    import laplace_prefix_scans_amd as lp
    for bad in (np.nan, np.inf, -np.inf):
        a = np.linspace(0, 1, 5000).astype(np.float32)
        a[1234] = bad
        with pytest.raises(lp.LaplexError) as ei:
            lp.laplex_sort_anchors(dev(a), check=True)
        assert ei.value.code == 5


def _sym_case(n, m, spread, seed, ties=False):
    r = _rng(seed)
    a = r.uniform(0, spread, n).astype(np.float32)
    if ties:
        a = np.round(a).astype(np.float32)
    x = r.standard_normal((n, m)).astype(np.float32)
    return a, x


SYM_CASES = [(1, 1), (2, 3), (7, 1), (255, 2), (4096, 1), (4097, 1), (5000, 3), (70001, 1), (70001, 8), (65536, 16),
             (12345, 5), (300000, 1), (100000, 4)]


@pytest.mark.parametrize("n,m", SYM_CASES)
def test_sym_parity(n, m):
    import laplace_prefix_scans_amd as lp
    for ties in (False, True):
        a, x = _sym_case(n, m, n / 8.0 + 1.0, 10 + n + m, ties)
        _, a_s, perm = gpu_sort(a)
        pa = host(perm)
        bad = np.nonzero(pa != oracle.stable_argsort(a))[0]
        assert bad.size == 0, "sym n=%d m=%d ties=%s: perm differs at %d positions, first %d" % (n, m, ties, bad.size, bad[0])
        y = host(lp.laplex_matvec_sym(a_s, perm, dev(x)))
        assert np.isfinite(y).all(), "sym n=%d m=%d ties=%s: %s" % (
            n, m, ties, describe_nonfinite(y, pa))
        ref = oracle.sym_apply(a, x)
        env = oracle.sym_apply(a, np.abs(x))
        err = oracle.normwise_error(y, ref, env)
        assert err <= TOL, "sym n=%d m=%d ties=%s err=%.3e" % (n, m, ties, err)


GEN_CASES = [(1, 1, 1), (5, 3, 2), (4096, 17, 1), (3000, 5000, 1), (20000, 700, 3), (100000, 100000, 1), (70000, 1000, 8),
             (1000, 70000, 4), (50000, 2, 1)]


@pytest.mark.parametrize("n,k,m", GEN_CASES)
def test_general_parity(n, k, m):
    import laplace_prefix_scans_amd as lp
    r = _rng(100 + n + k + m)
    a = r.normal(0, 30, n).astype(np.float32)
    b = r.normal(0, 30, k).astype(np.float32)
    b[: min(k, 5)] = a[: min(k, 5)] if n >= 5 else b[: min(k, 5)]   # exact coincidences a_i == b_j
    xb = r.standard_normal((k, m)).astype(np.float32)
    _, a_s, pa = gpu_sort(a)
    _, b_s, pb = gpu_sort(b)
    y = host(lp.laplex_matvec_general(a_s, pa, b_s, pb, dev(xb)))
    ref = oracle.general_apply(a, b, xb)
    env = oracle.general_apply(a, b, np.abs(xb))
    err = oracle.normwise_error(y, ref, env)
    assert err <= TOL, "general n=%d k=%d m=%d err=%.3e" % (n, k, m, err)


@pytest.mark.parametrize("n,m", [(1, 1), (9, 2), (4096, 1), (5000, 3), (70001, 8), (30000, 4), (200000, 1)])
def test_phased_sym_parity(n, m):
    import laplace_prefix_scans_amd as lp
    r = _rng(200 + n + m)
    a = r.uniform(0, n / 8.0 + 1, n).astype(np.float32)
    phi = r.uniform(0, 2 * np.pi, n).astype(np.float32)
    x = r.standard_normal((n, m)).astype(np.float32)
    _, a_s, perm = gpu_sort(a)
    y = host(lp.laplex_matvec_phased(a_s, perm, dev(phi), dev(x)))
    ref = oracle.phased_apply(a, phi, x)
    env = oracle.sym_apply(a, np.abs(x))
    err = oracle.normwise_error(y, ref, env)
    assert err <= TOL, "phased n=%d m=%d err=%.3e" % (n, m, err)


@pytest.mark.parametrize("n,k,m", [(1, 1, 1), (300, 200, 2), (20000, 3000, 1), (5000, 60000, 3), (40000, 40000, 8)])
def test_phased_general_parity(n, k, m):
    import laplace_prefix_scans_amd as lp
    r = _rng(300 + n + k + m)
    a = r.normal(0, 20, n).astype(np.float32)
    b = r.normal(0, 20, k).astype(np.float32)
    phi = r.uniform(0, 2 * np.pi, n).astype(np.float32)
    psi = r.uniform(0, 2 * np.pi, k).astype(np.float32)
    xb = r.standard_normal((k, m)).astype(np.float32)
    _, a_s, pa = gpu_sort(a)
    _, b_s, pb = gpu_sort(b)
    y = host(lp.laplex_matvec_phased(a_s, pa, dev(phi), dev(xb), b_sorted=b_s, perm_b=pb, psi=dev(psi)))
    ref = oracle.phased_apply(a, phi, xb, b=b, psi=psi)
    env = oracle.general_apply(a, b, np.abs(xb))
    err = oracle.normwise_error(y, ref, env)
    assert err <= TOL, "phased general n=%d k=%d m=%d err=%.3e" % (n, k, m, err)


def test_exact_special_cases():
    """n = 1 gives y = x exactly; K e_j has exactly 1.0 at j and its tie
    partners; anchors 200 apart make K a permutation (exp(-200) underflows)."""
    import laplace_prefix_scans_amd as lp
    x1 = np.array([[1.5, -2.25, 3.0]], np.float32)
    _, a_s, perm = gpu_sort(np.array([4.0], np.float32))
    assert np.array_equal(host(lp.laplex_matvec_sym(a_s, perm, dev(x1))), x1)
    r = _rng(5)
    n = 20000
    a = (r.integers(0, 3000, n) * 0.5).astype(np.float32)
    _, a_s, perm = gpu_sort(a)
    for j in (0, 777, 4096, n - 1):
        e = np.zeros(n, np.float32)
        e[j] = 1.0
        y = host(lp.laplex_matvec_sym(a_s, perm, dev(e)))
        assert np.all(y[a == a[j]] == 1.0), "tie partner of e_j not exactly 1"
        col = np.exp(-np.abs(a.astype(np.float64) - float(a[j])))
        assert np.max(np.abs(y - col)) <= TOL
    pi = r.permutation(5000)
    a = (200.0 * pi).astype(np.float32)
    b = (200.0 * np.arange(5000)).astype(np.float32)
    x = r.standard_normal((5000, 2)).astype(np.float32)
    _, a_s, pa = gpu_sort(a)
    _, b_s, pb = gpu_sort(b)
    y = host(lp.laplex_matvec_general(a_s, pa, b_s, pb, dev(x)))
    assert np.array_equal(y, x[pi]), "zero-temperature general apply is not the permutation"
    y = host(lp.laplex_matvec_sym(a_s, pa, dev(x)))
    assert np.array_equal(y, x), "zero-temperature symmetric apply is not the identity"


def test_general_k0_and_empty():
    import torch
    import laplace_prefix_scans_amd as lp
    a = np.linspace(0, 1, 100).astype(np.float32)
    _, a_s, pa = gpu_sort(a)
    b_s = torch.empty(0, dtype=torch.float32, device="cuda")
    pb = torch.empty(0, dtype=torch.uint32, device="cuda")
    y = host(lp.laplex_matvec_general(a_s, pa, b_s, pb, torch.empty((0, 2), device="cuda")))
    assert y.shape == (100, 2) and np.all(y == 0)
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    s, p = lp.laplex_sort_anchors(e)
    assert s.numel() == 0 and p.numel() == 0


def test_deterministic():
    """Same inputs, same bits (fixed reduction order; the look-back only moves integers)."""
    import laplace_prefix_scans_amd as lp
    a, x = _sym_case(300000, 2, 30000.0, 77)
    outs = []
    for _ in range(3):
        _, a_s, perm = gpu_sort(a)
        outs.append((host(perm), host(lp.laplex_matvec_sym(a_s, perm, dev(x)))))
    for p, y in outs[1:]:
        assert np.array_equal(p, outs[0][0])
        assert np.array_equal(y.view(np.uint32), outs[0][1].view(np.uint32))

"""GPU parity of the one-call sort + symmetric apply (laplex_sort_matvec_sym)
with the float64 oracle, and its bitwise agreement with the two-call path
(laplex_sort_anchors with a route, then laplex_matvec_sym).  With one column
x rides through the sort's passes as the keys' values, so these tests also
pin that the carried values come out in the sort's order."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([0x50F7, seed]))


def _case(n, m, seed, kind):
    r = _rng(seed)
    if kind == "ties":
        a = np.round(r.uniform(0, n / 8.0 + 1.0, n)).astype(np.float32)
    elif kind == "signed_zero":  # -0.0 and +0.0 (equal anchors) mixed with small values of both signs
        a = r.choice(np.array([-0.0, 0.0, 1.0, -1.0, 0.5], np.float32), n)
    else:
        a = r.uniform(-n / 16.0, n / 16.0, n).astype(np.float32)
    x = r.standard_normal((n, m)).astype(np.float32)
    return a, x


def _two_call(a, x, route):
    import laplace_prefix_scans_amd as lp
    ra = lp.route_buffer(a.size) if route else None
    a_s, perm = lp.laplex_sort_anchors(dev(a), route=ra, check=True)
    return host(lp.laplex_matvec_sym(a_s, perm, dev(x), route=ra))


CASES = [(1, 1), (2, 1), (3, 2), (1000, 1), (4096, 1), (8192, 1), (8193, 1), (70001, 1), (300000, 1), (600001, 1), (5000, 2),
         (9001, 3), (8191, 4), (6000, 5), (3001, 8)]


@pytest.mark.parametrize("n,m", CASES)
@pytest.mark.parametrize("kind", ["uniform", "ties", "signed_zero"])
def test_sort_matvec_parity(n, m, kind):
    import laplace_prefix_scans_amd as lp
    a, x = _case(n, m, n + 17 * m, kind)
    y = host(lp.laplex_sort_matvec_sym(dev(a), dev(x), check=True))
    assert np.isfinite(y).all()
    err = oracle.normwise_error(y, oracle.sym_apply(a, x), oracle.sym_apply(a, np.abs(x)))
    assert err <= TOL, "n=%d m=%d %s: %.2e" % (n, m, kind, err)
    # the same bits as the two-call path (routed when m <= 4, by index above)
    y2 = _two_call(a, x, m <= 4)
    assert np.array_equal(y.view(np.uint32), y2.reshape(y.shape).view(np.uint32))


def test_sort_matvec_vector_input_and_reuse():
    """A 1-D x gives a 1-D y; one workspace serves calls of different sizes
    (every call clears what it counts with), each equal to a fresh call."""
    import laplace_prefix_scans_amd as lp
    ws = lp.workspace(lp.LAPLEX_OP_SORT_SYM, 50000, 0, 1)
    for n in (50000, 777, 50000, 12345):
        a, x = _case(n, 1, 3 * n, "ties")
        y = lp.laplex_sort_matvec_sym(dev(a), dev(x[:, 0]), ws=ws)
        assert tuple(y.shape) == (n,)
        y_fresh = lp.laplex_sort_matvec_sym(dev(a), dev(x[:, 0]))
        assert np.array_equal(host(y).view(np.uint32), host(y_fresh).view(np.uint32))


def test_sort_matvec_rejects_nonfinite_and_bad_arguments():
    import torch
    import laplace_prefix_scans_amd as lp
    a = np.linspace(0, 9, 10000).astype(np.float32)
    a[777] = np.nan
    with pytest.raises(lp.LaplexError):
        lp.laplex_sort_matvec_sym(dev(a), torch.ones(10000, device="cuda"), check=True)
    a_ok = torch.arange(100, dtype=torch.float32, device="cuda")
    x = torch.ones(100, 2, device="cuda")
    with pytest.raises(ValueError):
        lp.laplex_sort_matvec_sym(a_ok, torch.ones(99, device="cuda"))
    with pytest.raises(lp.LaplexError):
        lp.laplex_sort_matvec_sym(a_ok, x, y=x)  # output on top of the input
    ws = lp.workspace(lp.LAPLEX_OP_SORT_SYM, 50, 0, 2)
    with pytest.raises(lp.LaplexError):
        lp.laplex_sort_matvec_sym(a_ok, x, ws=ws)  # workspace for fewer anchors
    e = torch.empty(0, device="cuda")
    assert lp.laplex_sort_matvec_sym(e, e).numel() == 0

"""GPU parity of the one-call general operator (laplex_sort_matvec_general),
which sorts only the input anchors b, runs the two scans over sorted b and
lets every output anchor find its interval in b by binary search, against
the float64 oracle (the pages' u/v form) and against the sort-handle path.

Cases cover the search's two levels (a sample of b staged in LDS as a search
tree, then one group of b): k from 1 to past the largest group size, every
group size at both ends of its range, ties between a and b (b before a),
outputs below and above every input, and k larger than n."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([0x5EA4, seed]))


def _case(n, k, m, seed, kind):
    r = _rng(seed)
    span = (n + k) / 8.0 + 1.0
    if kind == "ties":
        a = np.round(r.uniform(0, span, n)).astype(np.float32)
        b = np.round(r.uniform(0, span, k)).astype(np.float32)
    elif kind == "outside":  # half the outputs below every input, half above
        b = r.uniform(100.0, 100.0 + span, k).astype(np.float32)
        a = np.concatenate([r.uniform(80.0, 100.0, n // 2), r.uniform(100.0 + span, 120.0 + span, n - n // 2)])
        a = r.permutation(a).astype(np.float32)
    else:
        a = r.uniform(0, span, n).astype(np.float32)
        b = r.uniform(0, span, k).astype(np.float32)
    x = r.standard_normal((k, m)).astype(np.float32)
    return a, b, x


# k: groups of 8 (k <= 2^16), 16 (k <= 2^17), 32, 64 (k <= 2^19) and the
# wide fallback above
CASES = [(1, 1, 1), (5, 1, 1), (1, 5, 2), (1000, 37, 1), (70001, 4096, 1), (70001, 4097, 2), (300000, 70001, 3),
         (200000, (1 << 16) + 5, 8), (150000, 200000, 1), (50000, 300000, 1), (4097, 8193, 4),
         (30000, 1 << 16, 1), (30000, 1 << 17, 1), (20000, (1 << 17) + 1, 2), (30000, 1 << 19, 1),
         (40000, (1 << 19) + 3, 1), (20000, 700001, 2)]


@pytest.mark.parametrize("n,k,m", CASES)
@pytest.mark.parametrize("kind", ["uniform", "ties", "outside"])
def test_sort_matvec_general_parity(n, k, m, kind):
    import laplace_prefix_scans_amd as lp
    a, b, x = _case(n, k, m, n + 3 * k + 7 * m, kind)
    y = host(lp.laplex_sort_matvec_general(dev(a), dev(b), dev(x), check=True))
    assert np.isfinite(y).all()
    ref = oracle.general_apply(a, b, x)
    env = oracle.general_apply(a, b, np.abs(x))
    err = oracle.normwise_error(y, ref, env)
    assert err <= TOL, "n=%d k=%d m=%d %s: %.2e" % (n, k, m, kind, err)
    # the sort-handle path agrees within the same bar
    a_s, pa = lp.laplex_sort_anchors(dev(a))
    b_s, pb = lp.laplex_sort_anchors(dev(b))
    y2 = host(lp.laplex_matvec_general(a_s, pa, b_s, pb, dev(x)))
    assert oracle.normwise_error(y, y2.reshape(y.shape).astype(np.float64), env) <= 2 * TOL


def test_sort_matvec_general_vector_and_reuse():
    """1-D x gives 1-D y; one workspace serves calls of different sizes."""
    import laplace_prefix_scans_amd as lp
    ws = lp.workspace(lp.LAPLEX_OP_SORT_GENERAL, 90000, 20000, 1)
    for n, k in ((90000, 20000), (1000, 50), (90000, 20000)):
        a, b, x = _case(n, k, 1, 17 * n + k, "ties")
        y = lp.laplex_sort_matvec_general(dev(a), dev(b), dev(x[:, 0]), ws=ws)
        assert tuple(y.shape) == (n,)
        y_fresh = lp.laplex_sort_matvec_general(dev(a), dev(b), dev(x[:, 0]))
        assert np.array_equal(host(y).view(np.uint32), host(y_fresh).view(np.uint32))


def test_sort_matvec_general_empty_and_errors():
    import torch
    import laplace_prefix_scans_amd as lp
    a = dev(np.linspace(0, 9, 10, dtype=np.float32))
    y = torch.full((10, 2), 7.0, device="cuda")
    lp.laplex_sort_matvec_general(a, torch.empty(0, device="cuda"), torch.empty(0, 2, device="cuda"), y=y, check=True)
    assert np.all(host(y) == 0.0)
    an = np.linspace(0, 9, 5000).astype(np.float32)
    an[4321] = np.inf
    with pytest.raises(lp.LaplexError):  # a non-finite output anchor
        lp.laplex_sort_matvec_general(dev(an), a, torch.ones(10, device="cuda"), check=True)
    with pytest.raises(lp.LaplexError):  # a non-finite input anchor
        lp.laplex_sort_matvec_general(a, dev(an), torch.ones(5000, device="cuda"), check=True)
    with pytest.raises(ValueError):
        lp.laplex_sort_matvec_general(a, a, torch.ones(9, device="cuda"))
    x = torch.ones(10, device="cuda")
    with pytest.raises(lp.LaplexError):
        lp.laplex_sort_matvec_general(a, a, x, y=x)  # output on top of the input


@pytest.mark.timeout(300)
def test_sort_matvec_general_workload():
    """The general workload (n = 2^24 outputs, k = 2^16 inputs) in the launch
    configuration the benchmark times, every output against the oracle."""
    import laplace_prefix_scans_amd as lp
    from synth import make_workload
    w = make_workload("gen2p24k2p16")
    y = host(lp.laplex_sort_matvec_general(dev(w.a), dev(w.b), dev(w.x), check=True))
    print("gpu done", flush=True)
    ref = oracle.general_apply(w.a, w.b, w.x)
    env = oracle.general_apply(w.a, w.b, np.abs(w.x))
    err = oracle.normwise_error(y, ref, env)
    print("normwise error %.3e" % err, flush=True)
    assert err <= TOL

"""GPU parity of the weighted Gram matrix M = A diag(D) A^T (A = LAPLEX(a, b))
with the float64 definition, through the C-ABI.

Error measure: max |M - M_ref| / max E with the envelope E = A diag(|D|) A^T
(the size of the summands), bar 1e-5 as for the matvec."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([0x6A4, seed]))


def _case(n, k, seed, ties=False, signed=True, span=None):
    r = _rng(seed)
    span = (n + k) / 16.0 + 1.0 if span is None else span
    a = r.uniform(0, span, n).astype(np.float32)
    b = r.uniform(0, span, k).astype(np.float32)
    if ties:
        a, b = np.round(a).astype(np.float32), np.round(b).astype(np.float32)
    D = (r.standard_normal(k) if signed else r.uniform(0, 1, k)).astype(np.float32)
    return a, b, D


def _handles(a, b):
    import laplace_prefix_scans_amd as lp
    a_s, pa = lp.laplex_sort_anchors(dev(a), check=True)
    b_s, pb = lp.laplex_sort_anchors(dev(b), check=True)
    return a_s, pa, b_s, pb


def _gram(a, b, D, **kw):
    import laplace_prefix_scans_amd as lp
    a_s, pa, b_s, pb = _handles(a, b)
    return lp.laplex_gram_weighted(a_s, pa, b_s, pb, dev(D), **kw)


def _error(M, a, b, D, rows=None):
    idx = np.arange(a.size)
    rows = idx if rows is None else rows
    ref = oracle.gram_block(rows, idx, a, b, D)
    env = oracle.gram_block(rows, idx, a, b, D, absolute=True)
    return float(np.max(np.abs(M - ref)) / np.max(env))


CASES = [(1, 1), (1, 7), (5, 1), (64, 64), (300, 5000), (1000, 37), (2049, 2048), (4097, 4095), (3000, 9000)]


@pytest.mark.parametrize("n,k", CASES)
@pytest.mark.parametrize("ties", [False, True])
def test_gram_parity(n, k, ties):
    a, b, D = _case(n, k, 10 + n + 3 * k, ties)
    M = host(_gram(a, b, D))
    assert M.shape == (n, n) and np.isfinite(M).all()
    err = _error(M, a, b, D)
    assert err <= TOL, "n=%d k=%d ties=%s: %.3e" % (n, k, ties, err)
    assert np.array_equal(M.view(np.uint32), M.T.view(np.uint32)), "M is not exactly symmetric"


def test_gram_symmetric_handle_equispaced():
    """b = a (the same sort handle), D = 1, equispaced anchors: M = K^2 with
    K the Kac-Murdock-Szego matrix."""
    import laplace_prefix_scans_amd as lp
    n, h = 3000, 0.5
    a = (np.arange(n) * h).astype(np.float32)[::-1].copy()  # given in reverse order
    a_s, pa = lp.laplex_sort_anchors(dev(a))
    M = host(lp.laplex_gram_weighted(a_s, pa, a_s, pa, dev(np.ones(n, np.float32))))
    K = np.exp(-np.abs(a[:, None].astype(np.float64) - a[None, :]))
    ref = K @ K
    assert np.max(np.abs(M - ref)) / np.max(ref) <= TOL


def test_gram_slabs_match_the_whole_matrix():
    """Rows in slabs with a leading dimension larger than n: the same bits as
    the whole matrix, and the padding columns untouched."""
    import torch
    import laplace_prefix_scans_amd as lp
    n, k = 5000, 3000
    a, b, D = _case(n, k, 21, True)
    a_s, pa, b_s, pb = _handles(a, b)
    Dd = dev(D)
    whole = host(lp.laplex_gram_weighted(a_s, pa, b_s, pb, Dd))
    ld = n + 13
    for r0, rc in ((0, 1), (1, 17), (777, 1024), (n - 3, 3)):
        buf = torch.full((rc, ld), -7.0, device="cuda")
        lp.laplex_gram_weighted(a_s, pa, b_s, pb, Dd, M=buf[:, :n] if rc > 1 else buf, row_begin=r0, row_count=rc)
        got = host(buf)
        assert np.array_equal(got[:, :n].view(np.uint32), whole[r0:r0 + rc].view(np.uint32)), (r0, rc)
        if rc > 1:
            assert np.all(got[:, n:] == -7.0), "padding written"


def test_gram_no_columns_is_zero():
    import torch
    import laplace_prefix_scans_amd as lp
    a_s, pa = lp.laplex_sort_anchors(dev(np.linspace(-3, 3, 100).astype(np.float32)))
    e = torch.empty(0, device="cuda")
    M = torch.full((100, 100), 5.0, device="cuda")
    lp.laplex_gram_weighted(a_s, pa, e, torch.empty(0, dtype=torch.uint32, device="cuda"), e, M=M)
    assert np.all(host(M) == 0.0)


def test_gram_far_apart_groups():
    """Two groups of anchors 300 apart (exp(-300) underflows in float32): the
    off-diagonal blocks are exactly zero and each diagonal block is its own
    group's Gram matrix."""
    r = _rng(5)
    a1, a2 = r.uniform(0, 10, 700).astype(np.float32), r.uniform(310, 320, 500).astype(np.float32)
    b1, b2 = r.uniform(0, 10, 900).astype(np.float32), r.uniform(310, 320, 400).astype(np.float32)
    D1, D2 = r.uniform(0, 1, 900).astype(np.float32), r.uniform(0, 1, 400).astype(np.float32)
    M = host(_gram(np.concatenate([a1, a2]), np.concatenate([b1, b2]), np.concatenate([D1, D2])))
    assert np.all(M[:700, 700:] == 0.0) and np.all(M[700:, :700] == 0.0)
    assert _error(M[:700, :700], a1, b1, D1) <= TOL
    assert _error(M[700:, 700:], a2, b2, D2) <= TOL


def test_gram_rejects_bad_arguments():
    import torch
    import laplace_prefix_scans_amd as lp
    a_s, pa = lp.laplex_sort_anchors(dev(np.arange(50, dtype=np.float32)))
    b_s, pb = lp.laplex_sort_anchors(dev(np.arange(20, dtype=np.float32)))
    D = torch.ones(20, device="cuda")
    with pytest.raises(ValueError):
        lp.laplex_gram_weighted(a_s, pa, b_s, pb, torch.ones(19, device="cuda"))
    with pytest.raises(ValueError):
        lp.laplex_gram_weighted(a_s, pa, b_s, pb, D, M=torch.empty(50, 49, device="cuda"))
    with pytest.raises(lp.LaplexError):
        lp.laplex_gram_weighted(a_s, pa, b_s, pb, D, row_begin=45, row_count=10)
    buf = torch.ones(200, device="cuda")
    with pytest.raises(lp.LaplexError):  # M (one row) on top of the weights
        lp.laplex_gram_weighted(a_s, pa, b_s, pb, buf[:20], M=buf[10:60].view(1, 50), row_count=1)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_gram_full_workload():
    """The Gram workload at full size (n = k = 2^16, 16 GiB of M): blocks of
    rows and columns (extremes, tile edges, random) against the definition,
    exact symmetry on them, and M v against A (D * (A^T v)) by the scan oracle."""
    import torch
    import laplace_prefix_scans_amd as lp
    from synth import make_workload
    w = make_workload("gram2p16k2p16")
    a_s, pa, b_s, pb = _handles(w.a, w.b)
    M = lp.laplex_gram_weighted(a_s, pa, b_s, pb, dev(w.D))
    torch.cuda.synchronize()
    print("gpu done", flush=True)
    n = w.n
    r = _rng(16)
    perm = host(pa).astype(np.int64)
    rows = np.unique(np.concatenate([perm[[0, 1, 4095, 4096, n // 2, n - 1]], r.integers(0, n, 26)]))
    cols = np.unique(np.concatenate([perm[[0, 2, 4096, n - 2, n - 1]], r.integers(0, n, 27)]))
    blk = host(M[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    ref = oracle.gram_block(rows, cols, w.a, w.b, w.D)
    env = oracle.gram_block(rows, cols, w.a, w.b, w.D, absolute=True)
    err = float(np.max(np.abs(blk - ref)) / np.max(env))
    print("sampled block error %.3e" % err, flush=True)
    assert err <= TOL
    blk_t = host(M[torch.from_numpy(cols).cuda()][:, torch.from_numpy(rows).cuda()])
    assert np.array_equal(blk.view(np.uint32), blk_t.T.view(np.uint32))
    v = r.standard_normal(n)
    mv = host(M @ dev(v.astype(np.float32))).astype(np.float64)
    atv = oracle.general_apply(w.b, w.a, v.astype(np.float32))[:, 0]
    want = oracle.general_apply(w.a, w.b, (w.D * atv).astype(np.float32))[:, 0]
    scale = oracle.general_apply(w.a, w.b, (w.D * oracle.general_apply(w.b, w.a, np.abs(v).astype(np.float32))[:, 0])
                                 .astype(np.float32))[:, 0]
    err_mv = float(np.max(np.abs(mv - want)) / np.max(scale))
    print("M v error %.3e" % err_mv, flush=True)
    assert err_mv <= 1e-4  # float32 product of 2^16 terms on top of M's own error

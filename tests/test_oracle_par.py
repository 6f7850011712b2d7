"""The all-cores oracle (the benchmark's CPU baseline) against the one-core
oracle: the same stable argsort bit for bit, and the same operator within
float64 rounding (a chunked two-pass scan against the sequential one)."""
import numpy as np
import pytest

import oracle


def _cases():
    r = np.random.default_rng(np.random.SeedSequence([0x0A11C0, 1]))
    return {
        "n1": (np.array([2.5], np.float32), 1),
        "tiny_ties": (np.array([1.0, 1.0, -0.0, 0.0, 3.0, 1.0], np.float32), 2),
        "uniform": (r.uniform(0, 300, 10007).astype(np.float32), 1),
        "integer_ties": (r.integers(-40, 40, 20011).astype(np.float32), 3),
        "all_equal": (np.full(5003, 7.0, np.float32), 1),
        "reversed": (np.sort(r.standard_normal(9001).astype(np.float32))[::-1].copy(), 2),
        "signed_zero": (r.choice(np.array([0.0, -0.0, 1.5], np.float32), 7777), 1),
        "wide": ((r.standard_normal(6000) * 1e4).astype(np.float32), 16),
    }


@pytest.mark.parametrize("name", sorted(_cases()))
def test_par_matches_sequential(name):
    a, m = _cases()[name]
    x = np.random.default_rng(len(name)).standard_normal((a.size, m)).astype(np.float32)
    assert np.array_equal(oracle.stable_argsort_par(a), oracle.stable_argsort(a))
    y_par = oracle.sym_apply_par(a, x)
    y_seq = oracle.sym_apply(a, x)
    env = oracle.sym_apply(a, np.abs(x))
    assert oracle.normwise_error(y_par, y_seq, env) <= 1e-13


def test_par_rejects_nonfinite():
    a = np.linspace(0, 1, 100).astype(np.float32)
    a[17] = np.nan
    with pytest.raises(ValueError):
        oracle.sym_apply_par(a, np.ones(100, np.float32))


def test_par_uses_threads():
    assert oracle.par_threads() >= 1

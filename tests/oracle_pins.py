"""Pins of the CPU oracle against facts other than the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a closed form, an invariant, a library routine that computes the same thing
another way, or brute force on tiny inputs.  ``lib`` is a loaded C oracle
(``oracle.load(path)``), so the same checks can be pointed at copies of the
oracle with a planted mistake (see test_oracle_mutations.py).

Sources: "LAPLEX: The FFT of Learnable Laplace Kernels" (technical summary):
section 2.1 (operator and phased operator), 2.2 (sort, prefix/suffix scans,
general case through u and v), 2.3 (zero-temperature permutation/CountSketch
limit; uniform grid reduces to Toeplitz-FFT; Laplace kernel's Cauchy spectral
density, hence positive definiteness).  The Kac-Murdock-Szego inverse and the
tridiagonal precision matrix of the exponential (Ornstein-Uhlenbeck)
covariance are textbook facts, not on the pages.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from oracle import dense as odense

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([0x0AC1E, seed]))


def _close(got, want, tol, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    scale = max(1.0, float(np.max(np.abs(want)))) if want.size else 1.0
    err = float(np.max(np.abs(got - want))) / scale if want.size else 0.0
    assert err <= tol, "%s: relative error %.3e > %.1e" % (what, err, tol)


# ----------------------------------------------------------------------------- sort

def pin_sort_definition(lib):
    """Stable ascending argsort: a permutation, nondecreasing values, ties in
    input order; -0.0 == +0.0.  Checked by the definition and against NumPy's
    stable sort (an independent library routine)."""
    r = _rng(1)
    cases = [
        np.array([0.0, -0.0, 1.0, -0.0, 0.0], np.float32),
        np.array([5.0], np.float32),
        np.arange(50, dtype=np.float32)[::-1].copy(),
        np.arange(50, dtype=np.float32),
        np.full(37, 2.5, np.float32),
        r.integers(-5, 5, 4000).astype(np.float32),
        r.uniform(-1e30, 1e30, 3000).astype(np.float32),
        np.concatenate([r.standard_normal(2000).astype(np.float32), -np.zeros(10, np.float32), np.zeros(10, np.float32)]),
        r.uniform(0, 2**27, 5000).astype(np.float32),
    ]
    for a in cases:
        p = oracle.stable_argsort(a, lib=lib)
        n = a.size
        assert p.dtype == np.uint32 and p.size == n
        assert np.array_equal(np.sort(p), np.arange(n, dtype=np.uint32)), "not a permutation"
        s = a[p].astype(np.float64)
        assert np.all(s[1:] >= s[:-1]), "not ascending"
        ties = s[1:] == s[:-1]
        assert np.all(p[1:][ties] > p[:-1][ties]), "ties not in input order"
        assert np.array_equal(p, np.argsort(a, kind="stable").astype(np.uint32)), "differs from numpy stable argsort"
    p = oracle.stable_argsort(np.array([0.0, -0.0, 1.0, -0.0, 0.0], np.float32), lib=lib)
    assert p.tolist() == [0, 1, 3, 4, 2]


def pin_sort_rejects_nonfinite(lib):
    for bad in (np.nan, np.inf, -np.inf):
        a = np.array([1.0, bad, 0.0], np.float32)
        try:
            oracle.stable_argsort(a, lib=lib)
        except ValueError:
            continue
        raise AssertionError("non-finite anchor accepted")


# ----------------------------------------------------------------------------- hand examples

def _golden_cases():
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        return json.load(f)["cases"]


def pin_hand_examples(lib):
    """Small cases worked out by hand from the operator's definition."""
    for case in _golden_cases():
        a = np.array(case["a"], np.float32)
        x = np.array(case["x"], np.float32)
        want = np.array([sum(c * math.exp(-d) for c, d in row) for row in case["y_terms"]])
        if "b" in case:
            b = np.array(case["b"], np.float32)
            got_scan = oracle.general_apply(a, b, x, lib=lib)[:, 0]
            got_dense = odense.dense_apply(a, x, b=b)[:, 0]
        else:
            got_scan = oracle.sym_apply(a, x, lib=lib)[:, 0]
            got_dense = odense.dense_apply(a, x)[:, 0]
        _close(got_scan, want, 1e-15, "scan " + case["name"])
        _close(got_dense, want, 1e-15, "dense " + case["name"])


# ----------------------------------------------------------------------------- closed forms

def _kms_inverse_apply(h, z):
    """K^{-1} z for K_ij = rho^{|i-j|}, rho = e^{-h}: (1-rho^2)^{-1} times the
    tridiagonal matrix with diagonal (1, 1+rho^2, ..., 1+rho^2, 1) and
    off-diagonals -rho (Kac-Murdock-Szego)."""
    rho = math.exp(-h)
    n = z.shape[0]
    w = np.empty_like(z)
    diag = np.full(n, 1.0 + rho * rho)
    diag[0] = diag[-1] = 1.0
    if n == 1:
        diag[0] = 1.0 - rho * rho
    w[:] = diag[:, None] * z
    if n > 1:
        w[:-1] -= rho * z[1:]
        w[1:] -= rho * z[:-1]
    return w / (1.0 - rho * rho)


def pin_kms_inverse(lib):
    """Equispaced anchors a_i = i h: K is the Kac-Murdock-Szego matrix; its
    closed-form tridiagonal inverse must undo the oracle's K x."""
    r = _rng(2)
    for h in (0.125, 1.0, 4.0):
        for n, m in ((2, 1), (64, 1), (500, 3)):
            a = (np.arange(n) * h).astype(np.float32)
            x = r.standard_normal((n, m)).astype(np.float32)
            for name, z in (("scan", oracle.sym_apply(a, x, lib=lib)), ("dense", odense.dense_apply(a, x))):
                back = _kms_inverse_apply(h, z)
                _close(back, x, 1e-11, "KMS %s h=%g n=%d" % (name, h, n))


def _markov_precision_apply(t, z):
    """Q z where Q = K^{-1} for K_ij = exp(-|t_i - t_j|), t sorted distinct:
    with rho_i = exp(-(t_{i+1} - t_i)),
      Q_11 = 1/(1-rho_1^2), Q_nn = 1/(1-rho_{n-1}^2),
      Q_ii = 1/(1-rho_{i-1}^2) + rho_i^2/(1-rho_i^2),
      Q_{i,i+1} = Q_{i+1,i} = -rho_i/(1-rho_i^2)
    (precision of a stationary Ornstein-Uhlenbeck process sampled at t)."""
    t = np.asarray(t, np.float64)
    rho = np.exp(-(t[1:] - t[:-1]))
    g = 1.0 / (1.0 - rho * rho)
    # Q_ii = [i>0] g_{i-1} + [i<n-1] rho_i^2 g_i + [i=0]  (uses g = 1 + rho^2 g)
    diag = np.zeros(t.size)
    diag[1:] += g
    diag[:-1] += rho * rho * g
    diag[0] += 1.0
    off = -rho * g
    w = diag[:, None] * z
    w[:-1] += off[:, None] * z[1:]
    w[1:] += off[:, None] * z[:-1]
    return w


def pin_markov_tridiagonal(lib):
    """Arbitrary distinct anchors (given in shuffled order): the precision
    matrix of the exponential covariance is tridiagonal in sorted order."""
    r = _rng(3)
    for n, m in ((3, 1), (200, 2), (1500, 1)):
        t = np.cumsum(r.uniform(0.05, 2.0, n)).astype(np.float32)
        order = r.permutation(n)
        a = t[order]
        x = r.standard_normal((n, m)).astype(np.float32)
        srt = np.argsort(a, kind="stable")
        for name, z in (("scan", oracle.sym_apply(a, x, lib=lib)), ("dense", odense.dense_apply(a, x))):
            back = _markov_precision_apply(a[srt], z[srt])
            _close(back, x[srt], 1e-9, "Markov %s n=%d" % (name, n))


def pin_toeplitz_fft(lib):
    """Anchors on uniform grids: K is Toeplitz, so K x is a convolution and a
    circulant embedding with numpy.fft computes it independently.  With a grid
    offset s between a and b the kernel is not symmetric in i - j, which also
    fixes the orientation of the general operator."""
    r = _rng(4)
    for h, n, k, s, m in ((0.5, 300, 300, 0.0, 2), (0.25, 257, 100, 0.375, 1), (1.0, 90, 211, -2.5, 3)):
        a = (np.arange(n) * h).astype(np.float32)
        b = (np.arange(k) * h + s).astype(np.float32)
        x = r.standard_normal((k, m)).astype(np.float32)
        # c_d = exp(-|h d - s|) for d = i - j in [-(k-1), n-1]
        L = 1 << int(math.ceil(math.log2(n + k)))
        d = np.arange(L)
        dd = np.where(d < n, d, d - L)  # lags n..L-1 wrap to negative
        c = np.exp(-np.abs(h * dd - s))
        c[(dd >= n) | (dd <= -k)] = 0.0
        xp = np.zeros((L, m))
        xp[:k] = x
        want = np.real(np.fft.ifft(np.fft.fft(c)[:, None] * np.fft.fft(xp, axis=0), axis=0))[:n]
        if s == 0.0 and n == k:
            _close(oracle.sym_apply(a, x, lib=lib), want, 1e-12, "toeplitz sym scan")
            _close(odense.dense_apply(a, x), want, 1e-12, "toeplitz sym dense")
        _close(oracle.general_apply(a, b, x, lib=lib), want, 1e-12, "toeplitz general scan")
        _close(odense.dense_apply(a, x, b=b), want, 1e-12, "toeplitz general dense")


def pin_geometric_row_sums(lib):
    """(K 1)_i on the grid i h: two geometric series minus the diagonal."""
    for h, n in ((0.125, 400), (2.0, 33)):
        a = (np.arange(n) * h).astype(np.float32)
        rho = math.exp(-h)
        i = np.arange(n)
        want = (1 - rho ** (i + 1)) / (1 - rho) + (1 - rho ** (n - i)) / (1 - rho) - 1
        ones = np.ones(n, np.float32)
        _close(oracle.sym_apply(a, ones, lib=lib)[:, 0], want, 1e-12, "row sums scan")
        _close(odense.dense_apply(a, ones)[:, 0], want, 1e-12, "row sums dense")


# ----------------------------------------------------------------------------- invariants

def pin_columns(lib):
    """K e_j is column j, exp(-|a_i - a_j|); tie partners of j get exactly 1."""
    r = _rng(5)
    n = 300
    a = r.integers(0, 120, n).astype(np.float32) * np.float32(0.5)
    for j in (0, 17, 150, n - 1):
        e = np.zeros(n, np.float32)
        e[j] = 1.0
        col = np.exp(-np.abs(a.astype(np.float64) - float(a[j])))
        y = oracle.sym_apply(a, e, lib=lib)[:, 0]
        _close(y, col, 1e-13, "K e_j scan")
        assert np.all(y[a == a[j]] == 1.0), "tie partner not exactly 1"
        _close(odense.dense_apply(a, e)[:, 0], col, 1e-15, "K e_j dense")
    b = r.uniform(0, 60, 77).astype(np.float32)
    for j in (0, 40, 76):
        e = np.zeros(b.size, np.float32)
        e[j] = 1.0
        col = np.exp(-np.abs(a.astype(np.float64) - float(b[j])))
        _close(oracle.general_apply(a, b, e, lib=lib)[:, 0], col, 1e-13, "K_ab e_j scan")


def pin_symmetry_adjoint(lib):
    """<u, K v> = <K u, v> (symmetric operator) and <u, K_ab v> = <K_ba u, v>;
    the phased operator is adjoint to the one with (a, phi) and (b, psi) swapped."""
    r = _rng(6)
    n, k = 400, 150
    a = r.uniform(0, 80, n).astype(np.float32)
    b = r.uniform(-5, 85, k).astype(np.float32)
    u = r.standard_normal(n).astype(np.float32)
    v = r.standard_normal(n).astype(np.float32)
    lhs = float(u @ oracle.sym_apply(a, v, lib=lib)[:, 0])
    rhs = float(oracle.sym_apply(a, u, lib=lib)[:, 0] @ v)
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs)), "sym not symmetric"
    w = r.standard_normal(k).astype(np.float32)
    lhs = float(u @ oracle.general_apply(a, b, w, lib=lib)[:, 0])
    rhs = float(oracle.general_apply(b, a, u, lib=lib)[:, 0] @ w)
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs)), "general not adjoint"
    phi = r.uniform(0, 6.3, n).astype(np.float32)
    psi = r.uniform(0, 6.3, k).astype(np.float32)
    lhs = float(u @ oracle.phased_apply(a, phi, w, b=b, psi=psi, lib=lib)[:, 0])
    rhs = float(oracle.phased_apply(b, psi, u, b=a, psi=phi, lib=lib)[:, 0] @ w)
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs)), "phased not adjoint"
    lhs = float(u @ oracle.phased_apply(a, phi, v, lib=lib)[:, 0])
    rhs = float(oracle.phased_apply(a, phi, u, lib=lib)[:, 0] @ v)
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs)), "phased sym not symmetric"
    for q in (u, v):
        assert float(q @ odense.dense_apply(a, q)[:, 0]) > 0, "Laplace kernel not positive definite"


def pin_zero_temperature(lib):
    """Anchors 200 apart: off-diagonal weights are below e^-200, so K is a
    permutation (distinct positions) or a bucket-sum/CountSketch matrix
    (shared positions), to well below float64 resolution."""
    r = _rng(7)
    n = 1000
    pi = r.permutation(n)
    a = (200.0 * pi).astype(np.float32)
    b = (200.0 * np.arange(n)).astype(np.float32)
    x = r.standard_normal((n, 2)).astype(np.float32)
    y = oracle.general_apply(a, b, x, lib=lib)
    assert np.array_equal(y, x[pi].astype(np.float64)), "general: not a permutation"
    assert np.array_equal(odense.dense_apply(a, x, b=b), x[pi].astype(np.float64)), "dense: not a permutation"
    h = r.integers(0, 37, n)
    a2 = (200.0 * h).astype(np.float32)
    sums = np.zeros((37, 2))
    np.add.at(sums, h, x.astype(np.float64))
    _close(oracle.sym_apply(a2, x, lib=lib), sums[h], 1e-13, "CountSketch scan")
    _close(odense.dense_apply(a2, x), sums[h], 1e-13, "CountSketch dense")
    ys = oracle.sym_apply(a, x, lib=lib)
    assert np.array_equal(ys, x.astype(np.float64)), "sym at zero temperature is not the identity"


def pin_special_cases(lib):
    r = _rng(8)
    x1 = np.array([[3.25, -1.5]], np.float32)
    assert np.array_equal(oracle.sym_apply(np.array([7.0], np.float32), x1, lib=lib), x1.astype(np.float64)), "n=1"
    n = 129
    x = r.standard_normal((n, 3)).astype(np.float32)
    a = np.full(n, -3.5, np.float32)
    _close(oracle.sym_apply(a, x, lib=lib), np.repeat(x.astype(np.float64).sum(0, keepdims=True), n, 0), 1e-13, "all equal")
    # shift by an exactly representable integer on an integer grid
    a = r.integers(0, 200, 500).astype(np.float32)
    xs = r.standard_normal(500).astype(np.float32)
    y0 = oracle.sym_apply(a, xs, lib=lib)
    y1 = oracle.sym_apply(a + np.float32(1024.0), xs, lib=lib)
    _close(y1, y0, 1e-13, "shift invariance")
    assert np.array_equal(oracle.stable_argsort(a, lib=lib), oracle.stable_argsort(a + np.float32(1024.0), lib=lib))
    # linearity (dyadic values, so 2 u - v / 2 is exact in float32)
    u = (r.integers(-400, 400, 500) / 4.0).astype(np.float32)
    v = (r.integers(-400, 400, 500) / 4.0).astype(np.float32)
    lhs = oracle.sym_apply(a, (2.0 * u - 0.5 * v).astype(np.float32), lib=lib)
    rhs = 2.0 * oracle.sym_apply(a, u, lib=lib) - 0.5 * oracle.sym_apply(a, v, lib=lib)
    _close(lhs, rhs, 1e-12, "linearity")
    # k = 0 input anchors: empty sum
    assert np.array_equal(oracle.general_apply(a[:5], np.zeros(0, np.float32), np.zeros((0, 2), np.float32), lib=lib),
                          np.zeros((5, 2)))


def pin_general_reductions(lib):
    """b = a gives the symmetric operator; b a subset of a gives the symmetric
    operator on x scattered into the subset (zeros elsewhere)."""
    r = _rng(9)
    n = 600
    a = r.uniform(0, 100, n).astype(np.float32)
    a[::7] = a[3]
    x = r.standard_normal((n, 2)).astype(np.float32)
    _close(oracle.general_apply(a, a, x, lib=lib), oracle.sym_apply(a, x, lib=lib), 1e-12, "general(b=a)")
    sub = r.choice(n, 211, replace=False)
    xt = np.zeros_like(x)
    xt[sub] = x[sub]
    _close(oracle.general_apply(a, a[sub], x[sub], lib=lib), oracle.sym_apply(a, xt, lib=lib), 1e-12, "general subset")


def pin_phased(lib):
    """Phased operator: constant phases give the unphased operator; adding one
    constant to all phases changes nothing; and cos(phi - psi) = cos phi cos psi
    + sin phi sin psi (angle-difference identity) expresses it through the
    unphased dense operator."""
    r = _rng(10)
    n, k, m = 350, 120, 2
    a = r.uniform(0, 60, n).astype(np.float32)
    a[::9] = a[1]
    b = r.uniform(-3, 63, k).astype(np.float32)
    x = r.standard_normal((n, m)).astype(np.float32)
    xb = r.standard_normal((k, m)).astype(np.float32)
    c = np.full(n, 1.25, np.float32)
    _close(oracle.phased_apply(a, c, x, lib=lib), oracle.sym_apply(a, x, lib=lib), 1e-12, "constant phase sym")
    _close(oracle.phased_apply(a, c, xb, b=b, psi=np.full(k, 1.25, np.float32), lib=lib),
           oracle.general_apply(a, b, xb, lib=lib), 1e-12, "constant phase general")
    phi = r.uniform(0, 6.283, n).astype(np.float32)
    psi = r.uniform(0, 6.283, k).astype(np.float32)
    for (bb, pp, xx) in ((None, None, x), (b, psi, xb)):
        f64 = np.float64
        ph = phi.astype(f64)
        ps = (phi if pp is None else pp).astype(f64)
        xd = xx.astype(f64)
        ident = (np.cos(ph)[:, None] * odense.dense_apply(a, np.cos(ps)[:, None] * xd, b=bb)
                 + np.sin(ph)[:, None] * odense.dense_apply(a, np.sin(ps)[:, None] * xd, b=bb))
        dense = odense.dense_apply(a, xx, b=bb, phi=phi, psi=pp)
        _close(dense, ident, 1e-12, "phased dense vs angle-difference identity")
        scan = oracle.phased_apply(a, phi, xx, b=bb, psi=pp, lib=lib)
        _close(scan, dense, 1e-12, "phased scan vs dense")
    # phase shift: phi + 1, psi + 1 (rounded in float32, so compare against dense)
    sh = oracle.phased_apply(a, (phi + np.float32(1.0)).astype(np.float32), x, lib=lib)
    _close(sh, odense.dense_apply(a, x, phi=(phi + np.float32(1.0)).astype(np.float32)), 1e-12, "phase shift")


def pin_brute_force_tiny(lib):
    """Scan oracle against the dense definition on tiny adversarial inputs."""
    r = _rng(11)
    anchor_sets = [
        np.array([0.0], np.float32),
        np.array([1.0, 1.0], np.float32),
        np.array([0.0, -0.0, 0.0, 1e-30, -1e-30], np.float32),
        np.arange(16, dtype=np.float32)[::-1].copy(),
        np.array([-1e4, 0.0, 1e4, 5.0, 5.0, 5.0], np.float32),
        r.uniform(0, 3, 40).astype(np.float32),
        np.round(r.uniform(0, 6, 64)).astype(np.float32),
        r.standard_normal(97).astype(np.float32) * np.float32(20.0),
    ]
    for a in anchor_sets:
        n = a.size
        for m in (1, 3):
            x = r.standard_normal((n, m)).astype(np.float32)
            env = odense.dense_envelope(a, x)
            assert oracle.normwise_error(oracle.sym_apply(a, x, lib=lib), odense.dense_apply(a, x), env) < 1e-13, "sym"
            phi = r.uniform(0, 6.3, n).astype(np.float32)
            assert oracle.normwise_error(oracle.phased_apply(a, phi, x, lib=lib), odense.dense_apply(a, x, phi=phi), env) < 1e-13, "phased"
            for k in (1, 2, 9, 31):
                b = np.concatenate([a[: min(n, 2)], r.uniform(float(a.min()) - 2, float(a.max()) + 2, k)]).astype(np.float32)[:k]
                xb = r.standard_normal((k, m)).astype(np.float32)
                envb = odense.dense_envelope(a, xb, b=b)
                assert oracle.normwise_error(oracle.general_apply(a, b, xb, lib=lib), odense.dense_apply(a, xb, b=b), envb) < 1e-13, "general"
                psi = r.uniform(0, 6.3, k).astype(np.float32)
                assert oracle.normwise_error(oracle.phased_apply(a, phi, xb, b=b, psi=psi, lib=lib),
                                             odense.dense_apply(a, xb, b=b, phi=phi, psi=psi), envb) < 1e-13, "phased general"


def pin_dense_rows_c(lib):
    """C spot rows (plain definition, one pass) against the NumPy dense
    oracle and the scan oracle, on anchors spread wider than the 746 cut-off."""
    r = _rng(12)
    n, k, m = 3000, 2500, 2
    a = r.uniform(-2000, 2000, n).astype(np.float32)
    a[:50] = a[50]
    b = r.uniform(-2100, 2100, k).astype(np.float32)
    b[:20] = a[60]
    x = r.standard_normal((n, m)).astype(np.float32)
    xb = r.standard_normal((k, m)).astype(np.float32)
    phi = r.uniform(0, 6.3, n).astype(np.float32)
    psi = r.uniform(0, 6.3, k).astype(np.float32)
    rows = np.array([0, 1, 50, 60, 1234, n - 1])
    y, env = oracle.dense_rows_c(rows, a, x, lib=lib)
    _close(y, oracle.sym_apply(a, x, lib=lib)[rows], 1e-12, "C rows vs sym scan")
    _close(env, odense.dense_envelope(a, x)[rows], 1e-12, "C rows envelope")
    y, env = oracle.dense_rows_c(rows, a, xb, b=b, lib=lib)
    _close(y, oracle.general_apply(a, b, xb, lib=lib)[rows], 1e-12, "C rows vs general scan")
    _close(y, odense.dense_apply(a, xb, b=b)[rows], 1e-12, "C rows vs dense general")
    y, env = oracle.dense_rows_c(rows, a, xb, b=b, phi=phi, psi=psi, lib=lib)
    _close(y, odense.dense_apply(a, xb, b=b, phi=phi, psi=psi)[rows], 1e-12, "C rows phased general")
    y, env = oracle.dense_rows_c(rows, a, x, phi=phi, lib=lib)
    _close(y, oracle.phased_apply(a, phi, x, lib=lib)[rows], 1e-12, "C rows phased sym")


# ----------------------------------------------------------------------------- backward
# The operator is differentiable in its anchors (section 2.3); the backward
# formulas are the chain rule on the plain definition.  Pinned by central
# differences of the dense forward product (itself pinned above): f(a, x) =
# sum(g * K(a) x) has df/dx = K^T g exactly (f is linear in x) and df/da by
# central differences, which at a tie (|t| has a kink) give the sign(0) = 0
# value the oracle uses.

def _fd_anchor_grad(f, a, h):
    a = np.asarray(a, np.float64)
    out = np.empty(a.size)
    for k in range(a.size):
        ap, am = a.copy(), a.copy()
        ap[k] += h
        am[k] -= h
        out[k] = (f(ap) - f(am)) / (2.0 * h)
    return out


def _spread_anchors(r, n, gap):
    """Distinct anchors at least `gap` apart (in random order)."""
    return r.permutation(np.cumsum(r.uniform(gap, 4.0 * gap, n))).astype(np.float32)


def pin_backward_finite_differences(lib):
    r = _rng(61)
    h = 1e-5
    for ties in (False, True):
        n, m = 26, 2
        a = (r.integers(0, 9, n).astype(np.float32) if ties else _spread_anchors(r, n, 0.05))
        x = r.standard_normal((n, m)).astype(np.float32)
        g = r.standard_normal((n, m)).astype(np.float32)
        x64, g64 = x.astype(np.float64), g.astype(np.float64)
        fd_da = _fd_anchor_grad(lambda aa: float(np.sum(g64 * odense.dense_apply(aa, x64))), a, h)
        dx, da = oracle.sym_backward(a, x, g, lib=lib)
        _close(da, fd_da, 1e-7, "sym da vs central differences (ties=%s)" % ties)
        _close(dx, odense.dense_apply(a, g64).reshape(n, m), 1e-12, "sym dx vs K g (ties=%s)" % ties)
        dxd, dad = odense.dense_backward(a, x, g)
        _close(dad, fd_da, 1e-7, "dense sym da vs central differences")
        # df/dx_j = (K^T g)_j: the product is linear in x, so one difference each is exact up to rounding
        j, c = 3, 1
        xp, xm = x64.copy(), x64.copy()
        xp[j, c] += 0.5
        xm[j, c] -= 0.5
        fdx = float(np.sum(g64 * odense.dense_apply(a, xp))) - float(np.sum(g64 * odense.dense_apply(a, xm)))
        _close([dx[j, c]], [fdx], 1e-10, "sym dx vs difference in x")
        # general: K is n x k over rows a and columns b (shared grid: a/b ties)
        k = 19
        b = (r.integers(0, 9, k).astype(np.float32) if ties else _spread_anchors(r, k, 0.05) + np.float32(0.013))
        xb = r.standard_normal((k, m)).astype(np.float32)
        xb64 = xb.astype(np.float64)
        fd_da = _fd_anchor_grad(lambda aa: float(np.sum(g64 * odense.dense_apply(aa, xb64, b=b))), a, h)
        fd_db = _fd_anchor_grad(lambda bb: float(np.sum(g64 * odense.dense_apply(a, xb64, b=bb))), b, h)
        dxg, dag, dbg = oracle.general_backward(a, b, xb, g, lib=lib)
        _close(dag, fd_da, 1e-7, "general da vs central differences (ties=%s)" % ties)
        _close(dbg, fd_db, 1e-7, "general db vs central differences (ties=%s)" % ties)
        _close(dxg, odense.dense_apply(b, g64, b=a).reshape(k, m), 1e-12, "general dx vs K^T g")
        _, dad2, dbd2 = odense.dense_backward(a, xb, g, b=b)
        _close(dad2, fd_da, 1e-7, "dense general da vs central differences")
        _close(dbd2, fd_db, 1e-7, "dense general db vs central differences")


def pin_backward_brute_force(lib):
    """The scan-and-search backward against the dense definition at sizes the
    difference pin does not reach (several hundred anchors, ties, m = 3)."""
    r = _rng(62)
    for ties in (False, True):
        n, k, m = 700, 450, 3
        a = r.uniform(0, 90, n).astype(np.float32)
        b = r.uniform(0, 90, k).astype(np.float32)
        if ties:
            a, b = np.round(a), np.round(b)
        x = r.standard_normal((n, m)).astype(np.float32)
        xb = r.standard_normal((k, m)).astype(np.float32)
        g = r.standard_normal((n, m)).astype(np.float32)
        dx, da = oracle.sym_backward(a, x, g, lib=lib)
        dxd, dad = odense.dense_backward(a, x, g)
        _close(dx, dxd, 1e-12, "sym dx brute force")
        _close(da, dad, 1e-12, "sym da brute force")
        rows = np.array([0, 1, 77, n // 2, n - 1], np.int64)
        dar, envr = oracle.backward_rows(rows, a, x, g, lib=lib)
        _close(dar, dad[rows], 1e-12, "sym da at rows vs brute force")
        envd = (np.abs(g) * odense.dense_apply(a, np.abs(x)) + np.abs(x) * odense.dense_apply(a, np.abs(g))).sum(1)
        _close(envr, envd[rows], 1e-12, "sym da envelope at rows")
        dx, da, db = oracle.general_backward(a, b, xb, g, lib=lib)
        dxd, dad, dbd = odense.dense_backward(a, xb, g, b=b)
        _close(dx, dxd, 1e-12, "general dx brute force")
        _close(da, dad, 1e-12, "general da brute force")
        _close(db, dbd, 1e-12, "general db brute force")


# ----------------------------------------------------------------------------- weighted Gram
def _gram_golden_cases():
    with open(os.path.join(GOLDEN, "gram_examples.json")) as f:
        return json.load(f)["cases"]


def pin_gram_hand_examples(lib):
    """Weighted Gram matrices worked out by hand from M = A diag(D) A^T."""
    for case in _gram_golden_cases():
        a = np.array(case["a"], np.float32)
        b = np.array(case["b"], np.float32)
        D = np.array(case["D"], np.float32)
        want = np.array([[sum(c * math.exp(-d) for c, d in ent) for ent in row] for row in case["m_terms"]])
        _close(odense.gram_dense(a, b, D), want, 1e-15, "gram " + case["name"])


def pin_gram_scan_products(lib):
    """M v = A (D * (A^T v)), with A and A^T applied by the scan oracle (a
    different computation: sort, interval sums, recurrences), for weights of
    both signs, ties between a and b, and a block of rows and columns."""
    r = _rng(70)
    for ties in (False, True):
        n, k = 300, 500
        a = r.uniform(0, 60, n).astype(np.float32)
        b = r.uniform(0, 60, k).astype(np.float32)
        if ties:
            a, b = np.round(a), np.round(b)
        D = r.standard_normal(k).astype(np.float32)
        v = r.standard_normal((n, 2))
        M = odense.gram_dense(a, b, D)
        atv = oracle.general_apply(b, a, v.astype(np.float32), lib=lib)
        want = oracle.general_apply(a, b, (D[:, None] * atv).astype(np.float64).astype(np.float32), lib=lib)
        # the fp32 round trip of D * A^T v above is the only rounding: compare at its scale
        env = oracle.general_apply(a, b, np.abs(D[:, None] * atv).astype(np.float32), lib=lib)
        err = float(np.max(np.abs(M @ v.astype(np.float32).astype(np.float64) - want)) / np.max(env))
        assert err <= 1e-6, "gram M v vs A D A^T v (ties=%s): %.3e" % (ties, err)
        rows, cols = np.array([0, 7, 299]), np.array([3, 0, 150, 298])
        _close(odense.gram_block(rows, cols, a, b, D), M[np.ix_(rows, cols)], 1e-14, "gram block")


def pin_gram_kms(lib):
    """a = b = equispaced (spacing h), D = 1: M = K^2 with K the Kac-Murdock-
    Szego matrix, so its closed-form tridiagonal inverse applied twice gives I."""
    for h in (0.25, 1.0):
        n = 200
        a = (np.arange(n) * h).astype(np.float32)
        M = odense.gram_dense(a, a, np.ones(n, np.float32))
        back = _kms_inverse_apply(h, _kms_inverse_apply(h, M))
        _close(back, np.eye(n), 1e-9, "gram KMS h=%g" % h)


def pin_gram_continuum(lib):
    """Input anchors on a fine grid over [-L, L] with trapezoid weights: M_pq
    tends to the integral of exp(-|a_p - t| - |a_q - t|) dt over the line,
    which is (1 + |a_p - a_q|) exp(-|a_p - a_q|)."""
    h, L = 2.0 ** -8, 24.0
    t = np.arange(-L, L + h / 2, h).astype(np.float32)
    w = np.full(t.size, h, np.float32)
    w[0] = w[-1] = h / 2
    r = _rng(71)
    a = (np.round(r.uniform(-4, 4, 40) / h) * h).astype(np.float32)  # on grid nodes: kinks fall on nodes
    M = odense.gram_dense(a, t, w)
    d = np.abs(a[:, None].astype(np.float64) - a[None, :])
    _close(M, (1.0 + d) * np.exp(-d), 1e-5, "gram continuum limit")


def pin_gram_symmetric_psd(lib):
    """Nonnegative weights: M is symmetric positive semidefinite (a Gram
    matrix); with some weights negative it stays symmetric."""
    r = _rng(72)
    a = r.uniform(0, 30, 150).astype(np.float32)
    b = r.uniform(0, 30, 90).astype(np.float32)
    M = odense.gram_dense(a, b, r.uniform(0, 2, 90).astype(np.float32))
    _close(M, M.T, 1e-15, "gram symmetry")
    ev = np.linalg.eigvalsh((M + M.T) / 2)
    assert ev.min() >= -1e-12 * ev.max(), "gram not PSD: %.3e" % ev.min()
    # rank at most k
    k = 20
    b2 = r.uniform(0, 30, k).astype(np.float32)
    M2 = odense.gram_dense(a, b2, r.uniform(0.5, 2, k).astype(np.float32))
    sv = np.linalg.svd(M2, compute_uv=False)
    assert sv[k] <= 1e-12 * sv[0], "gram rank exceeds k"


def pin_phased_backward(lib):
    """Phased backward (anchors and phases are parameters too): the plain
    definition against central differences of <g, W x> in every anchor and
    every phase, symmetric and general, with and without ties; phases all
    zero reduce it to the scan oracle's symmetric backward (and give no phase
    gradient); a common phase shift changes nothing; the spot-row form agrees
    with the whole."""
    r = _rng(63)
    h = 1e-5
    for ties in (False, True):
        n, m = 24, 2
        a = (r.integers(0, 9, n).astype(np.float32) if ties else _spread_anchors(r, n, 0.05))
        phi = r.uniform(0, 2 * np.pi, n)
        x = r.standard_normal((n, m)).astype(np.float32)
        g = r.standard_normal((n, m)).astype(np.float32)
        x64, g64 = x.astype(np.float64), g.astype(np.float64)
        loss = lambda aa, pp: float(np.sum(g64 * odense.dense_apply(aa, x64, phi=pp)))
        dx, da, dphi = odense.dense_phased_backward(a, phi, x, g)
        _close(da, _fd_anchor_grad(lambda aa: loss(aa, phi), a, h), 1e-7, "phased sym da vs differences (ties=%s)" % ties)
        _close(dphi, _fd_anchor_grad(lambda pp: loss(a, pp), phi, h), 1e-7, "phased sym dphi vs differences")
        _close(dx, odense.dense_apply(a, g64, phi=phi).reshape(n, m), 1e-12, "phased sym dx vs W g")
        j, c = 5, 0
        xp, xm = x64.copy(), x64.copy()
        xp[j, c] += 0.5
        xm[j, c] -= 0.5
        fdx = float(np.sum(g64 * odense.dense_apply(a, xp, phi=phi))) - float(np.sum(g64 * odense.dense_apply(a, xm, phi=phi)))
        _close([dx[j, c]], [fdx], 1e-10, "phased sym dx vs difference in x")
        # general: rows (a, phi), columns (b, psi)
        k = 17
        b = (r.integers(0, 9, k).astype(np.float32) if ties else _spread_anchors(r, k, 0.05) + np.float32(0.013))
        psi = r.uniform(0, 2 * np.pi, k)
        xb = r.standard_normal((k, m)).astype(np.float32)
        xb64 = xb.astype(np.float64)
        gl = lambda aa, pp, bb, qq: float(np.sum(g64 * odense.dense_apply(aa, xb64, b=bb, phi=pp, psi=qq)))
        dxg, dag, dbg, dpg, dqg = odense.dense_phased_backward(a, phi, xb, g, b=b, psi=psi)
        _close(dag, _fd_anchor_grad(lambda aa: gl(aa, phi, b, psi), a, h), 1e-7, "phased general da vs differences")
        _close(dbg, _fd_anchor_grad(lambda bb: gl(a, phi, bb, psi), b, h), 1e-7, "phased general db vs differences")
        _close(dpg, _fd_anchor_grad(lambda pp: gl(a, pp, b, psi), phi, h), 1e-7, "phased general dphi vs differences")
        _close(dqg, _fd_anchor_grad(lambda qq: gl(a, phi, b, qq), psi, h), 1e-7, "phased general dpsi vs differences")
        _close(dxg, odense.dense_apply(b, g64, b=a, phi=psi, psi=phi).reshape(k, m), 1e-12, "phased general dx vs W^T g")
    # zero phases: the symmetric backward of the scan oracle, and no phase gradient
    n, m = 300, 3
    a = r.uniform(0, 40, n).astype(np.float32)
    x = r.standard_normal((n, m)).astype(np.float32)
    g = r.standard_normal((n, m)).astype(np.float32)
    dx0, da0, dp0 = odense.dense_phased_backward(a, np.zeros(n), x, g)
    dxs, das = oracle.sym_backward(a, x, g, lib=lib)
    _close(da0, das, 1e-12, "phased backward at zero phase vs symmetric backward")
    _close(dx0, dxs, 1e-12, "phased dx at zero phase vs K g")
    assert np.all(dp0 == 0.0), "phase gradient at zero phase"
    # a common shift of every phase leaves W, hence every gradient, unchanged
    phi = r.uniform(0, 2 * np.pi, n)
    r1 = odense.dense_phased_backward(a, phi, x, g)
    r2 = odense.dense_phased_backward(a, phi + 0.7, x, g)
    for u, v, nm in zip(r1, r2, ("dx", "da", "dphi")):
        _close(u, v, 1e-12, "phased backward under a common phase shift: " + nm)
    rows = np.array([0, 7, 150, n - 1])
    dar, dpr, env = odense.phased_backward_rows(rows, a, phi, x, g)
    _close(dar, r1[1][rows], 1e-12, "phased da at rows vs whole")
    _close(dpr, r1[2][rows], 1e-12, "phased dphi at rows vs whole")
    assert np.all(env >= np.abs(dar)) and np.all(env >= np.abs(dpr))


# ----------------------------------------------------------------------------- error measure

def _normwise_cases():
    with open(os.path.join(GOLDEN, "normwise_examples.json")) as f:
        return json.load(f)["cases"]


def pin_normwise_error(lib):
    """The parity tests' error measure against hand-computed values: per-column
    denominators, explicit denominators, zero envelopes, the worst row, vectors,
    and the envelope K0|x| of a two-anchor operator; shape mismatches raise."""
    for case in _normwise_cases():
        if "a" in case:
            a = np.array(case["a"], np.float32)
            x = np.array(case["x"], np.float32)
            env = odense.dense_envelope(a, x)
            env_hand = np.array([[sum(c * math.exp(-d) for c, d in col) for col in row] for row in case["env_terms"]])
            _close(env, env_hand, 1e-15, "envelope " + case["name"])
            y_ref = odense.dense_apply(a, x)
            y = y_ref + np.array(case["delta"])
            want = case["want_num"] / sum(c * math.exp(-d) for c, d in case["want_den_terms"])
            got = odense.normwise_error(y, y_ref, env)
        else:
            scale = np.array(case["env_scale"]) if "env_scale" in case else None
            got = odense.normwise_error(np.array(case["y"]), np.array(case["y_ref"]), np.array(case["env"]),
                                        env_scale=scale)
            want = case["want"]
        assert abs(got - want) <= 1e-15 * max(1.0, abs(want)), "%s: %r, expected %r" % (case["name"], got, want)
    for y, y_ref in ((np.zeros((3, 2)), np.zeros((2, 3))), (np.zeros(4), np.zeros(3)), (np.zeros((4, 2)), np.zeros(8))):
        try:
            odense.normwise_error(y, y_ref, np.ones_like(y_ref))
        except ValueError:
            continue
        raise AssertionError("shape mismatch %s vs %s accepted" % (y.shape, y_ref.shape))


ALL_PINS = [
    pin_normwise_error,
    pin_sort_definition,
    pin_sort_rejects_nonfinite,
    pin_hand_examples,
    pin_kms_inverse,
    pin_markov_tridiagonal,
    pin_toeplitz_fft,
    pin_geometric_row_sums,
    pin_columns,
    pin_symmetry_adjoint,
    pin_zero_temperature,
    pin_special_cases,
    pin_general_reductions,
    pin_phased,
    pin_brute_force_tiny,
    pin_dense_rows_c,
    pin_backward_finite_differences,
    pin_backward_brute_force,
    pin_gram_hand_examples,
    pin_gram_scan_products,
    pin_gram_kms,
    pin_gram_continuum,
    pin_gram_symmetric_psd,
    pin_phased_backward,
]

"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a temporary copy of the C oracle (or patches
the dense brute force's weight function), rebuilds it on the CPU, and checks
that at least one pin of oracle_pins.py then fails.  The oracle itself is not
modified.
"""
import os
import shutil

import numpy as np
import pytest

import oracle
from oracle import dense as odense
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "laplex_oracle.c")

# (name, original text, replacement, which occurrence)
C_MUTANTS = [
    ("merge_unstable", "if (src[q].v < src[p].v)", "if (src[q].v <= src[p].v)", 0),
    ("insertion_unstable", "while (j >= lo && buf0[j].v > t.v)", "while (j >= lo && buf0[j].v >= t.v)", 0),
    ("nonfinite_accepted", "if (!isfinite(a[i])) return -1;", "if (0) return -1;", 0),
    ("sym_prefix_decay_sign", "double d = exp(as[i - 1] - as[i]);", "double d = exp(as[i] - as[i - 1]);", 0),
    ("sym_suffix_decay_sign", "exp(as[i] - as[i + 1]);", "exp(as[i + 1] - as[i]);", 0),
    ("sym_diagonal_twice", "yr[c] = ls[i * m + c] + u[c] - (double)xr[c];", "yr[c] = ls[i * m + c] + u[c];", 0),
    ("sym_no_scatter", "double* yr = y + (size_t)perm[i] * m;", "double* yr = y + (size_t)i * m;", 0),
    ("sym_suffix_dropped", "u[c] = (double)xr[c] + d * u[c];", "u[c] = (double)xr[c];", 0),
    ("general_u_weight_sign", "double w = exp(bj - as[p]);", "double w = exp(as[p] - bj);", 0),
    ("general_v_weight_sign", "double w = exp(as[p - 1] - bj);", "double w = exp(bj - as[p - 1]);", 0),
    ("general_v_dropped", "vv[(p - 1) * m + c] += w * (double)xr[c];", "vv[(p - 1) * m + c] += 0.0 * w * (double)xr[c];", 0),
    ("general_x_unsorted", "const float* xr = x + (size_t)pb[j] * m;", "const float* xr = x + (size_t)j * m;", 0),
    ("general_prefix_decay_sign", "double d = exp(as[i - 1] - as[i]);", "double d = exp(as[i] - as[i - 1]);", 1),
    ("general_suffix_decay_sign", "exp(as[i] - as[i + 1]);", "exp(as[i + 1] - as[i]);", 1),
    ("general_y_unpermuted", "double* yr = y + (size_t)pa[i] * m;", "double* yr = y + (size_t)i * m;", 0),
    ("phased_input_phase_sign", "double complex e = cexp(-I * ph);", "double complex e = cexp(I * ph);", 0),
    ("phased_output_phase_sign", "double complex eo = cexp(I * (double)phi[pa[i]]);", "double complex eo = cexp(-I * (double)phi[pa[i]]);", 0),
    ("phased_imag_part", "yr[c] = creal(eo * w);", "yr[c] = cimag(eo * w);", 0),
    ("phased_diagonal_twice", "if (sym) w -= cexp(", "if (0) w -= cexp(", 0),
    ("phased_general_psi_unsorted", "cexp(-I * (double)psi[pb[j]]);", "cexp(-I * (double)psi[j]);", 0),
    ("phased_general_u_weight", "double w = exp(bj - as[p]);", "double w = exp(as[p] - bj);", 1),
    ("rows_cutoff_too_small", "if (d >= 746.0) continue;", "if (d >= 7.0) continue;", 0),
    ("rows_phase_sign", "cos(pi[r] - (double)psi[j])", "cos(pi[r] + (double)psi[j])", 0),
    ("rows_envelope_signed", "env[r * m + c] += w * fabs((double)xr[c]);", "env[r * m + c] += w * (double)xr[c];", 0),
    ("bwd_signed_sum_sign", "out[e * m + c] = lo - hi;", "out[e * m + c] = hi - lo;", 0),
    ("bwd_ties_counted_above", "q = upper_bound_d(ss, ns, te);", "q = lower_bound_d(ss, ns, te);", 0),
    ("bwd_ties_counted_below", "const int64_t p = lower_bound_d(ss, ns, te)", "const int64_t p = upper_bound_d(ss, ns, te)", 0),
    ("bwd_prefix_decay_sign", "const double d = exp(ss[j - 1] - ss[j]);", "const double d = exp(ss[j] - ss[j - 1]);", 0),
    ("bwd_left_weight_sign", "const double wl = p >= 1 ? exp(ss[p - 1] - te) : 0.0;", "const double wl = p >= 1 ? exp(te - ss[p - 1]) : 0.0;", 0),
    ("bwd_sym_da_sign", "da[i] = -acc;", "da[i] = acc;", 0),
    ("bwd_sym_second_term_dropped", "acc += (double)g[i * m + c] * sx[i * m + c] + (double)x[i * m + c] * sg[i * m + c];",
     "acc += (double)g[i * m + c] * sx[i * m + c];", 0),
    ("bwd_general_db_sign", "db[j] = -acc;", "db[j] = acc;", 0),
    ("bwd_general_da_unweighted", "acc += (double)g[i * m + c] * sa[i * m + c];", "acc += sa[i * m + c];", 0),
    ("bwd_rows_tie_sign", "const double sg = d > 0.0 ? 1.0 : (d < 0.0 ? -1.0 : 0.0);", "const double sg = d >= 0.0 ? 1.0 : -1.0;", 0),
    ("bwd_rows_one_term", "acc += sg * w * (gi * xj + xi * gj);", "acc += sg * w * (gi * xj);", 0),
]


def _replace_nth(text, old, new, nth):
    start = -1
    for _ in range(nth + 1):
        start = text.find(old, start + 1)
        assert start >= 0, "mutation anchor not found: %r (occurrence %d)" % (old, nth)
    return text[:start] + new + text[start + len(old):]


def _any_pin_fails(lib):
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lib)
        except Exception as e:  # AssertionError, ValueError, ...
            failed.append((pin.__name__, type(e).__name__))
    return failed


@pytest.mark.parametrize("mut", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_c_mutant_is_caught(mut, tmp_path):
    name, old, new, nth = mut
    text = open(SRC).read()
    src = tmp_path / ("mut_%s.c" % name)
    src.write_text(_replace_nth(text, old, new, nth))
    so = oracle.build(force=True, out=str(tmp_path / ("libmut_%s.so" % name)), src=str(src))
    lib = oracle.load(so)
    failed = _any_pin_fails(lib)
    assert failed, "planted mistake %s passed every pin" % name


DENSE_MUTANTS = {
    "no_abs": lambda ai, b, phi_i=None, psi=None: np.exp(-(ai[:, None] - b[None, :])) * (
        1.0 if phi_i is None else np.cos(phi_i[:, None] - psi[None, :])),
    "half_rate": lambda ai, b, phi_i=None, psi=None: np.exp(-0.5 * np.abs(ai[:, None] - b[None, :])) * (
        1.0 if phi_i is None else np.cos(phi_i[:, None] - psi[None, :])),
    "phase_sum": lambda ai, b, phi_i=None, psi=None: np.exp(-np.abs(ai[:, None] - b[None, :])) * (
        1.0 if phi_i is None else np.cos(phi_i[:, None] + psi[None, :])),
    "phase_sine": lambda ai, b, phi_i=None, psi=None: np.exp(-np.abs(ai[:, None] - b[None, :])) * (
        1.0 if phi_i is None else np.sin(phi_i[:, None] - psi[None, :])),
    "squared_distance": lambda ai, b, phi_i=None, psi=None: np.exp(-np.square(ai[:, None] - b[None, :])) * (
        1.0 if phi_i is None else np.cos(phi_i[:, None] - psi[None, :])),
}


@pytest.mark.parametrize("name", sorted(DENSE_MUTANTS))
def test_dense_mutant_is_caught(name, monkeypatch, oracle_lib):
    monkeypatch.setattr(odense, "_weights", DENSE_MUTANTS[name])
    failed = _any_pin_fails(oracle_lib)
    assert failed, "planted mistake %s in the dense oracle passed every pin" % name


GRAM_MUTANTS = {
    "no_weights": lambda ar, ac, d: ar @ ac.T,
    "weights_twice": lambda ar, ac, d: (ar * d[None, :]) @ (ac * d[None, :]).T,
    "abs_weights": lambda ar, ac, d: (ar * np.abs(d)[None, :]) @ ac.T,
    "weights_reversed": lambda ar, ac, d: (ar * d[None, ::-1]) @ ac.T,
    "weights_shifted": lambda ar, ac, d: (ar * np.roll(d, 1)[None, :]) @ ac.T,
    "squared_entries": lambda ar, ac, d: (ar * ar * d[None, :]) @ ac.T,
}


@pytest.mark.parametrize("name", sorted(GRAM_MUTANTS))
def test_gram_mutant_is_caught(name, monkeypatch, oracle_lib):
    monkeypatch.setattr(odense, "_gram_combine", GRAM_MUTANTS[name])
    failed = _any_pin_fails(oracle_lib)
    assert failed, "planted mistake %s in the Gram oracle passed every pin" % name


PHASED_BWD_MUTANTS = {
    "phase_terms_swapped": ("_phase_terms", lambda P: (np.sin(P), np.cos(P))),
    "phase_sine_sign": ("_phase_terms", lambda P: (np.cos(P), -np.sin(P))),
    "phase_sum": ("_phase_terms", lambda P: (np.cos(P), np.sin(P) * np.cos(P))),
    "row_term_only": ("_sym_fold", lambda row, col: row),
    "column_term_subtracted": ("_sym_fold", lambda row, col: row - col),
}


@pytest.mark.parametrize("name", sorted(PHASED_BWD_MUTANTS))
def test_phased_backward_mutant_is_caught(name, monkeypatch, oracle_lib):
    attr, fn = PHASED_BWD_MUTANTS[name]
    monkeypatch.setattr(odense, attr, fn)
    failed = _any_pin_fails(oracle_lib)
    assert failed, "planted mistake %s in the phased backward passed every pin" % name


def _nw_mutant(kind):
    """A copy of the normwise error measure with one planted mistake."""
    def f(y, y_ref, env, env_scale=None):
        def cols(v):
            v = np.asarray(v, np.float64)
            return v[:, None] if v.ndim == 1 else v
        if kind == "reshapes_silently":
            y = np.asarray(y, np.float64).reshape(np.shape(y_ref))
        y2, r2 = cols(y), cols(y_ref)
        if y2.shape != r2.shape:
            raise ValueError("shape")
        diff = (y2 - r2) if kind == "signed_numerator" else np.abs(y2 - r2)
        num = np.mean(diff, axis=0) if kind == "mean_over_rows" else np.max(diff, axis=0)
        e2 = np.abs(np.asarray(env, np.float64).reshape(r2.shape))
        den = np.max(e2, axis=0)
        if kind == "global_denominator":
            den = np.full_like(den, np.max(e2))
        if kind == "columns_swapped":
            den = den[::-1]
        if env_scale is not None and kind != "ignores_env_scale":
            den = np.asarray(env_scale, np.float64).ravel()
        if kind != "zero_envelope_divides":
            den = np.where(den > 0, den, 1.0)
        if kind == "vacuous":
            return 0.0
        with np.errstate(divide="ignore", invalid="ignore"):
            q = num / den
        return float(np.sum(q) if kind == "sum_over_columns" else np.max(q))
    return f


NORMWISE_MUTANTS = ["vacuous", "global_denominator", "ignores_env_scale", "mean_over_rows", "signed_numerator",
                    "columns_swapped", "sum_over_columns", "zero_envelope_divides", "reshapes_silently"]


@pytest.mark.parametrize("kind", NORMWISE_MUTANTS)
def test_normwise_mutant_is_caught(kind, monkeypatch, oracle_lib):
    monkeypatch.setattr(odense, "normwise_error", _nw_mutant(kind))
    failed = _any_pin_fails(oracle_lib)
    assert failed, "planted mistake %s in the error measure passed every pin" % kind

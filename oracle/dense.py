"""Dense float64 brute force of the LAPLEX operator -- TEST INFRASTRUCTURE ONLY.

The plain definition of "LAPLEX: The FFT of Learnable Laplace Kernels"
(technical summary, section 2.1 "The Operator"):

    LAPLEX(a, b)_ij              = exp(-|a_i - b_j|)
    LAPLEX(a, phi; b, psi)_ij    = exp(-|a_i - b_j|) * cos(phi_i - psi_j)

applied to x with no sort and no scan, rows processed in chunks so memory
stays bounded.  Inputs are widened to float64 exactly (float32 arrays, as
the GPU receives them, convert without rounding).  Row index i runs over the
output anchors a, column index j over the input anchors b (the pages relabel
the indices between the two formulas; the first index is always the output).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _chunk_rows(k: int, budget: int = 1 << 24) -> int:
    return max(1, budget // max(1, k))


def _weights(ai, b, phi_i=None, psi=None):
    w = np.exp(-np.abs(ai[:, None] - b[None, :]))
    if phi_i is not None:
        w *= np.cos(phi_i[:, None] - psi[None, :])
    return w


def dense_apply(a, x, b=None, phi=None, psi=None) -> np.ndarray:
    """y = LAPLEX(a[, phi]; b[, psi]) x in float64; b None -> b = a (and psi = phi)."""
    a = np.asarray(a, np.float64).ravel()
    b = a if b is None else np.asarray(b, np.float64).ravel()
    if phi is not None:
        phi = np.asarray(phi, np.float64).ravel()
        psi = phi if psi is None else np.asarray(psi, np.float64).ravel()
    x = np.asarray(x, np.float64)
    x2 = x.reshape(b.size, -1)
    y = np.zeros((a.size, x2.shape[1]), np.float64)
    step = _chunk_rows(b.size)
    for lo in range(0, a.size, step):
        hi = min(a.size, lo + step)
        w = _weights(a[lo:hi], b, None if phi is None else phi[lo:hi], psi)
        y[lo:hi] = w @ x2
    return y


def dense_envelope(a, x, b=None) -> np.ndarray:
    """K0 |x| with the unphased kernel: the scale of the normwise error measure."""
    return dense_apply(a, np.abs(np.asarray(x, np.float64)), b=b)


def normwise_error(y, y_ref, env, env_scale: Optional[np.ndarray] = None) -> float:
    """max over columns c of ||y_c - y_ref_c||_inf / ||(K0|x|)_c||_inf.

    y, y_ref and env are (rows,) or (rows, m) with the same shape ((rows,)
    and (rows, 1) count as the same); anything else raises ValueError.  A
    column whose envelope is zero (x_c = 0) is measured by its absolute
    error.  ``env_scale`` may supply the per-column denominators directly
    (e.g. the maximum over sampled rows, which is a lower bound and so a
    stricter test); env is then not used."""
    def cols(v, what):
        v = np.asarray(v, np.float64)
        if v.ndim == 1:
            return v[:, None]
        if v.ndim != 2:
            raise ValueError("%s must be 1-D or 2-D, got shape %s" % (what, v.shape))
        return v
    y2, r2 = cols(y, "y"), cols(y_ref, "y_ref")
    if y2.shape != r2.shape:
        raise ValueError("y has shape %s, y_ref %s" % (np.shape(y), np.shape(y_ref)))
    num = np.max(np.abs(y2 - r2), axis=0) if r2.shape[0] else np.zeros(r2.shape[1])
    if env_scale is None:
        e2 = cols(env, "env")
        if e2.shape != r2.shape:
            raise ValueError("env has shape %s, y_ref %s" % (np.shape(env), np.shape(y_ref)))
        den = np.max(np.abs(e2), axis=0) if e2.shape[0] else np.zeros(e2.shape[1])
    else:
        den = np.asarray(env_scale, np.float64).ravel()
        if den.size != r2.shape[1]:
            raise ValueError("env_scale has %d values for %d columns" % (den.size, r2.shape[1]))
    den = np.where(den > 0, den, 1.0)
    return float(np.max(num / den)) if num.size else 0.0


def dense_backward(a, x, g, b=None):
    """Backward of y = LAPLEX(a, b) x by the plain definition (float64), for an
    upstream gradient g = dL/dy.  With K_ij = exp(-|a_i - b_j|) and
    dK_ij/da_i = -sign(a_i - b_j) K_ij = -dK_ij/db_j (sign(0) = 0):
        dx = K^T g,   da_i = -sum_jc sign(a_i - b_j) K_ij g_ic x_jc,
        db_j = +sum_ic sign(a_i - b_j) K_ij g_ic x_jc.
    Symmetric (b None): one anchor set receives both terms; returns (dx, da).
    General: returns (dx, da, db)."""
    a = np.asarray(a, np.float64).ravel()
    sym = b is None
    b = a if sym else np.asarray(b, np.float64).ravel()
    x2 = np.asarray(x, np.float64).reshape(b.size, -1)
    g2 = np.asarray(g, np.float64).reshape(a.size, -1)
    D = a[:, None] - b[None, :]
    K = np.exp(-np.abs(D))
    SK = np.sign(D) * K
    dx = K.T @ g2
    da = -np.einsum("ij,ic,jc->i", SK, g2, x2)
    db = np.einsum("ij,ic,jc->j", SK, g2, x2)
    if sym:
        return dx, da + db
    return dx, da, db


def dense_phased_backward(a, phi, x, g, b=None, psi=None):
    """Backward of the phased operator y = LAPLEX(a, phi; b, psi) x by the plain
    definition (float64), for g = dL/dy.  With W_ij = K_ij cos(phi_i - psi_j),
    K_ij = exp(-|a_i - b_j|), the chain rule on each entry gives
        dx     = W^T g,
        da_i   = -sum_jc sign(a_i - b_j) W_ij g_ic x_jc,   db_j   = -(the same sum over i, with the opposite sign),
        dphi_i = -sum_jc K_ij sin(phi_i - psi_j) g_ic x_jc, dpsi_j = +sum_ic K_ij sin(phi_i - psi_j) g_ic x_jc
    (sign(0) = 0).  Symmetric (b None: b = a, psi = phi): each anchor and phase
    receives both terms; returns (dx, da, dphi).  General: (dx, da, db, dphi, dpsi)."""
    a = np.asarray(a, np.float64).ravel()
    phi = np.asarray(phi, np.float64).ravel()
    sym = b is None
    b = a if sym else np.asarray(b, np.float64).ravel()
    psi = phi if sym else np.asarray(psi, np.float64).ravel()
    x2 = np.asarray(x, np.float64).reshape(b.size, -1)
    g2 = np.asarray(g, np.float64).reshape(a.size, -1)
    D = a[:, None] - b[None, :]
    P = phi[:, None] - psi[None, :]
    K = np.exp(-np.abs(D))
    cosP, sinP = _phase_terms(P)
    W = K * cosP
    SW = np.sign(D) * W
    KS = K * sinP
    gx = g2 @ x2.T  # gx[i, j] = sum_c g_ic x_jc
    dx = W.T @ g2
    da = -(SW * gx).sum(axis=1)
    db = (SW * gx).sum(axis=0)
    dphi = -(KS * gx).sum(axis=1)
    dpsi = (KS * gx).sum(axis=0)
    if sym:
        return dx, _sym_fold(da, db), _sym_fold(dphi, dpsi)
    return dx, da, db, dphi, dpsi


def _phase_terms(P):
    """cos and sin of the phase differences."""
    return np.cos(P), np.sin(P)


def _sym_fold(row_term, col_term):
    """With b = a (and psi = phi) an anchor or phase is both a row and a column
    parameter: its gradient is the sum of the two terms."""
    return row_term + col_term


def phased_backward_rows(rows, a, phi, x, g, col_chunk: int = 1 << 20):
    """Anchor and phase gradients of the symmetric phased backward at selected
    rows by the plain definition, for sizes where only spot rows can be checked:
        da_i   = -sum_j sign(a_i - a_j) K_ij cos(phi_i - phi_j) s_ij,
        dphi_i = -sum_j K_ij sin(phi_i - phi_j) s_ij,   s_ij = sum_c (g_ic x_jc + x_ic g_jc),
    and their envelope  sum_j K_ij sum_c (|g_ic||x_jc| + |x_ic||g_jc|).
    Returns (da_rows, dphi_rows, env_rows), float64."""
    rows = np.asarray(rows, np.int64)
    a = np.asarray(a).ravel()
    phi = np.asarray(phi).ravel()
    n = a.size
    x2 = np.asarray(x).reshape(n, -1)
    g2 = np.asarray(g).reshape(n, -1)
    ai = a[rows].astype(np.float64)
    pi = phi[rows].astype(np.float64)
    gi = g2[rows].astype(np.float64)
    xi = x2[rows].astype(np.float64)
    da = np.zeros(rows.size)
    dphi = np.zeros(rows.size)
    env = np.zeros(rows.size)
    for lo in range(0, n, col_chunk):
        hi = min(n, lo + col_chunk)
        D = ai[:, None] - a[lo:hi].astype(np.float64)[None, :]
        P = pi[:, None] - phi[lo:hi].astype(np.float64)[None, :]
        K = np.exp(-np.abs(D))
        xj = x2[lo:hi].astype(np.float64)
        gj = g2[lo:hi].astype(np.float64)
        S = gi @ xj.T + xi @ gj.T
        E = np.abs(gi) @ np.abs(xj).T + np.abs(xi) @ np.abs(gj).T
        da -= (np.sign(D) * K * np.cos(P) * S).sum(axis=1)
        dphi -= (K * np.sin(P) * S).sum(axis=1)
        env += (K * E).sum(axis=1)
    return da, dphi, env


# ----------------------------------------------------------------------------- weighted Gram
def _gram_combine(ar_w, ac_w, d):
    """sum_j ar_w[p, j] d_j ac_w[q, j] for one chunk of input anchors."""
    return (ar_w * d[None, :]) @ ac_w.T


def gram_block(rows, cols, a, b, D, absolute: bool = False, col_chunk: int = 1 << 14) -> np.ndarray:
    """Entries M[rows][:, cols] of the weighted Gram matrix M = A diag(D) A^T,
    A = LAPLEX(a, b) (technical summary, section 2.2, Gram operators), by the
    plain definition  M_pq = sum_j D_j exp(-|a_p - b_j|) exp(-|a_q - b_j|),
    O(|rows| |cols| k), float64.  ``absolute`` uses |D| (the envelope that
    scales the normwise error)."""
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    a = np.asarray(a).ravel()
    b = np.asarray(b, np.float64).ravel()
    D = np.asarray(D, np.float64).ravel()
    if absolute:
        D = np.abs(D)
    ar = a[rows].astype(np.float64)
    ac = a[cols].astype(np.float64)
    out = np.zeros((rows.size, cols.size), np.float64)
    for lo in range(0, b.size, col_chunk):
        hi = min(b.size, lo + col_chunk)
        out += _gram_combine(_weights(ar, b[lo:hi]), _weights(ac, b[lo:hi]), D[lo:hi])
    return out


def gram_dense(a, b, D, absolute: bool = False) -> np.ndarray:
    """The whole n x n weighted Gram matrix by the plain definition (small n)."""
    n = np.asarray(a).size
    idx = np.arange(n)
    return gram_block(idx, idx, a, b, D, absolute=absolute)

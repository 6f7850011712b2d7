"""LAPLEX operator on AMD Instinct MI355X (gfx950).

Python binding of liblaplex.so (include/laplex.h).  Argument marshalling
only: every step of the computation runs in the HIP kernels of the library;
PyTorch provides device memory and the current stream.  If the library has
not been built the calls raise -- there is no fallback.

    a_sorted, perm = laplex_sort_anchors(a)          # sort handle of a
    y = laplex_matvec_sym(a_sorted, perm, x)         # y_i = sum_j exp(-|a_i - a_j|) x_j
    y = laplex_sort_matvec_sym(a, x, ws=ws)          # the same from unsorted anchors, in one call
    dx, da = laplex_sort_matvec_sym_backward(ws, g)  # its backward, from what the call left in ws
    y = laplex_matvec_general(a_sorted, perm, b_sorted, perm_b, xb)
    y = laplex_sort_matvec_general(a, b, xb)         # the same, sorting only b (few inputs b)
    y = laplex_matvec_phased(a_sorted, perm, phi, x)  # extra cos(phi_i - phi_j)
    dx, da = laplex_backward_sym(a_sorted, perm, x, g)  # gradients for g = dL/dy
    dxb, da, db = laplex_backward_general(a_sorted, perm, b_sorted, perm_b, xb, g)
    dx, da, dphi = laplex_backward_phased(a_sorted, perm, phi, x, g)
    M = laplex_gram_weighted(a_sorted, perm, b_sorted, perm_b, D)  # A diag(D) A^T
"""
from ._binding import (  # noqa: F401
    LAPLEX_OP_GENERAL,
    LAPLEX_OP_GENERAL_BACKWARD,
    LAPLEX_OP_GRAM,
    LAPLEX_OP_PHASED,
    LAPLEX_OP_PHASED_BACKWARD,
    LAPLEX_OP_PHASED_GENERAL_BACKWARD,
    LAPLEX_OP_PHASED_GENERAL,
    LAPLEX_OP_SORT,
    LAPLEX_OP_SORT_SYM,
    LAPLEX_OP_SORT_GENERAL,
    LAPLEX_OP_SYM,
    LAPLEX_OP_SYM_BACKWARD,
    LaplexError,
    lib,
    lib_path,
    laplex_backward_general,
    laplex_backward_phased,
    laplex_backward_phased_general,
    laplex_backward_sym,
    laplex_gram_weighted,
    laplex_matvec_general,
    laplex_matvec_phased,
    laplex_matvec_sym,
    laplex_matvec_sym_noalloc,
    LAPLEX_SCRATCH_BYTES,
    laplex_sort_matvec_general,
    laplex_sort_matvec_sym,
    laplex_sort_matvec_sym_backward,
    laplex_sort_anchors,
    laplex_status_poll,
    laplex_route_bytes,
    laplex_workspace_bytes,
    profile_launches,
    route_buffer,
    workspace,
)

"""The C-ABI library: it loads, exports every symbol include/laplex.h declares,
and rejects bad arguments on the host (no GPU work is started by any call
here: each one fails an argument check before a launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "laplex.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(laplex_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import laplace_prefix_scans_amd as lp
    if not os.path.exists(lp.lib_path()):
        pytest.skip("liblaplex.so not built")
    return lp.lib()


def test_header_declares_the_entry_points():
    names = _declared()
    for required in ("laplex_sort_anchors", "laplex_matvec_sym", "laplex_matvec_general", "laplex_matvec_phased",
                     "laplex_workspace_bytes", "laplex_status_poll", "laplex_status_string"):
        assert required in names


def test_every_declared_symbol_is_exported(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_workspace_sizes(L):
    import laplace_prefix_scans_amd as lp
    assert lp.laplex_workspace_bytes(lp.LAPLEX_OP_SORT, 1 << 20) >= 16 * (1 << 20)
    assert lp.laplex_workspace_bytes(lp.LAPLEX_OP_SYM, 1 << 20, 0, 16) >= 4 * 16 * (1 << 20)
    assert lp.laplex_workspace_bytes(lp.LAPLEX_OP_PHASED, 1000, 0, 3) > lp.laplex_workspace_bytes(lp.LAPLEX_OP_SYM, 1000, 0, 3)
    assert lp.laplex_workspace_bytes(lp.LAPLEX_OP_GENERAL, 1 << 24, 1 << 16, 1) > 0
    assert lp.laplex_workspace_bytes(lp.LAPLEX_OP_SORT, 1 << 32) == 0  # n out of range
    assert lp.laplex_workspace_bytes(99, 10) == 0
    assert lp.laplex_workspace_bytes(lp.LAPLEX_OP_GENERAL_BACKWARD, 1 << 20, 1 << 10, 2) > \
        lp.laplex_workspace_bytes(lp.LAPLEX_OP_GENERAL, 1 << 20, 1 << 10, 2)
    for op in range(12):
        a = lp.laplex_workspace_bytes(op, 4096, 100, 1)
        b = lp.laplex_workspace_bytes(op, 1 << 22, 1 << 20, 1)
        assert a % 256 == 0 and b % 256 == 0 and b >= a


def test_sizes_grow_with_n(L):
    """Sorts of up to 2^17 keys use 2048-key tiles and larger ones 8192-key
    tiles; route and workspace sizes still never shrink as n grows (a buffer
    sized for n serves every smaller n), across that switch and the size
    (2^19) from which the large tiles outnumber the small ones at 2^17."""
    import laplace_prefix_scans_amd as lp
    ns = [1, 2047, 2048, 2049, 1 << 16, (1 << 17) - 1, 1 << 17, (1 << 17) + 1, (1 << 17) + 8193, 1 << 18,
          (1 << 19) - 1, 1 << 19, (1 << 19) + 1, (1 << 19) + 8193, 1 << 20]
    sizes = [L.laplex_route_bytes(n) for n in ns]
    assert sizes == sorted(sizes), sizes
    for op in range(12):
        sizes = [lp.laplex_workspace_bytes(op, n, 1000, 2) for n in ns]
        assert sizes == sorted(sizes), (op, sizes)


def test_host_argument_errors(L):
    vp = ctypes.c_void_p
    A = vp(0x100000)      # never dereferenced: every call below fails a check first
    B = vp(0x200000)
    W = vp(0x400000)
    OK, NULL, SIZE, ALIGN, WS, OVERLAP = 0, 1, 2, 3, 4, 7
    # n == 0 / m == 0 are no-ops
    assert L.laplex_sort_anchors(None, 0, None, None, None, 0, None, 0, None) == OK
    assert L.laplex_matvec_sym(None, None, None, 0, 1, None, None, None, 0, None) == OK
    assert L.laplex_matvec_sym(A, B, None, 10, 0, A, B, W, 0, None) == OK
    # NULL
    assert L.laplex_sort_anchors(None, 10, B, A, None, 0, W, 1 << 30, None) == NULL
    assert L.laplex_matvec_sym(A, B, None, 10, 1, None, B, W, 1 << 30, None) == NULL
    assert L.laplex_status_poll(None, None) == NULL
    # size
    assert L.laplex_sort_anchors(A, 1 << 32, B, A, None, 0, W, 1 << 40, None) == SIZE
    assert L.laplex_matvec_sym(A, B, None, 1 << 32, 1, A, B, W, 1 << 40, None) == SIZE
    # alignment
    assert L.laplex_sort_anchors(vp(0x100002), 10, B, vp(0x300000), None, 0, W, 1 << 30, None) == ALIGN
    assert L.laplex_sort_anchors(A, 10, B, vp(0x300000), None, 0, vp(0x400010), 1 << 30, None) == ALIGN
    # workspace too small
    assert L.laplex_sort_anchors(A, 1000, B, vp(0x300000), None, 0, W, 64, None) == WS
    assert L.laplex_matvec_sym(A, vp(0x300000), None, 1000, 4, vp(0x500000), vp(0x600000), W, 64, None) == WS
    # overlap: y on top of x
    need = L.laplex_workspace_bytes(1, 1000, 0, 1)
    assert L.laplex_matvec_sym(A, vp(0x300000), None, 1000, 1, vp(0x500000), vp(0x500100), vp(0x10000000), need, None) == OVERLAP
    # the allocation-free variant refuses calls larger than its static scratch before any HIP call
    import laplace_prefix_scans_amd as lp
    big = 1 << 22
    assert lp.laplex_workspace_bytes(lp.LAPLEX_OP_SYM, big, 0, 4) > lp.LAPLEX_SCRATCH_BYTES
    assert L.laplex_matvec_sym_noalloc(A, B, None, big, 4, A, B, None) == 10
    assert L.laplex_matvec_sym_noalloc(A, B, None, 0, 4, A, B, None) == OK
    assert L.laplex_matvec_sym_noalloc(A, B, None, 1 << 32, 1, A, B, None) == SIZE
    assert L.laplex_sort_anchors(A, 1000, vp(0x100100), vp(0x300000), None, 0, vp(0x10000000), 1 << 30, None) == OVERLAP
    # general without b
    need = L.laplex_workspace_bytes(2, 100, 50, 1)
    assert L.laplex_matvec_general(A, vp(0x300000), None, 100, None, None, None, 50, 1, vp(0x500000), vp(0x600000), W, need, None) == NULL
    assert L.laplex_matvec_phased(A, vp(0x300000), None, None, 100, None, None, None, None, 0, 1, vp(0x500000),
                                  vp(0x600000), W, need, None) == NULL
    # general backward: no-ops, NULL, workspace, overlap (dx on top of g)
    GB = L.laplex_backward_general
    assert GB(None, None, None, 0, None, None, None, 0, 1, None, None, None, None, None, None, 0, None) == OK
    assert GB(A, B, None, 10, A, B, None, 5, 0, A, A, B, B, B, W, 0, None) == OK
    assert GB(A, B, None, 10, None, None, None, 0, 1, None, None, None, None, None, None, 0, None) == NULL  # k = 0 needs da
    assert GB(A, B, None, 10, A, B, None, 5, 1, None, A, B, B, B, W, 1 << 30, None) == NULL
    assert GB(A, B, None, 1 << 32, A, B, None, 5, 1, A, A, B, B, B, W, 1 << 40, None) == SIZE
    need = L.laplex_workspace_bytes(6, 1000, 300, 1)
    args = [A, vp(0x300000), None, 1000, vp(0x500000), vp(0x600000), None, 300, 1, vp(0x700000), vp(0x800000),
            vp(0x900000), vp(0xA00000), vp(0xB00000), vp(0x10000000)]
    assert GB(*args, 64, None) == WS
    bad = list(args)
    bad[11] = vp(0x800100)  # dx inside g
    assert GB(*bad, need, None) == OVERLAP
    bad = list(args)
    bad[12] = vp(0xA00002)  # da misaligned
    assert GB(*bad, need, None) == ALIGN
    # phased backward: no-op, NULL phases, workspace, overlap of dphi with phi
    PB = L.laplex_backward_phased
    assert PB(None, None, None, None, 0, 1, None, None, None, None, None, None, 0, None) == OK
    assert PB(A, B, None, None, 10, 1, A, A, B, B, B, W, 1 << 30, None) == NULL
    needp = L.laplex_workspace_bytes(8, 1000, 0, 2)
    pargs = [A, vp(0x300000), None, vp(0x500000), 1000, 2, vp(0x600000), vp(0x700000), vp(0x800000), vp(0x900000),
             vp(0xA00000), vp(0x10000000)]
    assert PB(*pargs, 64, None) == WS
    bad = list(pargs)
    bad[10] = vp(0x500100)  # dphi inside phi
    assert PB(*bad, needp, None) == OVERLAP
    # weighted Gram: no-ops, row range, NULL, workspace, overlap of M with the weights
    GW = L.laplex_gram_weighted
    assert GW(None, None, 0, None, None, 0, None, 0, 1, None, 0, None, 0, None) == OK
    assert GW(A, B, 10, A, B, 5, A, 0, 0, B, 10, W, 0, None) == OK
    assert GW(A, B, 10, A, B, 5, A, 8, 3, vp(0x900000), 10, W, 1 << 30, None) == 9  # rows past n
    assert GW(A, B, 10, A, B, 5, A, 0, 3, vp(0x900000), 9, W, 1 << 30, None) == 9   # ldm < n
    assert GW(A, B, 10, None, B, 5, A, 0, 3, vp(0x900000), 10, W, 1 << 30, None) == NULL
    assert GW(A, B, 1 << 32, A, B, 5, A, 0, 3, vp(0x900000), 1 << 32, W, 1 << 40, None) == SIZE
    assert GW(A, B, 10, A, B, 5, A, 0, 3, vp(0x900000), 1 << 62, W, 1 << 40, None) == SIZE  # M's extent overflows
    need = L.laplex_workspace_bytes(7, 1000, 300, 1)
    assert need > 0
    assert GW(A, vp(0x300000), 1000, vp(0x500000), vp(0x600000), 300, vp(0x700000), 0, 2, vp(0x900000), 1000,
              vp(0x10000000), 64, None) == WS
    assert GW(A, vp(0x300000), 1000, vp(0x500000), vp(0x600000), 300, vp(0x700000), 0, 2, vp(0x700100), 1000,
              vp(0x10000000), need, None) == OVERLAP
    # one-call sort + symmetric apply: no-ops, NULL, size, alignment, workspace, overlaps
    SM = L.laplex_sort_matvec_sym
    assert SM(None, 0, 1, None, None, None, 0, None) == OK
    assert SM(A, 10, 0, None, None, None, 0, None) == OK
    assert SM(A, 10, 1, None, B, W, 1 << 30, None) == NULL
    assert SM(A, 1 << 32, 1, A, B, W, 1 << 40, None) == SIZE
    assert SM(A, 10, 1 << 17, A, B, W, 1 << 40, None) == SIZE
    assert SM(A, 10, 1, vp(0x300002), B, W, 1 << 30, None) == ALIGN
    needs = L.laplex_workspace_bytes(10, 1000, 0, 1)
    assert needs > L.laplex_workspace_bytes(0, 1000, 0, 1)
    assert SM(A, 1000, 1, vp(0x500000), vp(0x600000), vp(0x10000000), needs - 256, None) == WS
    assert SM(A, 1000, 1, vp(0x500000), vp(0x500100), vp(0x10000000), needs, None) == OVERLAP  # y on x
    assert SM(A, 1000, 1, vp(0x500000), vp(0x100100), vp(0x10000000), needs, None) == OVERLAP  # y on a
    assert SM(vp(0x10000100), 1000, 1, vp(0x500000), vp(0x600000), vp(0x10000000), needs, None) == OVERLAP  # a in ws
    # one-call general operator
    SG = L.laplex_sort_matvec_general
    assert SG(None, 0, None, 0, 1, None, None, None, 0, None) == OK
    assert SG(A, 10, None, 5, 1, B, vp(0x300000), W, 1 << 30, None) == NULL  # k > 0 needs b
    assert SG(A, 10, A, 1 << 32, 1, B, vp(0x300000), W, 1 << 40, None) == SIZE
    needg = L.laplex_workspace_bytes(11, 1000, 300, 1)
    assert needg > 0
    assert SG(A, 1000, B, 300, 1, vp(0x300000), vp(0x400000), vp(0x10000000), needg - 256, None) == WS
    assert SG(A, 1000, B, 300, 1, vp(0x300000), vp(0x300100), vp(0x10000000), needg, None) == OVERLAP  # y on x
    assert SG(A, 1000, B, 300, 1, vp(0x300002), vp(0x400000), vp(0x10000000), needg, None) == ALIGN
    # backward from a one-call forward's workspace
    SB = L.laplex_sort_matvec_sym_backward
    assert SB(None, 0, 0, 1, None, None, None, None, 0, None) == OK
    assert SB(W, 1 << 30, 10, 1, None, B, A, W, 1 << 30, None) == NULL
    assert SB(W, 1 << 40, 1 << 32, 1, A, B, vp(0x300000), vp(0x20000000), 1 << 40, None) == SIZE
    needb = L.laplex_workspace_bytes(5, 1000, 0, 1)
    assert SB(vp(0x10000000), needs, 1000, 1, A, B, vp(0x300000), vp(0x20000000), needb - 256, None) == WS
    assert SB(vp(0x10000000), needs - 256, 1000, 1, A, B, vp(0x300000), vp(0x20000000), needb, None) == WS
    assert SB(vp(0x10000000), needs, 1000, 1, A, vp(0x100100), vp(0x300000), vp(0x20000000), needb, None) == OVERLAP  # dx on g
    assert SB(vp(0x10000000), needs, 1000, 1, A, vp(0x10000100), vp(0x300000), vp(0x20000000), needb, None) == OVERLAP
    # route: too small, misaligned, overlapping
    assert L.laplex_sort_anchors(A, 1000, B, vp(0x300000), vp(0x20000000), 16, vp(0x10000000), 1 << 30, None) == WS
    assert L.laplex_sort_anchors(A, 1000, B, vp(0x300000), vp(0x20000010), 1 << 20, vp(0x10000000), 1 << 30, None) == ALIGN
    assert L.laplex_sort_anchors(A, 1000, B, vp(0x300000), vp(0x100000), 1 << 20, vp(0x10000000), 1 << 30, None) == OVERLAP
    assert L.laplex_route_bytes(1 << 20) >= 4 * 2 * (1 << 20)
    assert L.laplex_route_bytes(1 << 32) == 0
    assert L.laplex_status_string(4) == b"workspace too small"


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    import laplace_prefix_scans_amd as lp
    with pytest.raises((ValueError, RuntimeError)):
        lp.laplex_sort_anchors(torch.zeros(8))

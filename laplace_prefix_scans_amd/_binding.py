"""ctypes binding of liblaplex.so (declarations in include/laplex.h)."""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblaplex.so")

LAPLEX_OP_SORT, LAPLEX_OP_SYM, LAPLEX_OP_GENERAL, LAPLEX_OP_PHASED, LAPLEX_OP_PHASED_GENERAL = 0, 1, 2, 3, 4
LAPLEX_OP_SYM_BACKWARD = 5
LAPLEX_OP_GENERAL_BACKWARD = 6
LAPLEX_OP_GRAM = 7
LAPLEX_OP_PHASED_BACKWARD = 8
LAPLEX_OP_PHASED_GENERAL_BACKWARD = 9
LAPLEX_OP_SORT_SYM = 10
LAPLEX_OP_SORT_GENERAL = 11

_STATUS = {
    0: "LAPLEX_OK", 1: "LAPLEX_ERR_NULL", 2: "LAPLEX_ERR_SIZE", 3: "LAPLEX_ERR_ALIGN", 4: "LAPLEX_ERR_WORKSPACE",
    5: "LAPLEX_ERR_NONFINITE", 6: "LAPLEX_ERR_HIP", 7: "LAPLEX_ERR_OVERLAP", 8: "LAPLEX_ERR_STALLED", 9: "LAPLEX_ERR_ARG",
    10: "LAPLEX_ERR_SCRATCH",
}
LAPLEX_SCRATCH_BYTES = 64 << 20  # include/laplex.h

_lock = threading.Lock()
_lib = None


class LaplexError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s: %s (%s)" % (where, _STATUS.get(code, "?"), _lib.laplex_status_string(code).decode()
                                          if _lib is not None else ""))


def lib_path() -> str:
    return LIB_PATH


def lib():
    """Load liblaplex.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("liblaplex.so is not built (python -m laplace_prefix_scans_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, u64, u32, sz, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_int
        L.laplex_workspace_bytes.argtypes = [i32, u64, u64, u32]
        L.laplex_workspace_bytes.restype = sz
        L.laplex_route_bytes.argtypes = [u64]
        L.laplex_route_bytes.restype = sz
        L.laplex_sort_anchors.argtypes = [vp, u64, vp, vp, vp, sz, vp, sz, vp]
        L.laplex_status_poll.argtypes = [vp, vp]
        L.laplex_matvec_sym.argtypes = [vp, vp, vp, u64, u32, vp, vp, vp, sz, vp]
        L.laplex_matvec_sym_noalloc.argtypes = [vp, vp, vp, u64, u32, vp, vp, vp]
        L.laplex_matvec_sym_noalloc.restype = i32
        L.laplex_sort_matvec_sym.argtypes = [vp, u64, u32, vp, vp, vp, sz, vp]
        L.laplex_sort_matvec_sym.restype = i32
        L.laplex_sort_matvec_sym_backward.argtypes = [vp, sz, u64, u32, vp, vp, vp, vp, sz, vp]
        L.laplex_sort_matvec_general.argtypes = [vp, u64, vp, u64, u32, vp, vp, vp, sz, vp]
        L.laplex_sort_matvec_general.restype = i32
        L.laplex_sort_matvec_sym_backward.restype = i32
        L.laplex_matvec_general.argtypes = [vp, vp, vp, u64, vp, vp, vp, u64, u32, vp, vp, vp, sz, vp]
        L.laplex_matvec_phased.argtypes = [vp, vp, vp, vp, u64, vp, vp, vp, vp, u64, u32, vp, vp, vp, sz, vp]
        L.laplex_backward_sym.argtypes = [vp, vp, vp, u64, u32, vp, vp, vp, vp, vp, sz, vp]
        L.laplex_backward_sym.restype = i32
        L.laplex_backward_general.argtypes = [vp, vp, vp, u64, vp, vp, vp, u64, u32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.laplex_backward_general.restype = i32
        L.laplex_gram_weighted.argtypes = [vp, vp, u64, vp, vp, u64, vp, u64, u64, vp, u64, vp, sz, vp]
        L.laplex_gram_weighted.restype = i32
        L.laplex_backward_phased.argtypes = [vp, vp, vp, vp, u64, u32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.laplex_backward_phased.restype = i32
        L.laplex_backward_phased_general.argtypes = [vp, vp, vp, vp, u64, vp, vp, vp, vp, u64, u32, vp, vp, vp, vp, vp, vp,
                                                     vp, vp, sz, vp]
        L.laplex_backward_phased_general.restype = i32
        for f in (L.laplex_sort_anchors, L.laplex_status_poll, L.laplex_matvec_sym, L.laplex_matvec_general,
                  L.laplex_matvec_phased):
            f.restype = i32
        L.laplex_status_string.argtypes = [i32]
        L.laplex_status_string.restype = ctypes.c_char_p
        L.laplex_profile_begin.argtypes = [u32]
        L.laplex_profile_begin.restype = i32
        L.laplex_profile_end.argtypes = []
        L.laplex_profile_end.restype = u32
        L.laplex_profile_get.argtypes = [u32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float),
                                         ctypes.POINTER(ctypes.c_uint64)]
        L.laplex_profile_get.restype = i32
        _lib = L
        return L


def _check(code: int, where: str):
    if code != 0:
        raise LaplexError(code, where)


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _vec(t: torch.Tensor, name: str, dtype=torch.float32) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _cols(x: torch.Tensor, rows: int, name: str = "x") -> int:
    _vec(x, name)
    if x.dim() == 1:
        if x.shape[0] != rows:
            raise ValueError("%s has %d rows, expected %d" % (name, x.shape[0], rows))
        return 1
    if x.dim() != 2 or x.shape[0] != rows:
        raise ValueError("%s must be (%d,) or (%d, m), got %s" % (name, rows, rows, tuple(x.shape)))
    return x.shape[1]


def laplex_workspace_bytes(op: int, n: int, k: int = 0, m: int = 1) -> int:
    return int(lib().laplex_workspace_bytes(op, n, k, m))


def workspace(op: int, n: int, k: int = 0, m: int = 1, device=None) -> torch.Tensor:
    """A byte tensor big enough for one call of ``op``."""
    nbytes = max(256, laplex_workspace_bytes(op, n, k, m))
    return torch.empty(nbytes, dtype=torch.uint8, device=device or torch.device("cuda"))


def _ws(ws: Optional[torch.Tensor], op, n, k, m, dev) -> torch.Tensor:
    if ws is None:
        return workspace(op, n, k, m, dev)
    if ws.device != dev or ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    return ws


def laplex_route_bytes(n: int) -> int:
    return int(lib().laplex_route_bytes(n))


def route_buffer(n: int, device=None) -> torch.Tensor:
    """A byte tensor that can receive the route of a sort of n anchors."""
    return torch.empty(max(256, laplex_route_bytes(n)), dtype=torch.uint8, device=device or torch.device("cuda"))


def laplex_sort_anchors(a: torch.Tensor, a_sorted: Optional[torch.Tensor] = None, perm: Optional[torch.Tensor] = None,
                        route: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                        check: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Stable ascending sort of the anchors: returns (a_sorted, perm) with
    a_sorted = a[perm] and perm a uint32 tensor.  ``route``: optional byte
    tensor (route_buffer(n)) that receives the sort's route for the applies.
    ``check=True`` waits for the stream and raises LaplexError if an anchor
    was NaN/Inf."""
    _vec(a, "a")
    if a.dim() != 1:
        raise ValueError("a must be 1-D")
    n, dev = a.shape[0], a.device
    a_sorted = torch.empty_like(a) if a_sorted is None else _vec(a_sorted, "a_sorted")
    perm = torch.empty(n, dtype=torch.uint32, device=dev) if perm is None else _vec(perm, "perm", torch.uint32)
    if route is not None:
        _vec(route, "route", torch.uint8)
    ws = _ws(ws, LAPLEX_OP_SORT, n, 0, 1, dev)
    L = lib()
    _check(L.laplex_sort_anchors(_ptr(a), n, _ptr(a_sorted), _ptr(perm), _ptr(route), 0 if route is None else route.numel(),
                                 _ptr(ws), ws.numel(), _stream(dev)), "laplex_sort_anchors")
    if check:
        _check(L.laplex_status_poll(_ptr(ws), _stream(dev)), "laplex_sort_anchors")
    return a_sorted, perm


def laplex_status_poll(ws: torch.Tensor) -> int:
    """Wait for the current stream and return the sort workspace's sticky status code."""
    return int(lib().laplex_status_poll(_ptr(ws), _stream(ws.device)))


def laplex_matvec_sym(a_sorted: torch.Tensor, perm: torch.Tensor, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None, route: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = LAPLEX(a, a) x for the sort handle (a_sorted, perm); x is (n,) or (n, m)."""
    _vec(a_sorted, "a_sorted")
    _vec(perm, "perm", torch.uint32)
    n, dev = a_sorted.shape[0], a_sorted.device
    m = _cols(x, n)
    y = torch.empty_like(x) if y is None else y
    _cols(y, n, "y")
    ws = _ws(ws, LAPLEX_OP_SYM, n, 0, m, dev)
    _check(lib().laplex_matvec_sym(_ptr(a_sorted), _ptr(perm), _ptr(route), n, m, _ptr(x), _ptr(y), _ptr(ws), ws.numel(),
                                   _stream(dev)), "laplex_matvec_sym")
    return y


def laplex_matvec_sym_noalloc(a_sorted: torch.Tensor, perm: torch.Tensor, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                              route: Optional[torch.Tensor] = None) -> torch.Tensor:
    """laplex_matvec_sym with the library's static device scratch as its
    workspace: the library call allocates nothing (pass y to allocate
    nothing here either).  Fits when laplex_workspace_bytes(LAPLEX_OP_SYM, n,
    0, m) <= LAPLEX_SCRATCH_BYTES; calls overlapping in time on one GPU race."""
    _vec(a_sorted, "a_sorted")
    _vec(perm, "perm", torch.uint32)
    n, dev = a_sorted.shape[0], a_sorted.device
    m = _cols(x, n)
    y = torch.empty_like(x) if y is None else y
    _cols(y, n, "y")
    _check(lib().laplex_matvec_sym_noalloc(_ptr(a_sorted), _ptr(perm), _ptr(route), n, m, _ptr(x), _ptr(y), _stream(dev)),
           "laplex_matvec_sym_noalloc")
    return y


def laplex_sort_matvec_sym(a: torch.Tensor, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                           ws: Optional[torch.Tensor] = None, check: bool = False) -> torch.Tensor:
    """y = LAPLEX(a, a) x from unsorted anchors in one call (the sort and the
    apply; with one column x rides through the sort).  ``ws``: optional
    workspace of laplex_workspace_bytes(LAPLEX_OP_SORT_SYM, n, 0, m) bytes;
    ``check=True`` waits and raises LaplexError if an anchor was NaN/Inf."""
    _vec(a, "a")
    if a.dim() != 1:
        raise ValueError("a must be 1-D")
    n, dev = a.shape[0], a.device
    m = _cols(x, n)
    y = torch.empty_like(x) if y is None else y
    _cols(y, n, "y")
    ws = _ws(ws, LAPLEX_OP_SORT_SYM, n, 0, m, dev)
    L = lib()
    _check(L.laplex_sort_matvec_sym(_ptr(a), n, m, _ptr(x), _ptr(y), _ptr(ws), ws.numel(), _stream(dev)),
           "laplex_sort_matvec_sym")
    if check:
        _check(L.laplex_status_poll(_ptr(ws), _stream(dev)), "laplex_sort_matvec_sym")
    return y


def laplex_sort_matvec_general(a: torch.Tensor, b: torch.Tensor, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                               ws: Optional[torch.Tensor] = None, check: bool = False) -> torch.Tensor:
    """y = LAPLEX(a, b) x from unsorted anchors in one call, sorting only b (for few input anchors b);
    x is (k,) or (k, m), y (n,) or (n, m).  ``check=True`` waits and raises LaplexError if an anchor
    was NaN/Inf."""
    _vec(a, "a")
    _vec(b, "b")
    if a.dim() != 1 or b.dim() != 1:
        raise ValueError("a and b must be 1-D")
    n, k, dev = a.shape[0], b.shape[0], a.device
    m = _cols(x, k)
    if y is None:
        y = torch.empty((n,) if x.dim() == 1 else (n, m), dtype=torch.float32, device=dev)
    if _cols(y, n, "y") != m:
        raise ValueError("y must have m = %d columns" % m)
    ws = _ws(ws, LAPLEX_OP_SORT_GENERAL, n, k, m, dev)
    L = lib()
    _check(L.laplex_sort_matvec_general(_ptr(a), n, _ptr(b), k, m, _ptr(x), _ptr(y), _ptr(ws), ws.numel(), _stream(dev)),
           "laplex_sort_matvec_general")
    if check:
        _check(L.laplex_status_poll(_ptr(ws), _stream(dev)), "laplex_sort_matvec_general")
    return y


def laplex_sort_matvec_sym_backward(fwd_ws: torch.Tensor, g: torch.Tensor, dx: Optional[torch.Tensor] = None,
                                    da: Optional[torch.Tensor] = None,
                                    ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(dx, da) for the upstream gradient g of y = laplex_sort_matvec_sym(a, x, ws=fwd_ws), from what that
    call left in fwd_ws (sorted anchors, route or permutation, x in sorted order); g is (n,) or (n, m)
    like x.  ``ws``: optional workspace of laplex_workspace_bytes(LAPLEX_OP_SYM_BACKWARD, n, 0, m) bytes."""
    _vec(fwd_ws, "fwd_ws", torch.uint8)
    _vec(g, "g")
    n, dev = g.shape[0], g.device
    m = _cols(g, n, "g")
    dx = torch.empty_like(g) if dx is None else dx
    _cols(dx, n, "dx")
    da = torch.empty(n, dtype=torch.float32, device=dev) if da is None else _vec(da, "da")
    if da.dim() != 1 or da.shape[0] != n:
        raise ValueError("da must be (%d,)" % n)
    ws = _ws(ws, LAPLEX_OP_SYM_BACKWARD, n, 0, m, dev)
    _check(lib().laplex_sort_matvec_sym_backward(_ptr(fwd_ws), fwd_ws.numel(), n, m, _ptr(g), _ptr(dx), _ptr(da), _ptr(ws),
                                                 ws.numel(), _stream(dev)), "laplex_sort_matvec_sym_backward")
    return dx, da


def laplex_backward_sym(a_sorted: torch.Tensor, perm: torch.Tensor, x: torch.Tensor, g: torch.Tensor,
                        dx: Optional[torch.Tensor] = None, da: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None, route: Optional[torch.Tensor] = None):
    """Backward of y = LAPLEX(a, a) x for the upstream gradient g = dL/dy:
    returns (dx = K g, same shape as x; da, (n,))."""
    _vec(a_sorted, "a_sorted")
    _vec(perm, "perm", torch.uint32)
    n, dev = a_sorted.shape[0], a_sorted.device
    m = _cols(x, n)
    if _cols(g, n, "g") != m:
        raise ValueError("g must have the shape of x")
    dx = torch.empty_like(g) if dx is None else dx
    _cols(dx, n, "dx")
    da = torch.empty(n, dtype=torch.float32, device=dev) if da is None else _vec(da, "da")
    ws = _ws(ws, LAPLEX_OP_SYM_BACKWARD, n, 0, m, dev)
    _check(lib().laplex_backward_sym(_ptr(a_sorted), _ptr(perm), _ptr(route), n, m, _ptr(x), _ptr(g), _ptr(dx), _ptr(da),
                                     _ptr(ws), ws.numel(), _stream(dev)), "laplex_backward_sym")
    return dx, da


def laplex_backward_phased(a_sorted: torch.Tensor, perm: torch.Tensor, phi: torch.Tensor, x: torch.Tensor, g: torch.Tensor,
                           dx: Optional[torch.Tensor] = None, da: Optional[torch.Tensor] = None,
                           dphi: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                           route: Optional[torch.Tensor] = None):
    """Backward of the symmetric phased operator y = LAPLEX(a, phi; a, phi) x for g = dL/dy:
    returns (dx, same shape as x; da, (n,); dphi, (n,))."""
    _vec(a_sorted, "a_sorted")
    _vec(perm, "perm", torch.uint32)
    _vec(phi, "phi")
    n, dev = a_sorted.shape[0], a_sorted.device
    if phi.shape[0] != n:
        raise ValueError("phi must have one phase per anchor")
    m = _cols(x, n)
    if _cols(g, n, "g") != m:
        raise ValueError("g must have the shape of x")
    dx = torch.empty_like(g) if dx is None else dx
    _cols(dx, n, "dx")
    da = torch.empty(n, dtype=torch.float32, device=dev) if da is None else _vec(da, "da")
    dphi = torch.empty(n, dtype=torch.float32, device=dev) if dphi is None else _vec(dphi, "dphi")
    ws = _ws(ws, LAPLEX_OP_PHASED_BACKWARD, n, 0, m, dev)
    _check(lib().laplex_backward_phased(_ptr(a_sorted), _ptr(perm), _ptr(route), _ptr(phi), n, m, _ptr(x), _ptr(g),
                                        _ptr(dx), _ptr(da), _ptr(dphi), _ptr(ws), ws.numel(), _stream(dev)),
           "laplex_backward_phased")
    return dx, da, dphi


def laplex_backward_phased_general(a_sorted: torch.Tensor, perm_a: torch.Tensor, phi: torch.Tensor, b_sorted: torch.Tensor,
                                   perm_b: torch.Tensor, psi: torch.Tensor, x: torch.Tensor, g: torch.Tensor,
                                   ws: Optional[torch.Tensor] = None, route_a: Optional[torch.Tensor] = None,
                                   route_b: Optional[torch.Tensor] = None, out=None):
    """Backward of y = LAPLEX(a, phi; b, psi) x for g = dL/dy (x: (k,) or (k, m); g: (n,) or (n, m)):
    returns (dx, shape of x; da, (n,); db, (k,); dphi, (n,); dpsi, (k,)).  `out`: optional tuple of
    the five output tensors."""
    _vec(a_sorted, "a_sorted")
    _vec(perm_a, "perm_a", torch.uint32)
    _vec(phi, "phi")
    _vec(b_sorted, "b_sorted")
    _vec(perm_b, "perm_b", torch.uint32)
    _vec(psi, "psi")
    n, k, dev = a_sorted.shape[0], b_sorted.shape[0], a_sorted.device
    if phi.shape[0] != n or psi.shape[0] != k:
        raise ValueError("phi and psi must have one phase per anchor")
    m = _cols(x, k)
    if _cols(g, n, "g") != m or g.dim() != x.dim():
        raise ValueError("g must have n rows and the columns of x")
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = (torch.empty_like(x), torch.empty(n, **f32), torch.empty(k, **f32), torch.empty(n, **f32),
               torch.empty(k, **f32))
    dx, da, db, dphi, dpsi = out
    _cols(dx, k, "dx")
    for t, name in ((da, "da"), (db, "db"), (dphi, "dphi"), (dpsi, "dpsi")):
        _vec(t, name)
    ws = _ws(ws, LAPLEX_OP_PHASED_GENERAL_BACKWARD, n, k, m, dev)
    _check(lib().laplex_backward_phased_general(_ptr(a_sorted), _ptr(perm_a), _ptr(route_a), _ptr(phi), n, _ptr(b_sorted),
                                                _ptr(perm_b), _ptr(route_b), _ptr(psi), k, m, _ptr(x), _ptr(g), _ptr(dx),
                                                _ptr(da), _ptr(db), _ptr(dphi), _ptr(dpsi), _ptr(ws), ws.numel(),
                                                _stream(dev)), "laplex_backward_phased_general")
    return dx, da, db, dphi, dpsi


def laplex_backward_general(a_sorted: torch.Tensor, perm_a: torch.Tensor, b_sorted: torch.Tensor, perm_b: torch.Tensor,
                            x: torch.Tensor, g: torch.Tensor, dx: Optional[torch.Tensor] = None,
                            da: Optional[torch.Tensor] = None, db: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None, route_a: Optional[torch.Tensor] = None,
                            route_b: Optional[torch.Tensor] = None):
    """Backward of y = LAPLEX(a, b) x for the upstream gradient g = dL/dy
    (x: (k,) or (k, m); g: (n,) or (n, m)): returns (dx = K^T g, shape of x;
    da, (n,); db, (k,))."""
    _vec(a_sorted, "a_sorted")
    _vec(perm_a, "perm_a", torch.uint32)
    _vec(b_sorted, "b_sorted")
    _vec(perm_b, "perm_b", torch.uint32)
    n, k, dev = a_sorted.shape[0], b_sorted.shape[0], a_sorted.device
    m = _cols(x, k)
    if _cols(g, n, "g") != m or g.dim() != x.dim():
        raise ValueError("g must have n rows and the columns of x")
    dx = torch.empty_like(x) if dx is None else dx
    _cols(dx, k, "dx")
    da = torch.empty(n, dtype=torch.float32, device=dev) if da is None else _vec(da, "da")
    db = torch.empty(k, dtype=torch.float32, device=dev) if db is None else _vec(db, "db")
    ws = _ws(ws, LAPLEX_OP_GENERAL_BACKWARD, n, k, m, dev)
    _check(lib().laplex_backward_general(_ptr(a_sorted), _ptr(perm_a), _ptr(route_a), n, _ptr(b_sorted), _ptr(perm_b),
                                         _ptr(route_b), k, m, _ptr(x), _ptr(g), _ptr(dx), _ptr(da), _ptr(db), _ptr(ws),
                                         ws.numel(), _stream(dev)), "laplex_backward_general")
    return dx, da, db


def laplex_gram_weighted(a_sorted: torch.Tensor, perm_a: torch.Tensor, b_sorted: torch.Tensor, perm_b: torch.Tensor,
                         D: torch.Tensor, M: Optional[torch.Tensor] = None, row_begin: int = 0,
                         row_count: Optional[int] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows [row_begin, row_begin + row_count) of M = A diag(D) A^T, A = LAPLEX(a, b), rows and columns in
    the original order of a.  M: (row_count, >= n) float32 with unit column stride (a new (row_count, n)
    tensor if None)."""
    _vec(a_sorted, "a_sorted")
    _vec(perm_a, "perm_a", torch.uint32)
    _vec(b_sorted, "b_sorted")
    _vec(perm_b, "perm_b", torch.uint32)
    _vec(D, "D")
    n, k, dev = a_sorted.shape[0], b_sorted.shape[0], a_sorted.device
    if D.shape[0] != k:
        raise ValueError("D must have one weight per anchor of b")
    rc = n - row_begin if row_count is None else row_count
    if M is None:
        M = torch.empty((rc, n), dtype=torch.float32, device=dev)
    if M.dim() != 2 or M.shape[0] != rc or M.shape[1] < n or M.stride(1) != 1 or M.dtype != torch.float32 \
            or M.device != dev:
        raise ValueError("M must be a float32 (row_count, >= n) tensor with unit column stride on %s" % dev)
    ldm = M.stride(0) if rc > 1 else max(n, M.stride(0))  # one row: the stride is never used
    ws = _ws(ws, LAPLEX_OP_GRAM, n, k, 1, dev)
    _check(lib().laplex_gram_weighted(_ptr(a_sorted), _ptr(perm_a), n, _ptr(b_sorted), _ptr(perm_b), k, _ptr(D),
                                      row_begin, rc, _ptr(M), ldm, _ptr(ws), ws.numel(), _stream(dev)),
           "laplex_gram_weighted")
    return M


def laplex_matvec_general(a_sorted: torch.Tensor, perm_a: torch.Tensor, b_sorted: torch.Tensor, perm_b: torch.Tensor,
                          x: torch.Tensor, y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                          route_a: Optional[torch.Tensor] = None, route_b: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = LAPLEX(a, b) x; x is (k,) or (k, m), y is (n,) or (n, m)."""
    _vec(a_sorted, "a_sorted")
    _vec(perm_a, "perm_a", torch.uint32)
    _vec(b_sorted, "b_sorted")
    _vec(perm_b, "perm_b", torch.uint32)
    n, k, dev = a_sorted.shape[0], b_sorted.shape[0], a_sorted.device
    m = _cols(x, k)
    if y is None:
        y = torch.empty((n,) if x.dim() == 1 else (n, m), dtype=torch.float32, device=dev)
    _cols(y, n, "y")
    ws = _ws(ws, LAPLEX_OP_GENERAL, n, k, m, dev)
    _check(lib().laplex_matvec_general(_ptr(a_sorted), _ptr(perm_a), _ptr(route_a), n, _ptr(b_sorted), _ptr(perm_b),
                                       _ptr(route_b), k, m, _ptr(x), _ptr(y), _ptr(ws), ws.numel(), _stream(dev)),
           "laplex_matvec_general")
    return y


def laplex_matvec_phased(a_sorted: torch.Tensor, perm_a: torch.Tensor, phi: torch.Tensor, x: torch.Tensor,
                         b_sorted: Optional[torch.Tensor] = None, perm_b: Optional[torch.Tensor] = None,
                         psi: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                         ws: Optional[torch.Tensor] = None, route_a: Optional[torch.Tensor] = None,
                         route_b: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = LAPLEX(a, phi; b, psi) x.  Without b: the symmetric phased operator (b = a, psi = phi)."""
    _vec(a_sorted, "a_sorted")
    _vec(perm_a, "perm_a", torch.uint32)
    _vec(phi, "phi")
    n, dev = a_sorted.shape[0], a_sorted.device
    if b_sorted is None:
        k, op = 0, LAPLEX_OP_PHASED
        m = _cols(x, n)
    else:
        _vec(b_sorted, "b_sorted")
        _vec(perm_b, "perm_b", torch.uint32)
        _vec(psi, "psi")
        k, op = b_sorted.shape[0], LAPLEX_OP_PHASED_GENERAL
        m = _cols(x, k)
    if y is None:
        y = torch.empty((n,) if x.dim() == 1 else (n, m), dtype=torch.float32, device=dev)
    _cols(y, n, "y")
    ws = _ws(ws, op, n, k, m, dev)
    _check(lib().laplex_matvec_phased(_ptr(a_sorted), _ptr(perm_a), _ptr(route_a), _ptr(phi), n, _ptr(b_sorted), _ptr(perm_b),
                                      _ptr(route_b), _ptr(psi), k, m, _ptr(x), _ptr(y), _ptr(ws), ws.numel(), _stream(dev)),
           "laplex_matvec_phased")
    return y


class profile_launches:
    """Context manager recording the duration of every kernel the library
    launches inside it (HIP events on each launch's stream).

        with profile_launches() as prof:
            ...
        prof.records  # [(kernel name, ms, elements), ...] in launch order
    """

    def __init__(self, capacity: int = 65536):
        self.capacity = capacity
        self.records = []

    def __enter__(self):
        _check(lib().laplex_profile_begin(self.capacity), "laplex_profile_begin")
        return self

    def __exit__(self, *exc):
        L = lib()
        cnt = L.laplex_profile_end()
        name, ms, units = ctypes.c_char_p(), ctypes.c_float(), ctypes.c_uint64()
        self.records = []
        for i in range(cnt):
            _check(L.laplex_profile_get(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(units)), "laplex_profile_get")
            self.records.append((name.value.decode(), float(ms.value), int(units.value)))
        return False

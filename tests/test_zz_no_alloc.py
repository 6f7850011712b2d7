"""The allocation-free symmetric apply (laplex_matvec_sym_noalloc: the
library's static device scratch as workspace) against laplex_matvec_sym with
a caller workspace: bitwise the same output, on two calls in a row of which
the second is smaller (the scratch keeps the first call's contents), and
within the parity bar of the float64 oracle; calls too large for the
scratch are refused before any launch."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev, gpu_sort, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _case(n, m, seed):
    r = np.random.default_rng(np.random.SeedSequence([0x5C7A, seed]))
    a = r.uniform(0, n / 8.0 + 1.0, n).astype(np.float32)
    x = r.standard_normal((n, m)).astype(np.float32)
    return a, x


# (first call, second smaller call): routed one column, routed three columns, rows by index
SEQUENCES = [((1000003, 1, True), (70001, 1, True)),
             ((200003, 3, True), (5000, 3, True)),
             ((300001, 8, False), (4097, 8, False))]


@pytest.mark.parametrize("calls", SEQUENCES, ids=["routed_m1", "routed_m3", "index_m8"])
def test_noalloc_matches_workspace_call(calls):
    import torch
    import laplace_prefix_scans_amd as lp
    for i, (n, m, routed) in enumerate(calls):
        print("noalloc call %d: n=%d m=%d routed=%s" % (i, n, m, routed), flush=True)
        assert lp.laplex_workspace_bytes(lp.LAPLEX_OP_SYM, n, 0, m) <= lp.LAPLEX_SCRATCH_BYTES
        a, x = _case(n, m, 10 * i + m)
        a_d = dev(a)
        route = lp.route_buffer(n) if routed else None
        a_s, perm = lp.laplex_sort_anchors(a_d, route=route, check=True)
        x_d = dev(x)
        y_ws = lp.laplex_matvec_sym(a_s, perm, x_d, route=route)
        y = torch.empty_like(x_d)
        lp.laplex_matvec_sym_noalloc(a_s, perm, x_d, y=y, route=route)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ws.view(torch.int32)), "n=%d m=%d: differs from the workspace call" % (n, m)
        yh = host(y)
        assert np.isfinite(yh).all()
        err = oracle.normwise_error(yh, oracle.sym_apply(a, x), oracle.sym_apply(a, np.abs(x)))
        assert err <= TOL, "n=%d m=%d err=%.3e" % (n, m, err)


def test_noalloc_refuses_calls_beyond_the_scratch():
    import torch
    import laplace_prefix_scans_amd as lp
    n, m = 1 << 22, 4
    assert lp.laplex_workspace_bytes(lp.LAPLEX_OP_SYM, n, 0, m) > lp.LAPLEX_SCRATCH_BYTES
    a_s = torch.zeros(n, dtype=torch.float32, device="cuda")
    perm = torch.zeros(n, dtype=torch.uint32, device="cuda")
    x = torch.zeros((n, m), dtype=torch.float32, device="cuda")
    with pytest.raises(lp.LaplexError) as ei:
        lp.laplex_matvec_sym_noalloc(a_s, perm, x)
    assert ei.value.code == 10

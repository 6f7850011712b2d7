"""Failure paths forced from the host, with every kernel still exiting
normally: a look-back wait that reaches its spin limit.

LAPLEX_DEBUG_STALL=<k> makes laplex_sort_anchors run its look-back passes
without publishing and with a spin limit of k, so every tile that looks back
waits for a predecessor that never publishes, gives up after k spins and
raises the watchdog flag; the passes after it stop at once.  The sort must
then report LAPLEX_ERR_STALLED through laplex_status_poll, and the same
workspace must sort correctly again once the variable is gone (the status
is cleared by every call)."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

STALLED = 8


@pytest.mark.parametrize("n", [20001, 1 << 22])  # look-back in every pass; first pass from the tile tables
def test_forced_stall_is_reported(n, monkeypatch):
    import laplace_prefix_scans_amd as lp
    r = np.random.default_rng(np.random.SeedSequence([0x57A11, n]))
    a = r.uniform(0, n / 4.0, n).astype(np.float32)
    a_d = dev(a)
    ws = lp.workspace(lp.LAPLEX_OP_SORT, n)
    print("forced stall: n=%d" % n, flush=True)
    monkeypatch.setenv("LAPLEX_DEBUG_STALL", "4")
    lp.laplex_sort_anchors(a_d, ws=ws)
    assert lp.laplex_status_poll(ws) == STALLED
    monkeypatch.delenv("LAPLEX_DEBUG_STALL")
    a_s, perm = lp.laplex_sort_anchors(a_d, ws=ws)
    assert lp.laplex_status_poll(ws) == 0
    assert np.array_equal(host(perm), oracle.stable_argsort(a)), "the sort after a stall is not the stable argsort"
    assert np.array_equal(host(a_s).view(np.uint32), a[host(perm)].view(np.uint32))


def test_stall_hook_leaves_one_call_paths_alone(monkeypatch):
    """Only the standalone sort honours the hook: the one-call operator, whose
    apply follows its sort in the same call, sorts normally under it."""
    import laplace_prefix_scans_amd as lp
    n = 50001
    r = np.random.default_rng(np.random.SeedSequence([0x57A11, 7]))
    a = r.uniform(0, n / 4.0, n).astype(np.float32)
    x = r.standard_normal(n).astype(np.float32)
    monkeypatch.setenv("LAPLEX_DEBUG_STALL", "4")
    ws = lp.workspace(lp.LAPLEX_OP_SORT_SYM, n, 0, 1)
    y = lp.laplex_sort_matvec_sym(dev(a), dev(x), ws=ws)
    assert lp.laplex_status_poll(ws) == 0
    err = oracle.normwise_error(host(y), oracle.sym_apply(a, x), oracle.sym_apply(a, np.abs(x)))
    assert err <= 1e-5

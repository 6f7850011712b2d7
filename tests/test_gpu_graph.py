"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph): a whole
step (sorts and the operator) captured once and replayed several times, with
new inputs copied in and eager work between the replays; every replay must
give the same bits as the same step run eagerly.  The library allocates
nothing and clears its counters with kernels, so a captured step holds only
kernel nodes."""
import numpy as np
import pytest

from gpu_util import have_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([0x6A9, seed]))


def _setup(kind, n, k, m):
    """Static input/output tensors, a function filling the inputs for replay
    r, the step, and the outputs to compare."""
    import torch
    import laplace_prefix_scans_amd as lp
    dev = torch.device("cuda")
    a = torch.empty(n, device=dev)
    a_s, pa = torch.empty(n, device=dev), torch.empty(n, dtype=torch.uint32, device=dev)
    ws_a = lp.workspace(lp.LAPLEX_OP_SORT, n, device=dev)
    ra = lp.route_buffer(n, device=dev) if m <= 4 else None
    st = {"a": a}
    if kind in ("general", "gen_backward", "gram", "phased_gen_backward"):
        b = torch.empty(k, device=dev)
        b_s, pb = torch.empty(k, device=dev), torch.empty(k, dtype=torch.uint32, device=dev)
        ws_b = lp.workspace(lp.LAPLEX_OP_SORT, k, device=dev)
        rb = lp.route_buffer(k, device=dev) if m <= 4 else None
        st["b"] = b
    rows_x = k if kind in ("general", "gen_backward", "gram", "phased_gen_backward", "sort_general") else n
    x = torch.empty(rows_x, m, device=dev)
    st["x"] = x
    outs = []
    if kind == "sort_general":
        b = torch.empty(k, device=dev)
        st["b"] = b
        y = torch.empty(n, m, device=dev)
        ws = lp.workspace(lp.LAPLEX_OP_SORT_GENERAL, n, k, m, device=dev)

        def op():
            lp.laplex_sort_matvec_general(a, b, x, y=y, ws=ws)
        outs = [y]
    elif kind == "sort_sym_backward":
        g = torch.empty(n, m, device=dev)
        st["g"] = g
        y = torch.empty(n, m, device=dev)
        dx, da = torch.empty(n, m, device=dev), torch.empty(n, device=dev)
        ws = lp.workspace(lp.LAPLEX_OP_SORT_SYM, n, 0, m, device=dev)
        ws_b = lp.workspace(lp.LAPLEX_OP_SYM_BACKWARD, n, 0, m, device=dev)

        def op():
            lp.laplex_sort_matvec_sym(a, x, y=y, ws=ws)
            lp.laplex_sort_matvec_sym_backward(ws, g, dx=dx, da=da, ws=ws_b)
        outs = [y, dx, da]
    elif kind == "sort_sym":
        y = torch.empty(n, m, device=dev)
        ws = lp.workspace(lp.LAPLEX_OP_SORT_SYM, n, 0, m, device=dev)

        def op():
            lp.laplex_sort_matvec_sym(a, x, y=y, ws=ws)
        outs = [y]
    elif kind == "sym":
        y = torch.empty(n, m, device=dev)
        ws = lp.workspace(lp.LAPLEX_OP_SYM, n, 0, m, device=dev)

        def op():
            lp.laplex_matvec_sym(a_s, pa, x, y=y, ws=ws, route=ra)
        outs = [y]
    elif kind == "phased":
        phi = torch.empty(n, device=dev)
        st["phi"] = phi
        y = torch.empty(n, m, device=dev)
        ws = lp.workspace(lp.LAPLEX_OP_PHASED, n, 0, m, device=dev)

        def op():
            lp.laplex_matvec_phased(a_s, pa, phi, x, y=y, ws=ws, route_a=ra)
        outs = [y]
    elif kind == "general":
        y = torch.empty(n, m, device=dev)
        ws = lp.workspace(lp.LAPLEX_OP_GENERAL, n, k, m, device=dev)

        def op():
            lp.laplex_sort_anchors(b, b_s, pb, route=rb, ws=ws_b)
            lp.laplex_matvec_general(a_s, pa, b_s, pb, x, y=y, ws=ws, route_a=ra, route_b=rb)
        outs = [y]
    elif kind == "sym_backward":
        g = torch.empty(n, m, device=dev)
        st["g"] = g
        dx, da = torch.empty(n, m, device=dev), torch.empty(n, device=dev)
        ws = lp.workspace(lp.LAPLEX_OP_SYM_BACKWARD, n, 0, m, device=dev)

        def op():
            lp.laplex_backward_sym(a_s, pa, x, g, dx=dx, da=da, ws=ws, route=ra)
        outs = [dx, da]
    elif kind == "gen_backward":
        g = torch.empty(n, m, device=dev)
        st["g"] = g
        dx, da, db = torch.empty(k, m, device=dev), torch.empty(n, device=dev), torch.empty(k, device=dev)
        ws = lp.workspace(lp.LAPLEX_OP_GENERAL_BACKWARD, n, k, m, device=dev)

        def op():
            lp.laplex_sort_anchors(b, b_s, pb, route=rb, ws=ws_b)
            lp.laplex_backward_general(a_s, pa, b_s, pb, x, g, dx=dx, da=da, db=db, ws=ws, route_a=ra, route_b=rb)
        outs = [dx, da, db]
    elif kind == "phased_backward":
        phi = torch.empty(n, device=dev)
        g = torch.empty(n, m, device=dev)
        st["phi"] = phi
        st["g"] = g
        dx, da, dphi = torch.empty(n, m, device=dev), torch.empty(n, device=dev), torch.empty(n, device=dev)
        ws = lp.workspace(lp.LAPLEX_OP_PHASED_BACKWARD, n, 0, m, device=dev)

        def op():
            lp.laplex_backward_phased(a_s, pa, phi, x, g, dx=dx, da=da, dphi=dphi, ws=ws, route=ra)
        outs = [dx, da, dphi]
    elif kind == "phased_gen_backward":
        phi, psi = torch.empty(n, device=dev), torch.empty(k, device=dev)
        g = torch.empty(n, m, device=dev)
        st["phi"] = phi
        st["psi"] = psi
        st["g"] = g
        out = (torch.empty(k, m, device=dev), torch.empty(n, device=dev), torch.empty(k, device=dev),
               torch.empty(n, device=dev), torch.empty(k, device=dev))
        ws = lp.workspace(lp.LAPLEX_OP_PHASED_GENERAL_BACKWARD, n, k, m, device=dev)

        def op():
            lp.laplex_sort_anchors(b, b_s, pb, route=rb, ws=ws_b)
            lp.laplex_backward_phased_general(a_s, pa, phi, b_s, pb, psi, x, g, ws=ws, route_a=ra, route_b=rb, out=out)
        outs = list(out)
    else:  # gram
        D = torch.empty(k, device=dev)
        st["D"] = D
        M = torch.empty(n, n, device=dev)
        ws = lp.workspace(lp.LAPLEX_OP_GRAM, n, k, 1, device=dev)

        def op():
            lp.laplex_sort_anchors(b, b_s, pb, ws=ws_b)
            lp.laplex_gram_weighted(a_s, pa, b_s, pb, D, M=M, ws=ws)
        outs = [M]

    def step():
        lp.laplex_sort_anchors(a, a_s, pa, route=ra, ws=ws_a)
        op()

    def fill(r):
        g = _rng(1000 * r + n)
        for name, t in st.items():
            if name in ("a", "b"):
                t.copy_(torch.from_numpy(np.round(g.uniform(0, t.numel() / 8.0 + 1, t.numel())).astype(np.float32)
                                         if r % 2 else g.uniform(0, t.numel() / 8.0 + 1, t.numel()).astype(np.float32)))
            elif name in ("phi", "psi"):
                t.copy_(torch.from_numpy(g.uniform(0, 2 * np.pi, t.numel()).astype(np.float32)))
            elif name == "D":
                t.copy_(torch.from_numpy(g.uniform(0, 1, t.numel()).astype(np.float32)))
            else:
                t.copy_(torch.from_numpy(g.standard_normal(tuple(t.shape)).astype(np.float32)))
    return step, fill, outs, [a_s, pa]


@pytest.mark.parametrize("kind,n,k,m", [("sort_sym", 100000, 0, 1), ("sort_general", 90000, 7000, 2), ("sort_sym_backward", 80000, 0, 1), ("sym", 100000, 0, 1), ("sym", 70001, 0, 8), ("phased", 50000, 0, 4),
                                        ("general", 90000, 7000, 1), ("sym_backward", 60000, 0, 2),
                                        ("gen_backward", 40000, 9000, 1), ("gram", 3000, 5000, 1),
                                        ("phased_backward", 30000, 0, 3), ("phased_gen_backward", 20000, 6000, 2)])
def test_graph_replays_match_eager(kind, n, k, m):
    import torch
    step, fill, outs, handle = _setup(kind, n, k, m)
    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(1, 5):
        fill(r)                      # new inputs, copied in eagerly
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs + handle]
        step()                       # the same step, eagerly
        torch.cuda.synchronize()
        for i, (u, v) in enumerate(zip(got, outs + handle)):
            assert torch.equal(u.view(torch.int32), v.view(torch.int32)), (kind, r, i)  # same bits
        assert torch.isfinite(junk)

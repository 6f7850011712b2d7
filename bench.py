#!/usr/bin/env python3
"""LAPLEX operator benchmark on one MI355X (gfx950).

One step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: the stable sort of the anchors (for the general
operator: of a and of b) followed by the operator apply, y = LAPLEX x.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  ``value`` is the whole step's throughput in output
elements (n*m) per second.  ``roofline`` describes the kernel with the most
time per step: its algorithmic bytes per launch (each array it must read or
write, once, at its useful size) over its average launch duration, measured
with HIP events bracketing each launch on its own stream during the timed
steps.  ``traffic`` is the HBM bytes per launch of that kernel from a
committed rocprofv3 counter summary (profiles/), or null when none matches
the current kernel sources.  ``cpu_baseline`` times the float64 CPU oracle on
a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LAPLEX matvec Gelem/s and achieved HBM GB/s (% of peak), n=2^20..2^30"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
CSRC = os.path.join(ROOT, "laplace_prefix_scans_amd", "csrc")


def source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def kernel_bytes(name: str, units: int, m: int, k: int = 0) -> float:
    """Algorithmic bytes of one launch: every array the kernel must touch, once,
    at its useful size (a random row access counts its 4m useful bytes).
    ``units`` = elements (rows) the launch processes; ``k`` = input anchors of
    the general operator."""
    route = 2.0 + 1536.0 / 4096.0   # u16 position per element + 1.5 KiB of digit tables per 4096-element tile
    table = {
        "k_sort_hist": 4.0,                      # read anchors
        "k_onesweep_first": 12.0,                # read anchors; write keys and indices
        "k_onesweep_mid": 16.0,                  # read and write key + value
        "k_onesweep_last": 16.0,
        "k_onesweep_first_routed": 12.0 + route,
        "k_onesweep_mid_routed": 16.0 + route,
        "k_onesweep_last_routed": 16.0 + route,
        "k_sym_gather_reduce": 8.0 + 8.0 * m,    # perm, sorted anchors, x rows in (random), sorted rows out
        "k_sym_apply": 8.0 + 8.0 * m,            # sorted anchors, perm, sorted rows in, y rows out (random)
        "k_sym_reduce": 4.0 + 4.0 * m,           # sorted anchors, sorted rows
        "k_sym_apply_sorted": 4.0 + 8.0 * m,     # sorted anchors, sorted rows in, sorted rows out
        "k_phased_gather_reduce": 16.0 + 8.0 * m,
        "k_phased_apply": 12.0 + 8.0 * m,
        "k_phased_reduce": 8.0 + 4.0 * m,
        "k_phased_apply_sorted": 8.0 + 8.0 * m,
        "k_gather_rows": 4.0 + 8.0 * m,
        "k_gen_reduce": 4.0 + 4.0 * m,
        "k_phased_gen_reduce": 8.0 + 4.0 * m,
    }
    for w in (1, 2, 3, 4):
        table["k_route_fwd_w%d" % w] = route + 8.0 * w   # position, row in, row out
        table["k_route_inv_w%d" % w] = route + 8.0 * w
    if name in table:
        return table[name] * units
    if name in ("k_gen_apply", "k_phased_gen_apply"):
        return (8.0 + 4.0 * m) * units + (4.0 + 4.0 * m) * k
    if name in ("k_gen_apply_sorted", "k_phased_gen_apply_sorted"):
        return (4.0 + 4.0 * m) * units + (4.0 + 4.0 * m) * k
    return 0.0


def load_traffic(workload: str, kernel: str, src_hash: str):
    """HBM bytes per launch of ``kernel`` from a committed counter summary, or None."""
    path = os.path.join(ROOT, "profiles", "counters_%s.txt" % workload)
    if not os.path.exists(path):
        return None, None
    meta, rows = {}, {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#") and "=" in line:
                kk, vv = line[1:].split("=", 1)
                meta[kk.strip()] = vv.strip()
            elif line and not line.startswith("#"):
                parts = line.split()
                if len(parts) >= 3:
                    rows[parts[0]] = (float(parts[1]), float(parts[2]))
    if meta.get("source_hash") != src_hash or kernel not in rows:
        return None, path
    factor = float(meta.get("copy_factor", "1.0"))
    fetch_kib, write_kib = rows[kernel]
    return (fetch_kib + write_kib) * 1024.0 * factor, path


def cpu_baseline(workload: str, log2_sample: int):
    """The float64 oracle (sort + scans, one host core) on a bounded sample."""
    import oracle
    from synth import make_workload, WORKLOADS

    full = make_workload(workload, scale=0) if workload in ("sym4096",) else None
    n_full = {"sym4096": 4096, "sym2p20m16": 1 << 20, "gen2p24k2p16": 1 << 24, "phased3x1024x1024m8": 3 << 20,
              "sym2p30": 1 << 30}[workload]
    scale = 0
    while (n_full >> scale) > (1 << log2_sample):
        scale += 1
    w = full if full is not None else make_workload(workload, scale=scale)
    lib = oracle.load()
    t0 = time.perf_counter()
    reps = 0
    while True:
        if w.kind == "sym":
            oracle.sym_apply(w.a, w.x, lib=lib)
        elif w.kind == "general":
            oracle.general_apply(w.a, w.b, w.x, lib=lib)
        else:
            oracle.phased_apply(w.a, w.phi, w.x, lib=lib)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 1000:
            break
    elems = w.n * w.m * reps
    return {
        "value": elems / dt / 1e9,
        "unit": "Gelem/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%s scaled to n=%d m=%d%s (same distributions), %d run(s) in %.1f s, float64 C oracle incl. its sort" % (
            workload, w.n, w.m, (" k=%d" % w.k) if w.kind == "general" else "", reps, dt),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sym2p30")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-route", action="store_true", help="move x and y by index instead of along the sort route")
    ap.add_argument("--cpu-sample-log2", type=int, default=25)
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import laplace_prefix_scans_amd as lp
    from synth import make_workload

    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    w = make_workload(args.workload)
    t_gen = time.perf_counter() - t_gen
    n, m, k = w.n, w.m, w.k
    use_route = m <= 4 and not args.no_route
    a = torch.from_numpy(w.a).to(dev)
    x = torch.from_numpy(w.x).to(dev)
    ra = lp.route_buffer(n, device=dev) if use_route else None
    a_s = torch.empty_like(a)
    pa = torch.empty(n, dtype=torch.uint32, device=dev)
    ws_sort_a = lp.workspace(lp.LAPLEX_OP_SORT, n, device=dev)
    y = torch.empty((n, m), dtype=torch.float32, device=dev)
    if w.kind == "general":
        b = torch.from_numpy(w.b).to(dev)
        b_s = torch.empty_like(b)
        pb = torch.empty(k, dtype=torch.uint32, device=dev)
        rb = lp.route_buffer(k, device=dev) if use_route else None
        ws_sort_b = lp.workspace(lp.LAPLEX_OP_SORT, k, device=dev)
        ws_apply = lp.workspace(lp.LAPLEX_OP_GENERAL, n, k, m, device=dev)
    elif w.kind == "phased":
        phi = torch.from_numpy(w.phi).to(dev)
        ws_apply = lp.workspace(lp.LAPLEX_OP_PHASED, n, 0, m, device=dev)
    else:
        ws_apply = lp.workspace(lp.LAPLEX_OP_SYM, n, 0, m, device=dev)
    del w.a, w.x

    def step():
        lp.laplex_sort_anchors(a, a_s, pa, route=ra, ws=ws_sort_a)
        if w.kind == "general":
            lp.laplex_sort_anchors(b, b_s, pb, route=rb, ws=ws_sort_b)
            lp.laplex_matvec_general(a_s, pa, b_s, pb, x, y=y, ws=ws_apply, route_a=ra, route_b=rb)
        elif w.kind == "phased":
            lp.laplex_matvec_phased(a_s, pa, phi, x, y=y, ws=ws_apply, route_a=ra)
        else:
            lp.laplex_matvec_sym(a_s, pa, x, y=y, ws=ws_apply, route=ra)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if lp.laplex_status_poll(ws_sort_a) != 0:
        raise RuntimeError("sort reported a device-side error")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with lp.profile_launches(capacity=64 * max(1, args.steps)) as prof:
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # per-kernel statistics from the launch events (each records its element count)
    stats = {}
    for name, ms, units in prof.records:
        s_ = stats.setdefault(name, {"ms": 0.0, "launches": 0, "bytes": 0.0})
        s_["ms"] += ms
        s_["launches"] += 1
        s_["bytes"] += kernel_bytes(name, units, m, k)
    kernels = {}
    for name, s in stats.items():
        avg = s["ms"] / s["launches"]
        bpl = s["bytes"] / s["launches"]
        kernels[name] = {
            "ms_per_step": round(s["ms"] / args.steps, 4),
            "launches_per_step": s["launches"] // args.steps,
            "avg_launch_ms": round(avg, 4),
            "alg_bytes_per_launch": bpl,
            "alg_GBps": round(bpl / (avg * 1e-3) / 1e9, 1) if avg > 0 else None,
        }
    dom = max(stats, key=lambda q: stats[q]["ms"])
    dk = kernels[dom]
    src = source_hash()
    traffic, traffic_src = load_traffic(args.workload, dom, src)
    achieved = dk["alg_GBps"]
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": achieved,
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4) if achieved else None,
        "traffic": traffic,
        "alg_bytes_per_launch": dk["alg_bytes_per_launch"],
        "avg_launch_ms": dk["avg_launch_ms"],
    }
    step_bytes = sum(s["bytes"] for s in stats.values()) / args.steps
    line = {
        "metric": METRIC,
        "value": round(n * m / (ms_per_step * 1e-3) / 1e9, 4),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "kind": w.kind, "n": n, "m": m, "k": k if w.kind == "general" else None,
                   "step": "sort + apply", "route": use_route, "recipe": w.recipe},
        "roofline": roofline,
        "step_alg_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "kernels": kernels,
        "source_hash": src,
        "host_gen_s": round(t_gen, 1),
    }
    if args.calib_copy:
        src_t = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst_t = torch.empty_like(src_t)
        for _ in range(3):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        line["calib_copy_bytes_each_way"] = 1 << 30
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_sample_log2)
    print(json.dumps(line))


if __name__ == "__main__":
    main()

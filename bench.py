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


# sources of the memory-system probes, which are not operator kernels
PROBE_SOURCES = ("laplex_probe.hip",)


def source_hash() -> str:
    """Hash of the operator's kernel sources (the probes excluded), stamped on
    each profile so that counters taken on other kernels are not used."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp")) and f not in PROBE_SOURCES:
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


SMALL_SORT_MAX = 1 << 17              # sorts of at most this many keys use 2048-key tiles, larger ones 8192


def sort_tile(n: int) -> int:
    return 2048 if n <= SMALL_SORT_MAX else 8192


def route_bytes_per_elem(n: int) -> float:
    """Per element per routed pass: a u16 tile-local position, plus u16 run
    starts and u32 run positions (256 digits) per tile."""
    return 2.0 + 1536.0 / sort_tile(n)


def kernel_bytes(name: str, units: int, m: int, k: int = 0) -> float:
    """Algorithmic bytes of one launch: every array the kernel must touch, once,
    at its useful size (a random row access counts its 4m useful bytes).
    ``units`` = elements (rows) the launch processes; ``k`` = input anchors of
    the general operator.  A sort pass moves 16 bytes per key (key and value
    in and out; 12 in the first pass, which makes the indices), the figures of
    the planned byte model; the route a pass records and the route passes
    that move rows along it are bookkeeping, counted by overhead_bytes."""
    table = {
        "k_sort_hist": 4.0,                      # read anchors
        "k_onesweep_first": 12.0,                # read anchors; write keys and indices
        "k_onesweep_mid": 16.0,                  # read and write key + value
        "k_onesweep_last": 16.0,
        "k_onesweep_first_routed": 12.0,
        "k_onesweep_mid_routed": 16.0,
        "k_onesweep_last_routed": 16.0,
        "k_onesweep_first_pay": 16.0,            # read anchors and x; write keys and x
        "k_onesweep_last_pay": 16.0,             # read key + x; write sorted anchors and sorted x
        "k_onesweep_first_pay_routed": 16.0,
        "k_onesweep_last_pay_routed": 16.0,
        "k_sym_apply": 8.0 + 8.0 * m,            # sorted anchors, perm, sorted rows in, y rows out (random)
        "k_sym_reduce": 4.0 + 4.0 * m,           # sorted anchors, sorted rows
        "k_sym_apply_sorted": 4.0 + 8.0 * m,     # sorted anchors, sorted rows in, sorted rows out
        "k_sym_fu": 4.0 + 12.0 * m,              # sorted anchors and rows in; both scans out
        "k_phased_apply": 12.0 + 8.0 * m,
        "k_phased_reduce": 8.0 + 4.0 * m,
        "k_phased_apply_sorted": 8.0 + 8.0 * m,
        "k_gather_rows": 4.0 + 8.0 * m,          # perm, rows in (random), sorted rows out
        "k_gather_rows_ph": 12.0 + 8.0 * m,      # the same plus the phases
        "k_gen_reduce": 4.0 + 4.0 * m,
        "k_phased_gen_reduce": 8.0 + 4.0 * m,
        "k_bwd_reduce": 4.0 + 8.0 * m,           # sorted anchors, sorted x and g rows
        "k_bwd_apply": 8.0 + 12.0 * m,           # sorted anchors, x and g rows in; dx rows and da out
        "k_scatter_rows": 4.0 + 8.0 * m,         # perm, sorted rows in, rows out (random)
        "k_scatter_rows2": 12.0 + 8.0 * m,       # the same plus one float per row (da) in and out
        "k_scatter_rows3": 20.0 + 8.0 * m,       # the same plus two floats per row (da, dphi)
        "k_gather_rows2": 4.0 + 16.0 * m,        # perm, x and g rows in (random), sorted rows out
        "k_gather_rows2_ph": 12.0 + 16.0 * m,    # the same plus the phases
        "k_gbwd_reduce": 4.0 + 4.0 * m,          # merged anchors, x rows (at b) and g rows (at a)
        "k_pbwd_reduce": 8.0 + 8.0 * m,          # sorted anchors and phases, x and g rows
        "k_pbwd_apply": 16.0 + 12.0 * m,         # anchors, phases, x and g rows in; dx rows, da, dphi out
        "k_gram_fill": 4.0,                      # per entry of M: written once (row/column families are O(n))
        "k_gram_families": 8.0,                  # merged anchors and weights in; families out at a (20 B per a)
        "k_gram_double": 8.0,                    # anchors in and doubled anchors out
        "k_gram_dprefix": 12.0,                  # sorted weights in, float64 prefix out
    }
    for w in (1, 2, 3, 4):
        table["k_route_fwd_w%d" % w] = 8.0 * w   # row in, row out
        table["k_route_inv_w%d" % w] = 8.0 * w
    if name in table:
        return table[name] * units
    if name == "k_gbwd_apply":  # merged anchors, x and g rows in; da (n), db and dx rows (k) out
        return (8.0 + 4.0 * m) * units + 4.0 * m * k
    if name == "k_gen_search":  # outputs' anchors in, y rows out; sorted b and both scans read once
        return (4.0 + 4.0 * m) * units + (4.0 + 8.0 * m) * k
    if name in ("k_gen_apply", "k_phased_gen_apply"):
        return (8.0 + 4.0 * m) * units + (4.0 + 4.0 * m) * k
    if name in ("k_gen_apply_sorted", "k_phased_gen_apply_sorted"):
        return (4.0 + 4.0 * m) * units + (4.0 + 4.0 * m) * k
    return 0.0


def overhead_bytes(name: str, units: int) -> float:
    """Route bookkeeping of one launch: the positions and run tables a routed
    sort pass writes, or a route pass reads, per element of the sort."""
    if name.startswith(("k_route_fwd", "k_route_inv")) or (name.startswith("k_onesweep") and name.endswith("_routed")):
        return route_bytes_per_elem(units) * units
    return 0.0


def model_step_bytes(kind: str, n: int, m: int, k: int) -> dict:
    """Bytes one step must move by the planned byte model, whatever kernels
    run: the sort 64 B per anchor (histogram 4, first pass 12, three passes of
    16) and the apply (symmetric 16 + 28m per anchor: gather 4 + 8m, forward
    scan 4 + 8m, suffix scan with combine and scatter 8 + 12m; phased
    32 + 36m; general with sparse injections 24 per output anchor + O(k))."""
    if kind == "sym":
        sort, apply_ = 64.0 * n, (16.0 + 28.0 * m) * n
    elif kind == "phased":
        sort, apply_ = 64.0 * n, (32.0 + 36.0 * m) * n
    elif kind == "general":
        sort, apply_ = 64.0 * (n + k), 24.0 * n + (4.0 + 8.0 * m) * k
    else:
        return {}
    return {"sort": sort, "apply": apply_, "step": sort + apply_}


# rocprofv3 kernel names (template arguments stripped) -> launch labels
ROCPROF_LABELS = {
    "k_sort_hist": "k_sort_hist",
    "k_sort_offsets": "k_sort_offsets",
    "k_fill_u32": "k_fill_u32",
    "k_tile_carry": "k_tile_carry",
    "k_gather_rows": "k_gather_rows",
}


def rocprof_label(name: str, pass_index: int = 0, routed: bool = True) -> str:
    import re
    if "at::native::" in name:  # torch's own kernels (input fills in the timed program): name the functor
        fm = re.search(r"(\w*Functor)", name) or re.search(r"at::native::(?:\w+::)*(\w+)", name)
        return "torch_" + (fm.group(1) if fm else "kernel")
    base = re.sub(r"\(.*$", "", name).replace("void ", "").replace("laplex::", "").strip()
    m = re.match(r"(k_\w+)<(.*)>$", base)
    kern, targs = (m.group(1), [t.strip() for t in m.group(2).split(",")]) if m else (base, [])
    if kern == "k_onesweep":
        label = {"0": "k_onesweep_first", "1": "k_onesweep_mid", "2": "k_onesweep_last"}[targs[0]]
        pay = len(targs) > 2 and targs[2] == "true"
        return label + ("_pay" if pay else "") + ("_routed" if routed else "")
    if kern in ("k_route_fwd", "k_route_inv", "k_route_inv_chunked"):
        return "%s_w%s" % (kern.replace("_chunked", ""), targs[0])
    if kern == "k_sym_reduce":
        return "k_phased_reduce" if targs[1] == "true" else "k_sym_reduce"
    if kern == "k_sym_apply":
        ph, scatter = targs[1] == "true", targs[2] == "true"
        return ("k_phased_apply" if ph else "k_sym_apply") + ("" if scatter else "_sorted")
    if kern == "k_gen_reduce":
        return "k_phased_gen_reduce" if targs[1] == "true" else "k_gen_reduce"
    if kern == "k_gen_apply":
        ph, scatter = targs[1] == "true", targs[2] == "true"
        return ("k_phased_gen_apply" if ph else "k_gen_apply") + ("" if scatter else "_sorted")
    return ROCPROF_LABELS.get(kern, kern)


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
    fetch_kib, write_kib = rows[kernel]
    fetch_factor = float(meta.get("fetch_factor", "1.0"))
    write_factor = float(meta.get("write_factor", "1.0"))
    return (fetch_kib * fetch_factor + write_kib * write_factor) * 1024.0, path


def rocprof_summary(stats_csv: str, fetch_csv: str, write_csv: str, workload: str, command: str) -> str:
    """Text summaries of a rocprofv3 kernel-trace --stats run and of two --pmc runs
    (FETCH_SIZE, WRITE_SIZE).  The counters are scaled by what they read for the
    plain 1 GiB device copy the benchmark runs with --calib-copy."""
    import csv
    out = []
    out.append("# rocprofv3 kernel statistics, workload %s" % workload)
    out.append("# command: rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- %s" % command)
    out.append("# source_hash = %s" % source_hash())
    out.append("# %-26s %6s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us"))
    from synth import WORKLOADS
    # the sort records its route exactly when the benchmark moves rows along it
    routed = WORKLOADS[workload][1] != "gram" and workload not in ("sym2p20m16", "phased3x1024x1024m8")
    agg = {}
    for r in csv.DictReader(open(stats_csv)):
        lab = rocprof_label(r["Name"], routed=routed)
        a = agg.setdefault(lab, [0, 0.0, float("inf"), 0.0])
        calls = int(r["Calls"])
        a[0] += calls
        a[1] += float(r["TotalDurationNs"])
        a[2] = min(a[2], float(r["MinNs"]))
        a[3] = max(a[3], float(r["MaxNs"]))
    for lab, (c, tot, mn, mx) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        out.append("%-28s %6d %12.1f %12.1f %12.1f" % (lab, c, tot / c / 1e3, mn / 1e3, mx / 1e3))
    kernels_txt = "\n".join(out) + "\n"

    def per_dispatch(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
    write = per_dispatch(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)  # 1 GiB in KiB
    copy_f = [v for k, vs in fetch.items() if "copyBuffer" in k for v in vs]
    copy_w = [v for k, vs in write.items() if "copyBuffer" in k for v in vs]
    fetch_factor = gib_kib / max(copy_f) if copy_f else 1.0
    write_factor = gib_kib / max(copy_w) if copy_w else 1.0
    c = []
    c.append("# rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch, mean over dispatches), workload %s" % workload)
    c.append("# commands: rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- %s" % command)
    c.append("#           rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- %s" % command)
    c.append("# calibration: a plain device copy of 1 GiB (bench.py --calib-copy) reads FETCH_SIZE %.0f KiB and"
             " WRITE_SIZE %.0f KiB" % (max(copy_f) if copy_f else 0, max(copy_w) if copy_w else 0))
    c.append("# fetch_factor = %.4f" % fetch_factor)
    c.append("# write_factor = %.4f" % write_factor)
    c.append("# source_hash = %s" % source_hash())
    c.append("# %-26s %14s %14s   (raw counter values; bytes = KiB * 1024 * factor)" % ("kernel", "FETCH_KiB", "WRITE_KiB"))
    lab_f, lab_w = {}, {}
    for k, vs in fetch.items():
        lab_f.setdefault(rocprof_label(k, routed=routed), []).extend(vs)
    for k, vs in write.items():
        lab_w.setdefault(rocprof_label(k, routed=routed), []).extend(vs)
    for lab in sorted(lab_f, key=lambda q: -sum(lab_f[q]) / len(lab_f[q])):
        if "copyBuffer" in lab:
            continue
        fv = sum(lab_f[lab]) / len(lab_f[lab])
        wv = sum(lab_w.get(lab, [0.0])) / max(1, len(lab_w.get(lab, [0.0])))
        c.append("%-28s %14.1f %14.1f" % (lab, fv, wv))
    return kernels_txt, "\n".join(c) + "\n"


def host_info() -> dict:
    """Host cores, CPU model and available memory, for the CPU baseline."""
    info = {"nproc": os.cpu_count()}
    try:
        info["affinity_cores"] = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable"):
                    info["mem_available_GB"] = round(int(line.split()[1]) / 2 ** 20, 1)
    except OSError:
        pass
    return info


def cpu_baseline(workload: str, log2_sample: int):
    """The float64 oracle on a bounded sample of the workload: on all host
    cores (the OpenMP oracle, symmetric operator) and on one core (the
    sequential C oracle, every operator), each repeated for about 10 s."""
    import oracle
    from synth import make_workload

    full = make_workload(workload, scale=0) if workload in ("sym4096",) else None
    n_full = {"sym4096": 4096, "sym2p20m16": 1 << 20, "gen2p24k2p16": 1 << 24, "phased3x1024x1024m8": 3 << 20,
              "sym2p30": 1 << 30, "gram2p16k2p16": 1 << 16}[workload]
    if workload == "gram2p16k2p16":
        log2_sample = min(log2_sample, 12)  # the oracle's Gram is the O(n^2 k) definition
    scale = 0
    while (n_full >> scale) > (1 << log2_sample):
        scale += 1
    w = full if full is not None else make_workload(workload, scale=scale)
    lib = oracle.load()
    from threadpoolctl import threadpool_limits

    def timed(fn):
        t0 = time.perf_counter()
        reps = 0
        while True:
            fn()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or reps >= 1000:
                return reps, dt

    with threadpool_limits(limits=1):  # one core for the sequential leg (NumPy's BLAS in the Gram one)
        if w.kind == "sym":
            reps, dt = timed(lambda: oracle.sym_apply(w.a, w.x, lib=lib))
        elif w.kind == "general":
            reps, dt = timed(lambda: oracle.general_apply(w.a, w.b, w.x, lib=lib))
        elif w.kind == "gram":
            reps, dt = timed(lambda: oracle.gram_dense(w.a, w.b, w.D))
        else:
            reps, dt = timed(lambda: oracle.phased_apply(w.a, w.phi, w.x, lib=lib))
    elems = (w.n * w.n if w.kind == "gram" else w.n * w.m)
    what = ("float64 dense definition of A diag(D) A^T (NumPy, one BLAS thread)" if w.kind == "gram"
            else "float64 C oracle incl. its sort")
    sample = "%s scaled to n=%d m=%d%s (same distributions)" % (
        workload, w.n, w.m, (" k=%d" % w.k) if w.kind in ("general", "gram") else "")
    single = {"value": elems * reps / dt / 1e9, "unit": "Gelem/s", "cores": 1, "kind": "oracle",
              "sample": "%s, %d run(s) in %.1f s, %s" % (sample, reps, dt, what)}
    if w.kind != "sym":
        single["note"] = "the all-cores oracle covers the symmetric operator; this workload's baseline is one core"
        single["host"] = host_info()
        return single
    threads = oracle.par_threads()
    reps_p, dt_p = timed(lambda: oracle.sym_apply_par(w.a, w.x))
    return {"value": elems * reps_p / dt_p / 1e9, "unit": "Gelem/s", "cores": threads, "kind": "oracle",
            "sample": "%s, %d run(s) in %.1f s, float64 OpenMP oracle incl. its sort (merge sort split among the "
                      "threads, chunked two-pass scan)" % (sample, reps_p, dt_p),
            "single_core": single, "host": host_info()}


STEP_TARGET_FRAC = 0.60  # sustained fraction of peak HBM bandwidth the n = 2^30 symmetric step is held to


def step_model(kind: str, n: int, m: int, k: int, ms: float):
    """The step against the planned byte model: its bytes over the measured
    step time, as a fraction of peak, beside the 60 % target."""
    b = model_step_bytes(kind, n, m, k)
    if not b:
        return None
    gbps = b["step"] / (ms * 1e-3) / 1e9
    return {"bytes_per_step": b["step"], "sort_bytes": b["sort"], "apply_bytes": b["apply"],
            "achieved_GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4), "target_frac": STEP_TARGET_FRAC,
            "roofline_ms": round(b["step"] / (HBM_PEAK_GBPS * 1e9) * 1e3, 4)}


def time_call(lp, torch, bstep, n, m, k, args):
    """A call `bstep` other than the step (the backward for a seeded upstream
    gradient, or the apply alone given a sort handle): its own timed loop,
    reported beside the step."""
    for _ in range(args.warmup):
        bstep()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with lp.profile_launches(capacity=64 * max(1, args.steps)) as prof:
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            bstep()
        e1.record()
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    kern_ms, kern_bytes = 0.0, 0.0
    per = {}
    for name, kms, units in prof.records:
        b = kernel_bytes(name, units, m, k)
        kern_ms += kms
        kern_bytes += b
        r = per.setdefault(name, [0.0, 0, 0.0])
        r[0] += kms
        r[1] += 1
        r[2] += b
    kern_ms /= args.steps
    kern_bytes /= args.steps
    gbps = kern_bytes / (kern_ms * 1e-3) / 1e9 if kern_ms > 0 else None
    kernels = {name: {"ms_per_call": round(v[0] / args.steps, 4), "launches_per_call": v[1] // args.steps,
                      "alg_GBps": round(v[2] / (v[0] * 1e-3) / 1e9, 1) if v[0] > 0 else None}
               for name, v in per.items()}
    return {"ms_per_call": round(ms, 4), "kernel_ms": round(kern_ms, 4), "alg_GB": round(kern_bytes / 1e9, 3),
            "alg_GBps": round(gbps, 1) if gbps else None,
            "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4) if gbps else None,
            "Gelem_per_s": round(n * m / (ms * 1e-3) / 1e9, 4), "kernels": kernels}


def micro(args):
    """Memory-system rates behind the choice between moving rows by index and
    moving them along the sort's route, on arrays of 2^30 floats (4 GiB):
    a streaming copy, a random 4-byte gather y = x[p] and scatter y[p] = x
    for a uniformly random permutation p (the order a sort of iid anchors
    produces), and random 64-byte rows (16 floats) gathered by index, each by
    torch's kernels; then the probe library's streaming patterns.  Each is
    timed with HIP events over repeated launches."""
    import torch
    n = 1 << 30
    dev = torch.device("cuda:0")
    x = torch.randn(n, device=dev)
    y = torch.empty_like(x)
    g = torch.Generator(device=dev).manual_seed(11)
    p = torch.randperm(n, device=dev, generator=g)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {}
    ms = timed(lambda: y.copy_(x))
    out["copy"] = {"ms": round(ms, 3), "GBps": round(2 * 4 * n / (ms * 1e-3) / 1e9, 1), "bytes": "4 B read + 4 B written per element"}
    ms = timed(lambda: torch.index_select(x, 0, p, out=y))
    out["gather_4B"] = {"ms": round(ms, 3), "useful_GBps": round(2 * 4 * n / (ms * 1e-3) / 1e9, 1),
                        "bytes": "4 B read at random + 4 B written per element (index reads not counted)"}
    ms = timed(lambda: y.index_copy_(0, p, x))
    out["scatter_4B"] = {"ms": round(ms, 3), "useful_GBps": round(2 * 4 * n / (ms * 1e-3) / 1e9, 1),
                         "bytes": "4 B read + 4 B written at random per element (index reads not counted)"}
    del p
    rows = n // 16
    x2, y2 = x.view(rows, 16), y.view(rows, 16)
    pr = torch.randperm(rows, device=dev, generator=g)
    ms = timed(lambda: torch.index_select(x2, 0, pr, out=y2))
    out["gather_64B_rows"] = {"ms": round(ms, 3), "useful_GBps": round(2 * 4 * n / (ms * 1e-3) / 1e9, 1),
                              "bytes": "64-byte rows read at random + written in order"}
    # the streaming patterns of liblaplex_probe.so (include/laplex_probe.h),
    # each over the same 4 GiB: two copy shapes, a read, a write, and one
    # radix pass's data movement (8192-pair tiles into 256 regions) without
    # its ranking
    import ctypes
    probe_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "laplace_prefix_scans_amd", "liblaplex_probe.so")
    if not os.path.exists(probe_path):
        raise RuntimeError("liblaplex_probe.so is not built (python -m laplace_prefix_scans_amd.build)")
    probe = ctypes.CDLL(probe_path)
    probe.laplex_probe.restype = ctypes.c_int
    probe.laplex_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    nbytes = 4 * n

    def run_probe(kind):
        rc = probe.laplex_probe(kind, x.data_ptr(), y.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError("laplex_probe(%d) returned %d" % (kind, rc))

    for kind, name, moved, what in ((0, "probe_copy_1", 2, "copy, one 16-byte piece per thread, 4 KiB per workgroup, per-XCD ranges"),
                                    (1, "probe_copy_8", 2, "copy, eight 16-byte pieces per thread, 32 KiB per workgroup"),
                                    (2, "probe_read", 1, "read, one 16-byte piece per thread"),
                                    (3, "probe_write", 1, "write, one 16-byte piece per thread"),
                                    (4, "probe_runs", 2, "8192-pair tiles read whole, written as 256 runs of 256 bytes")):
        ms = timed(lambda: run_probe(kind))
        out[name] = {"ms": round(ms, 3), "GBps": round(moved * nbytes / (ms * 1e-3) / 1e9, 1), "bytes": what}
    print(json.dumps({"micro": out, "n_floats": n, "peak_GBps": HBM_PEAK_GBPS}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sym2p30")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-route", action="store_true", help="move x and y by index instead of along the sort route")
    ap.add_argument("--two-call", action="store_true",
                    help="time the sort handles + laplex_matvec_sym / laplex_matvec_general instead of the one-call "
                         "laplex_sort_matvec_sym (symmetric, m = 1: x carried through the sort) or "
                         "laplex_sort_matvec_general (general: only b sorted, outputs search their interval)")
    ap.add_argument("--cpu-sample-log2", type=int, default=25)
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward (symmetric, general, phased)")
    ap.add_argument("--no-apply-only", action="store_true", help="skip timing the apply alone given a sort handle")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache timing (steps after a 512 MiB scrub)")
    ap.add_argument("--no-graph", action="store_true", help="skip timing the step replayed from a HIP graph")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--rocprof-summary", nargs=3, metavar=("STATS_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/kernels_<workload>.txt and profiles/counters_<workload>.txt from rocprofv3 output")
    ap.add_argument("--rocprof-command", default="", help="the program command line the rocprofv3 runs profiled")
    ap.add_argument("--micro", action="store_true",
                    help="print the memory-system micro-benchmark (copy, random gather and scatter) and exit")
    args = ap.parse_args()
    if args.micro:
        micro(args)
        return
    if args.rocprof_summary:
        ktxt, ctxt = rocprof_summary(*args.rocprof_summary, workload=args.workload, command=args.rocprof_command)
        os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
        with open(os.path.join(ROOT, "profiles", "kernels_%s.txt" % args.workload), "w") as f:
            f.write(ktxt)
        with open(os.path.join(ROOT, "profiles", "counters_%s.txt" % args.workload), "w") as f:
            f.write(ctxt)
        print(ktxt + ctxt)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (got --gpus %d)" % args.gpus,
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
    # symmetric, one column, routed: the sort and the apply in one call, x
    # carried through the sort's passes as the keys' values
    one_call = w.kind == "sym" and m == 1 and use_route and not args.two_call
    # general: only b sorted, the scans over b, each output searching its interval
    one_call_gen = w.kind == "general" and not args.two_call
    a = torch.from_numpy(w.a).to(dev)
    x = torch.from_numpy(w.x).to(dev)
    # the sort handle of a (the one-call path keeps its own in its workspace)
    ra = lp.route_buffer(n, device=dev) if use_route and not one_call else None
    a_s = torch.empty_like(a) if not one_call else None
    pa = torch.empty(n, dtype=torch.uint32, device=dev) if not one_call else None
    ws_sort_a = lp.workspace(lp.LAPLEX_OP_SORT, n, device=dev) if not one_call else None
    y = torch.empty((n, m), dtype=torch.float32, device=dev) if w.kind != "gram" else None
    if w.kind == "gram":
        b = torch.from_numpy(w.b).to(dev)
        Dw = torch.from_numpy(w.D).to(dev)
        b_s = torch.empty_like(b)
        pb = torch.empty(k, dtype=torch.uint32, device=dev)
        rb = None
        ws_sort_b = lp.workspace(lp.LAPLEX_OP_SORT, k, device=dev)
        ws_apply = lp.workspace(lp.LAPLEX_OP_GRAM, n, k, 1, device=dev)
        Mg = torch.empty((n, n), dtype=torch.float32, device=dev)
        ra = None
    elif w.kind == "general":
        b = torch.from_numpy(w.b).to(dev)
        b_s = torch.empty_like(b)
        pb = torch.empty(k, dtype=torch.uint32, device=dev)
        rb = lp.route_buffer(k, device=dev) if use_route else None
        ws_sort_b = lp.workspace(lp.LAPLEX_OP_SORT, k, device=dev)
        ws_apply = lp.workspace(lp.LAPLEX_OP_SORT_GENERAL if one_call_gen else lp.LAPLEX_OP_GENERAL, n, k, m, device=dev)
    elif w.kind == "phased":
        phi = torch.from_numpy(w.phi).to(dev)
        ws_apply = lp.workspace(lp.LAPLEX_OP_PHASED, n, 0, m, device=dev)
    elif one_call:
        ws_apply = lp.workspace(lp.LAPLEX_OP_SORT_SYM, n, 0, m, device=dev)
    else:
        ws_apply = lp.workspace(lp.LAPLEX_OP_SYM, n, 0, m, device=dev)
    del w.a, w.x

    def step():
        if one_call:
            lp.laplex_sort_matvec_sym(a, x, y=y, ws=ws_apply)
            return
        if one_call_gen:
            lp.laplex_sort_matvec_general(a, b, x, y=y, ws=ws_apply)
            return
        lp.laplex_sort_anchors(a, a_s, pa, route=ra, ws=ws_sort_a)
        if w.kind == "gram":
            lp.laplex_sort_anchors(b, b_s, pb, ws=ws_sort_b)
            lp.laplex_gram_weighted(a_s, pa, b_s, pb, Dw, M=Mg, ws=ws_apply)
        elif w.kind == "general":
            lp.laplex_sort_anchors(b, b_s, pb, route=rb, ws=ws_sort_b)
            lp.laplex_matvec_general(a_s, pa, b_s, pb, x, y=y, ws=ws_apply, route_a=ra, route_b=rb)
        elif w.kind == "phased":
            lp.laplex_matvec_phased(a_s, pa, phi, x, y=y, ws=ws_apply, route_a=ra)
        else:
            lp.laplex_matvec_sym(a_s, pa, x, y=y, ws=ws_apply, route=ra)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if lp.laplex_status_poll(ws_apply if one_call or one_call_gen else ws_sort_a) != 0:
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

    # cold caches: each step timed alone after writing a 512 MiB scrub buffer
    # (larger than the L2s and the 256 MiB Infinity Cache); for workloads whose
    # working set could stay cached between steps
    cold = None
    if not args.no_cold and n * max(1, m) <= (1 << 26):
        scrub = torch.empty(1 << 27, dtype=torch.float32, device=dev)
        times = []
        for i in range(max(3, min(args.steps, 10))):
            scrub.fill_(float(i))
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            step()
            c1.record()
            torch.cuda.synchronize()
            times.append(c0.elapsed_time(c1))
        del scrub
        cold = {"ms_per_step_median": round(float(sorted(times)[len(times) // 2]), 4), "steps": len(times),
                "scrub_MiB": 512}

    # the same step captured once in a HIP graph and replayed: no host launch
    # cost between kernels (for workloads small enough for that to matter)
    graph = None
    if not args.no_graph and n * max(1, m) <= (1 << 26):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            step()
        for _ in range(max(1, args.warmup)):
            cg.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            cg.replay()
        g1.record()
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        graph = {"ms_per_step": round(gms, 4), "Gelem_per_s": round(n * m / (gms * 1e-3) / 1e9, 4) if w.kind != "gram"
                 else round(n * n / (gms * 1e-3) / 1e9, 4), "replays": args.steps}
        del cg

    # per-kernel statistics from the launch events (each records its element count)
    stats = {}
    for name, ms, units in prof.records:
        s_ = stats.setdefault(name, {"ms": 0.0, "launches": 0, "bytes": 0.0, "over": 0.0})
        s_["ms"] += ms
        s_["launches"] += 1
        s_["bytes"] += kernel_bytes(name, units, m, k)
        s_["over"] += overhead_bytes(name, units)
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
            "overhead_bytes_per_launch": s["over"] / s["launches"],
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
        # route bookkeeping the launch also moves (not algorithmic)
        "overhead_bytes_per_launch": dk["overhead_bytes_per_launch"],
    }
    step_bytes = sum(s["bytes"] for s in stats.values()) / args.steps

    # the step split into its sort (row a1) and its apply (rows a2-a7, given
    # the sort handle): kernel time and algorithmic bytes of each part (on the
    # one-call path the sort passes also carry x into sorted order, row a2)
    def part(names):
        ms = sum(stats[q]["ms"] for q in names) / args.steps
        by = sum(stats[q]["bytes"] for q in names) / args.steps
        gbps = by / (ms * 1e-3) / 1e9 if ms > 0 else None
        return {"kernel_ms": round(ms, 4), "alg_GB": round(by / 1e9, 3), "alg_GBps": round(gbps, 1) if gbps else None,
                "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4) if gbps else None,
                "Gelem_per_s": round(out_elems / (ms * 1e-3) / 1e9, 4) if ms > 0 else None}
    sort_names = [q for q in stats if q.startswith(("k_sort", "k_onesweep", "k_fill"))]
    apply_names = [q for q in stats if q not in sort_names]
    out_elems = n * n if w.kind == "gram" else n * m
    line = {
        "metric": METRIC,
        "value": round(out_elems / (ms_per_step * 1e-3) / 1e9, 4),
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
        "config": {"workload": args.workload, "kind": w.kind, "n": n, "m": m,
                   "k": k if w.kind in ("general", "gram") else None,
                   "step": "sort a and b + all n^2 entries of M" if w.kind == "gram" else
                   "sort + apply in one call (x carried through the sort)" if one_call else
                   "sort of b + apply in one call (scans over b, each output searches its interval)" if one_call_gen
                   else "sort + apply",
                   "route": use_route and w.kind != "gram", "recipe": w.recipe},
        "roofline": roofline,
        "step_alg_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_model": step_model(w.kind, n, m, k, ms_per_step),
        "sort_part": part(sort_names),
        "apply_part": part(apply_names),
        "kernels": kernels,
        "cold": cold,
        "graph": graph,
        "source_hash": src,
        "host_gen_s": round(t_gen, 1),
    }
    if w.kind in ("sym", "general", "phased") and not args.no_backward:
        if one_call_gen:  # the backward takes sort handles of a and b: build them (untimed)
            lp.laplex_sort_anchors(a, a_s, pa, route=ra, ws=ws_sort_a)
            lp.laplex_sort_anchors(b, b_s, pb, route=rb, ws=ws_sort_b)
        gen = torch.Generator(device=dev).manual_seed(0x6AAD)
        g = torch.randn((n,) if x.dim() == 1 else (n, m), generator=gen, device=dev)
        da = torch.empty(n, dtype=torch.float32, device=dev)
        dx = torch.empty_like(x)
        if w.kind == "sym" and one_call:
            # the backward of the timed one-call forward, from what it left
            # in its workspace (sorted anchors, route, x in sorted order)
            ws_b = lp.workspace(lp.LAPLEX_OP_SYM_BACKWARD, n, 0, m, device=dev)

            def bstep():
                lp.laplex_sort_matvec_sym_backward(ws_apply, g, dx=dx, da=da, ws=ws_b)
            what = "dx = K g and da, from g and the one-call forward's workspace"
        elif w.kind == "sym":
            ws_b = lp.workspace(lp.LAPLEX_OP_SYM_BACKWARD, n, 0, m, device=dev)

            def bstep():
                lp.laplex_backward_sym(a_s, pa, x, g, dx=dx, da=da, ws=ws_b, route=ra)
            what = "dx = K g and da, from x and g"
        elif w.kind == "phased":
            ws_b = lp.workspace(lp.LAPLEX_OP_PHASED_BACKWARD, n, 0, m, device=dev)
            dphi = torch.empty(n, dtype=torch.float32, device=dev)

            def bstep():
                lp.laplex_backward_phased(a_s, pa, phi, x, g, dx=dx, da=da, dphi=dphi, ws=ws_b, route=ra)
            what = "dx = W g, da and dphi, from x and g"
        else:
            ws_b = lp.workspace(lp.LAPLEX_OP_GENERAL_BACKWARD, n, k, m, device=dev)
            db = torch.empty(k, dtype=torch.float32, device=dev)

            def bstep():
                lp.laplex_backward_general(a_s, pa, b_s, pb, x, g, dx=dx, da=da, db=db, ws=ws_b, route_a=ra,
                                           route_b=rb)
            what = "dx = K^T g, da and db, from x and g"
        line["backward_part"] = time_call(lp, torch, bstep, n, m, k, args)
        line["backward_part"]["outputs"] = what
        del ws_b
    if w.kind in ("sym", "general", "phased") and not args.no_apply_only:
        # the apply alone, given sort handles built beforehand (untimed): the
        # figure for callers that sort once and apply many times
        if one_call or one_call_gen:
            del ws_apply
            torch.cuda.empty_cache()
            ra = lp.route_buffer(n, device=dev) if use_route else None
            a_s, pa = torch.empty_like(a), torch.empty(n, dtype=torch.uint32, device=dev)
            ws_sort_a = lp.workspace(lp.LAPLEX_OP_SORT, n, device=dev)
        lp.laplex_sort_anchors(a, a_s, pa, route=ra, ws=ws_sort_a)
        if w.kind == "general":
            lp.laplex_sort_anchors(b, b_s, pb, route=rb, ws=ws_sort_b)
            ws_ap = lp.workspace(lp.LAPLEX_OP_GENERAL, n, k, m, device=dev)

            def astep():
                lp.laplex_matvec_general(a_s, pa, b_s, pb, x, y=y, ws=ws_ap, route_a=ra, route_b=rb)
        elif w.kind == "phased":
            ws_ap = lp.workspace(lp.LAPLEX_OP_PHASED, n, 0, m, device=dev)

            def astep():
                lp.laplex_matvec_phased(a_s, pa, phi, x, y=y, ws=ws_ap, route_a=ra)
        else:
            ws_ap = lp.workspace(lp.LAPLEX_OP_SYM, n, 0, m, device=dev)

            def astep():
                lp.laplex_matvec_sym(a_s, pa, x, y=y, ws=ws_ap, route=ra)
        torch.cuda.synchronize()
        del ws_sort_a
        ap = time_call(lp, torch, astep, n, m, k, args)
        mb = model_step_bytes(w.kind, n, m, k)["apply"]
        gbps = mb / (ap["ms_per_call"] * 1e-3) / 1e9
        ap["model_bytes"] = mb
        ap["model_GBps"] = round(gbps, 1)
        ap["model_frac"] = round(gbps / HBM_PEAK_GBPS, 4)
        ap["what"] = "y = K x given the sort handle%s" % (" and its route" if use_route else "")
        line["apply_only"] = ap
        del ws_ap
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

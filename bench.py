"""Benchmark: one full exact DBSCAN fit per step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

A step is the whole path on one synthetic point set already resident in
HBM: ingest/layout, the all-pairs neighbour-count pass, core flags, the
union-find merge with border assignment, and canonical labels.  The
default workload is the 1,000,000-point, 3-d set (200 Gaussian blobs, 100
random walks, 10% uniform noise; eps 0.003, MinPts 16).

Prints one JSON line.  `value` is ordered pair evaluations per second of
whole fits (N^2 per fit / wall time of the timed fits).  `roofline` is for
the dominant kernel, the count pass: its algorithmic FP32 work (3d
operations per ordered pair: d subtractions, d multiplications, d-1
additions, 1 comparison) over its average duration measured with HIP events
recorded by the library on the fit's stream, against the MI355X fp32 vector
peak.  `per_config` times the same fit on each of the other four workloads
(full fit, count pass, merge, roofline fractions, parity against the
oracle's digests).  `pcie_inclusive` times the host-array entry (device
allocation, copies in and out) on the same workload; it is never `value`.
`cpu_baseline` times the brute-force oracle in a child process on the
host's cores (OpenMP threads one per physical core, bound with
OMP_PLACES=cores and OMP_PROC_BIND=spread) on a bounded sample of the same
workload (its first M points), and names the host CPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 vector peak (packed FMA counted)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--max-edges", type=int, default=1 << 30)
    ap.add_argument("--tile-merge", action="store_true",
                    help="force the second tile pass instead of the edge list")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target length of the oracle sample run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--prune", action="store_true",
                    help="time the exact tile-pruned fit as the main line")
    ap.add_argument("--screen", action="store_true",
                    help="time the screened count pass as the main line")
    ap.add_argument("--no-screen-line", action="store_true",
                    help="skip the screen_mode measurements")
    ap.add_argument("--no-graph-line", action="store_true",
                    help="skip the sparse eps-graph export leg")
    ap.add_argument("--no-pruned-line", action="store_true",
                    help="skip the extra pruned_mode measurement")
    ap.add_argument("--no-host-entry", action="store_true",
                    help="skip timing dbscan_fit on host arrays (copies in "
                         "and out included; reported apart, never as value)")
    ap.add_argument("--configs", default="1,2,3,4,5",
                    help="workloads timed as per_config lines besides the "
                         "main one (comma list, or 'none')")
    ap.add_argument("--cpu-baseline-child", action="store_true",
                    help=argparse.SUPPRESS)
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help=argparse.SUPPRESS)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB, "
                         "so a counter run can scale FETCH_SIZE/WRITE_SIZE")
    return ap.parse_args()


COUNTER_PROFILE = os.path.join(ROOT, "profiles",
                               "k_count_blobs_walks3d_n1000000_counters.md")
COUNT_SOURCES = ["all_pairs_distance_amd/csrc/k_count.hip",
                 "all_pairs_distance_amd/csrc/count_common.h",
                 "all_pairs_distance_amd/csrc/device.h",
                 "all_pairs_distance_amd/csrc/internal.h"]


def profiled_traffic(workload_name: str):
    """HBM-side bytes per count-kernel launch from the committed counter
    summary (scaled FETCH_SIZE + WRITE_SIZE), or None when that summary was
    taken on another workload or on kernel sources that have changed since."""
    if workload_name != "blobs_walks3d_n1000000" or not os.path.exists(COUNTER_PROFILE):
        return None
    fields = {}
    for line in open(COUNTER_PROFILE):
        if ":" in line and line.startswith("count-kernel-"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for src in COUNT_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if fields.get("count-kernel-sources-sha256") != h.hexdigest():
        return None
    return float(fields["count-kernel-traffic-bytes-per-launch"])


def digest(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a.astype("<i4")).tobytes()).hexdigest()


def _read(path):
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return None


def host_record() -> dict:
    """The host CPU: model, sockets, physical cores, threads per core, and
    the physical cores this process may run on (its affinity mask)."""
    model = None
    for line in (_read("/proc/cpuinfo") or "").splitlines():
        if line.startswith("model name"):
            model = line.split(":", 1)[1].strip()
            break
    online = []
    for name in os.listdir("/sys/devices/system/cpu"):
        if name.startswith("cpu") and name[3:].isdigit():
            online.append(int(name[3:]))
    topo = {}
    for c in online:
        base = f"/sys/devices/system/cpu/cpu{c}/topology/"
        pkg, core = _read(base + "physical_package_id"), _read(base + "core_id")
        if pkg is not None and core is not None:
            topo[c] = (int(pkg), int(core))
    allowed = sorted(os.sched_getaffinity(0))
    phys_all = set(topo.values())
    phys_allowed = {topo[c] for c in allowed if c in topo}
    sockets = len({p for p, _ in phys_all}) or None
    return {
        "cpu_model": model,
        "sockets": sockets,
        "physical_cores": len(phys_all) or None,
        "logical_cpus": len(online) or os.cpu_count(),
        "threads_per_core": (round(len(topo) / len(phys_all))
                             if phys_all else None),
        "cpus_allowed": len(allowed),
        "physical_cores_allowed": len(phys_allowed) or len(allowed),
    }


def cpu_baseline_child(args):
    """Child process: time the oracle's full fit on the first M points of
    the workload, M chosen for about --cpu-seconds of work.  Prints one JSON
    line.  Touches no GPU."""
    import oracle
    from all_pairs_distance_amd import datagen
    x, eps, min_pts, _ = datagen.make_workload(args.workload)
    o = oracle.get()
    m = 20000
    _, _, t = o.fit(x[:m], eps, min_pts, n_threads=args.cpu_threads)
    # fit time grows with M^2: pick M for about the target length
    m = int(min(x.shape[0], m * (args.cpu_seconds / max(t, 1e-3)) ** 0.5))
    _, _, t = o.fit(x[:m], eps, min_pts, n_threads=args.cpu_threads)
    print(json.dumps({"m": m, "seconds": t}), flush=True)


def cpu_baseline(args):
    """The oracle timed on the host's cores in a child process with one
    OpenMP thread per physical core it may use (at most OMP_NUM_THREADS),
    bound with OMP_PLACES=cores and OMP_PROC_BIND=spread."""
    host = host_record()
    cores = host["physical_cores_allowed"]
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(cores, cap) if cap > 0 else cores
    env = dict(os.environ, OMP_PLACES="cores", OMP_PROC_BIND="spread",
               OMP_NUM_THREADS=str(threads))
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child",
           "--workload", str(args.workload), "--cpu-seconds",
           str(args.cpu_seconds), "--cpu-threads", str(threads)]
    p = subprocess.run(cmd, env=env, capture_output=True, text=True,
                       timeout=30 * args.cpu_seconds + 120)
    if p.returncode != 0:
        raise RuntimeError(f"oracle baseline failed: {p.stderr[-2000:]}")
    r = json.loads(p.stdout.strip().splitlines()[-1])
    m, t = r["m"], r["seconds"]
    return {"value": m * m / t, "unit": "pair evaluations/s",
            "cores": threads, "kind": "oracle",
            "threads": threads,
            "omp": {"OMP_NUM_THREADS": threads, "OMP_PLACES": "cores",
                    "OMP_PROC_BIND": "spread"},
            "host": host,
            "sample": f"full oracle fit (counts, core flags, merge, borders, "
                      f"labels) of the first {m} of the workload's "
                      f"{args.n} points ({t:.1f} s, {m * m:.3g} ordered "
                      f"pairs)"}


def graph_leg(apd, torch, xt, n, d, eps, stream, steps, g, no_parity):
    """Time the sparse eps-graph export (pruned count pass, then row
    offsets, pair scatter and row sort) with buffers of the exact size,
    learnt from one sizing call."""
    import ctypes
    c = apd._c()
    flags = apd.FLAG_PRUNE_TILES | apd.FLAG_TIME_PHASES
    row_ptr = torch.empty(n + 1, dtype=torch.int64, device=xt.device)

    def call(ws, col, cap):
        nnz = ctypes.c_int64(0)
        info = c.dbscan_info()
        st = c.dbscan_graph_device(
            xt.data_ptr(), n, d, eps, row_ptr.data_ptr(),
            col.data_ptr() if col is not None else None, cap, nnz,
            ws.data_ptr(), ws.numel(), stream.cuda_stream, flags, info)
        return st, nnz.value, info

    ws = torch.empty(c.dbscan_graph_workspace_bytes(n, d, 0), dtype=torch.uint8,
                     device=xt.device)
    st, nnz, info = call(ws, None, 0)
    if st not in (0, c.ERR_CAPACITY):
        raise apd.DbscanError(st, info.hip_error)
    pairs_needed = int(info.n_edges)
    ws = torch.empty(c.dbscan_graph_workspace_bytes(n, d, pairs_needed),
                     dtype=torch.uint8, device=xt.device)
    col = torch.empty(max(nnz, 1), dtype=torch.int32, device=xt.device)
    st, _, info = call(ws, col, nnz)                  # warm-up
    if st != 0:
        raise apd.DbscanError(st, info.hip_error)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    infos = []
    start.record(stream)
    for _ in range(steps):
        st, _, info = call(ws, col, nnz)
        if st != 0:
            raise apd.DbscanError(st, info.hip_error)
        infos.append(info)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    parity = "unchecked"
    if not no_parity and g is not None and "graph_sha256" in g:
        h = hashlib.sha256()
        h.update(row_ptr.cpu().numpy().astype("<i8").tobytes())
        h.update(col[:nnz].cpu().numpy().astype("<i4").tobytes())
        parity = ("row_ptr+col_idx bit-exact vs oracle"
                  if h.hexdigest() == g["graph_sha256"] else "MISMATCH vs oracle")
    mean = lambda f: float(np.mean([getattr(i, f) for i in infos]))
    return {
        "what": "sparse eps-graph export (dbscan_graph_device, CSR, rows "
                "ascending, self included) with the pruned count pass",
        "ms_per_step": ms,
        "nnz": nnz,
        "entries_per_s": nnz / (ms / 1e3),
        "phases_ms": {"layout_sort_boxes": mean("ms_layout"),
                      "count": mean("ms_count"),
                      "row_offsets": mean("ms_core"),
                      "scatter": mean("ms_merge"),
                      "row_sort": mean("ms_label")},
        "parity": parity,
    }


def fit_runner(apd, torch, x, max_edges, dev):
    """Device buffers and a timed-fit helper for one workload."""
    n, d = x.shape
    xt = torch.from_numpy(x).to(dev)
    ws = apd.Workspace(n, d, max_edges, device=dev)
    labels = torch.empty(n, dtype=torch.int32, device=dev)
    counts = torch.empty(n, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(fl, eps, min_pts):
        info = apd.dbscan_info()
        st = apd.dbscan_fit_device_ex(
            xt.data_ptr(), n, d, eps, min_pts, labels.data_ptr(),
            counts.data_ptr(), ws.ptr, ws.nbytes, stream.cuda_stream, fl, info)
        if st != 0:
            raise apd.DbscanError(st, info.hip_error)
        return info

    def timed(fl, eps, min_pts, steps, warmup):
        for _ in range(warmup):
            step(fl, eps, min_pts)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        infos = []
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(steps):
            infos.append(step(fl, eps, min_pts))
        stop.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return infos, start.elapsed_time(stop) / steps, wall

    return xt, labels, counts, stream, timed


def golden_entry(key, x):
    """The oracle's stored digests of workload `key` if they describe
    exactly these input bytes."""
    from all_pairs_distance_amd import datagen
    path = os.path.join(ROOT, "tests", "golden", "workloads.json")
    if not os.path.exists(path):
        return None
    g = json.load(open(path)).get(str(key))
    return g if g and g["points_sha256"] == datagen.sha256_points(x) else None


def parity_of(g, labels, counts):
    if g is None:
        return "no oracle digests for these inputs"
    ok = (digest(labels) == g["labels_sha256"]
          and digest(counts) == g["counts_sha256"])
    return "labels+counts bit-exact vs oracle" if ok else "MISMATCH vs oracle"


def fractions(d, n, ms_count, ms_merge, pass2):
    """Count-pass fp32 rate (3d flops per ordered pair) over the peak; the
    same per distinct distance; and counted over count + merge with the
    tile merge's evaluated pairs added."""
    pairs = float(n) * float(n)
    achieved = 3.0 * d * pairs / (ms_count / 1e3) / 1e12
    return {
        "achieved_tflops": achieved,
        "frac": achieved / PEAK_FP32_TFLOPS,
        "frac_distinct_pairs": achieved / 2 * (n - 1) / n / PEAK_FP32_TFLOPS,
        "frac_count_plus_merge": 3.0 * d * (pairs + pass2)
        / ((ms_count + ms_merge) / 1e3) / 1e12 / PEAK_FP32_TFLOPS,
    }


def host_entry_leg(apd, x, eps, min_pts, labels_ref, reps=3):
    """dbscan_fit_counts on host arrays (allocation, copies in and out, fit,
    frees): median of `reps` after one warm-up."""
    apd.fit_host(x, eps, min_pts)
    ts = []
    lab_h = None
    for _ in range(reps):
        t0 = time.perf_counter()
        lab_h = apd.fit_host(x, eps, min_pts)
        ts.append(time.perf_counter() - t0)
    t_h = float(np.median(ts))
    n = x.shape[0]
    return {
        "value": float(n) * float(n) / t_h, "unit": "pair evaluations/s",
        "ms": t_h * 1e3,
        "what": "dbscan_fit on host arrays: device allocation, copies in "
                "and out, fit, frees (median of %d)" % reps,
        "labels_match_device_entry": bool(np.array_equal(lab_h, labels_ref)),
    }


def main():
    args = parse()
    if args.cpu_baseline_child:
        cpu_baseline_child(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding of the count pass is a design note only)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import all_pairs_distance_amd as apd
    from all_pairs_distance_amd import datagen

    x, eps, min_pts, w = datagen.make_workload(args.workload)
    n, d = x.shape
    args.n = n
    dev = torch.device("cuda:0")
    if args.calibrate_copy_mib:
        src = torch.ones(args.calibrate_copy_mib << 18, dtype=torch.float32,
                         device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    xt, labels, counts, stream, timed_fit = fit_runner(apd, torch, x,
                                                       args.max_edges, dev)
    flags = (apd.FLAG_TIME_PHASES
             | (apd.FLAG_FORCE_TILE_MERGE if args.tile_merge else 0)
             | (apd.FLAG_PRUNE_TILES if args.prune else 0)
             | (apd.FLAG_SCREEN if args.screen else 0))

    def timed(fl, steps, warmup):
        return timed_fit(fl, eps, min_pts, steps, warmup)

    infos, ms_per_step, wall = timed(flags, args.steps, args.warmup)

    pairs = float(n) * float(n)
    value = pairs / (ms_per_step / 1e3)
    ms_count = float(np.mean([i.ms_count for i in infos]))
    ms_merge = float(np.mean([i.ms_merge for i in infos]))
    flops_count = 3.0 * d * pairs
    achieved = flops_count / (ms_count / 1e3) / 1e12
    last = infos[-1]
    fr = fractions(d, n, ms_count, ms_merge, float(last.pass2_pairs))

    # the mode legs below reuse the label buffer: keep the default fit's
    labels_fit = labels.cpu().numpy()
    parity = "unchecked"
    g = None
    if not args.no_parity:
        g = golden_entry(args.workload, x)
        parity = parity_of(g, labels_fit, counts.cpu().numpy())

    out = {
        "metric": "pair evaluations/sec for full DBSCAN fit + % FP32 VALU peak, 1 GPU",
        "value": value,
        "unit": "pair evaluations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "n": n, "d": d, "eps": eps, "min_pts": min_pts,
            "merge": {1: "edge list", 2: "tile pass"}.get(last.merge_mode, "none"),
            "n_core": last.n_core, "n_edges": last.n_edges,
            "parity": parity,
        },
        "phases_ms": {
            "layout": float(np.mean([i.ms_layout for i in infos])),
            "count": ms_count,
            "core": float(np.mean([i.ms_core for i in infos])),
            "merge": ms_merge,
            "label": float(np.mean([i.ms_label for i in infos])),
            "wall_per_step": wall * 1e3 / args.steps,
        },
        "roofline": {
            "kernel": "k_count (neighbour-count pass)",
            "bound": "alu",
            "achieved": achieved,
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_TFLOPS,
            "traffic": profiled_traffic(w.name),
            "traffic_unit": "bytes per launch (HBM side, rocprofv3 FETCH_SIZE x2 "
                            "+ WRITE_SIZE x1, scale from a 256 MiB copy)",
            "flops_per_launch": flops_count,
            "credit": "3d flops per ordered pair; each distance evaluated once "
                      "decides two ordered pairs",
            "frac_distinct_pairs": fr["frac_distinct_pairs"],
            "frac_count_plus_merge": fr["frac_count_plus_merge"],
        },
    }
    out["config"]["tiles_kept"] = last.tiles_kept
    out["config"]["tiles_total"] = last.tiles_total

    def mode_leg(fl, what, ref=None):
        # ref: the oracle digests this mode must reproduce (the fit's own
        # unless the mode changes the distance form)
        ref = g if ref is None else ref
        m_infos, m_ms, _ = timed(fl, args.steps, 1)
        m_last = m_infos[-1]
        m_parity = "unchecked"
        if not args.no_parity and parity != "unchecked" and ref:
            m_parity = parity_of(ref, labels.cpu().numpy(), counts.cpu().numpy())
        return {
            "what": what,
            "value": pairs / (m_ms / 1e3),
            "unit": "pair relations decided/s",
            "ms_per_step": m_ms,
            "ms_count": float(np.mean([i.ms_count for i in m_infos])),
            "ms_layout_sort_boxes": float(np.mean([i.ms_layout for i in m_infos])),
            "tiles_kept": m_last.tiles_kept,
            "tiles_total": m_last.tiles_total,
            "parity": m_parity,
        }

    if not args.prune and not args.no_pruned_line:
        out["pruned_mode"] = mode_leg(
            flags | apd.FLAG_PRUNE_TILES,
            "same fit with exact tile pruning (DBSCAN_FLAG_PRUNE_TILES): "
            "block pairs whose fp32 box-gap bound exceeds eps^2 are "
            "skipped, every pair is still decided")
    if not args.screen and not args.no_screen_line:
        out["screen_mode"] = mode_leg(
            flags | apd.FLAG_SCREEN,
            "same fit with the screened count pass (DBSCAN_FLAG_SCREEN): "
            "hoisted-norm screen with a proven error bound, exact distance "
            "for the undecided pairs; identical results")
        out["pruned_screen_mode"] = mode_leg(
            flags | apd.FLAG_SCREEN | apd.FLAG_PRUNE_TILES,
            "tile pruning and the screened count pass together")
        out["expanded_mode"] = mode_leg(
            (flags & ~apd.FLAG_PRUNE_TILES) | apd.FLAG_EXPANDED,
            "fit deciding pairs with the hoisted-norm form T + P - sum "
            "2 x_k y_k itself (DBSCAN_FLAG_EXPANDED; screened); checked "
            "against the oracle's same form",
            ref=(g or {}).get("expanded") or {})
    if not args.no_graph_line:
        out["graph_mode"] = graph_leg(apd, torch, xt, n, d, eps, stream,
                                      args.steps, g, args.no_parity)
    if not args.no_host_entry:
        out["pcie_inclusive"] = host_entry_leg(apd, x, eps, min_pts, labels_fit)
    del xt, labels, counts, timed_fit
    torch.cuda.empty_cache()

    # the other workloads: the same default fit, each on buffers of its own
    keys = [] if args.configs == "none" else [
        int(k) for k in args.configs.split(",") if k.strip()]
    per = {}
    for key in keys:
        if key == args.workload:
            continue
        xk, eps_k, m_k, wk = datagen.make_workload(key)
        nk, dk = xk.shape
        xt_k, lab_k, cnt_k, _, timed_k = fit_runner(apd, torch, xk,
                                                     args.max_edges, dev)
        k_infos, k_ms, _ = timed_k(apd.FLAG_TIME_PHASES, eps_k, m_k,
                                   args.steps, args.warmup)
        k_last = k_infos[-1]
        kc = float(np.mean([i.ms_count for i in k_infos]))
        km = float(np.mean([i.ms_merge for i in k_infos]))
        lab_np = lab_k.cpu().numpy()
        entry = {
            "n": nk, "d": dk, "eps": eps_k, "min_pts": m_k,
            "ms_fit": k_ms,
            "pairs_per_s": float(nk) * float(nk) / (k_ms / 1e3),
            "phases_ms": {
                "layout": float(np.mean([i.ms_layout for i in k_infos])),
                "count": kc,
                "core": float(np.mean([i.ms_core for i in k_infos])),
                "merge": km,
                "label": float(np.mean([i.ms_label for i in k_infos])),
            },
            "merge": {1: "edge list", 2: "tile pass"}.get(k_last.merge_mode, "none"),
            "n_core": k_last.n_core, "n_edges": k_last.n_edges,
            "parity": ("unchecked" if args.no_parity else
                       parity_of(golden_entry(key, xk), lab_np,
                                 cnt_k.cpu().numpy())),
        }
        entry.update(fractions(dk, nk, kc, km, float(k_last.pass2_pairs)))
        if not args.no_host_entry:
            entry["pcie_inclusive_ms"] = host_entry_leg(
                apd, xk, eps_k, m_k, lab_np)["ms"]
        per[wk.name] = entry
        del xt_k, lab_k, cnt_k, timed_k
        torch.cuda.empty_cache()
    if per:
        out["per_config"] = per
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

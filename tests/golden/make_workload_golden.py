"""Write tests/golden/workloads.json: the oracle's result on the five named
synthetic workloads, as SHA-256 digests and summary counts.

Only the oracle is called (never the GPU library).  Run from the repository
root:  python tests/golden/make_workload_golden.py [--threads T] [--graph]
[--expanded] [keys...]   (--graph adds the digest of the sparse eps-graph
to existing entries, leaving the fit's fields as they are; --expanded adds,
under "expanded", the fit and graph digests of the hoisted-norm distance
form)
Each workload is written as soon as it finishes, so a partial run keeps its
finished entries.  The GPU parity tests compare the library's labels and
neighbour counts with these digests bit for bit, after checking that the
input digest still matches (the generator is deterministic per numpy
version).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from all_pairs_distance_amd import datagen  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "workloads.json")


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def graph_digest(row_ptr: np.ndarray, col_idx: np.ndarray) -> str:
    """SHA-256 over row_ptr (little-endian int64) followed by col_idx
    (little-endian int32)."""
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(row_ptr.astype("<i8")).tobytes())
    h.update(np.ascontiguousarray(col_idx.astype("<i4")).tobytes())
    return h.hexdigest()


def summary(labels: np.ndarray, counts: np.ndarray, min_pts: int) -> dict:
    core = counts >= min_pts
    noise = labels == -1
    return {
        "n_core": int(core.sum()),
        "n_border": int((~core & ~noise).sum()),
        "n_noise": int(noise.sum()),
        "n_clusters": int(np.unique(labels[~noise]).size),
        "sum_counts": int(counts.astype(np.int64).sum()),
        "max_count": int(counts.max()),
    }


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--threads", type=int, default=0)
    ap.add_argument("--graph", action="store_true")
    ap.add_argument("--expanded", action="store_true")
    ap.add_argument("keys", nargs="*", type=int, default=[1, 2, 3, 4, 5])
    args = ap.parse_args()
    table = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            table = json.load(f)
    o = oracle.get()
    for k in args.keys:
        x, eps, min_pts, w = datagen.make_workload(k)
        print(f"workload {k} {w.name}: n={w.n} d={w.d}", flush=True)
        t0 = time.time()
        if args.expanded:
            entry = table[str(k)]
            assert entry["points_sha256"] == datagen.sha256_points(x)
            labels, counts, fit_s = o.fit(x, eps, min_pts, n_threads=args.threads,
                                          form="expanded")
            sub = {
                "labels_sha256": digest(labels.astype("<i4")),
                "counts_sha256": digest(counts.astype("<i4")),
                **summary(labels, counts, min_pts),
                "oracle_fit_seconds": round(fit_s, 3),
            }
            del labels, counts
            if k <= 3:   # the graphs of the two largest sets take too long
                row_ptr, col_idx = o.graph(x, eps, n_threads=args.threads,
                                           form="expanded")
                sub["graph_sha256"] = graph_digest(row_ptr, col_idx)
                sub["graph_nnz"] = int(row_ptr[-1])
                del row_ptr, col_idx
            entry["expanded"] = sub
            with open(OUT, "w") as f:
                json.dump(table, f, indent=1, sort_keys=True)
                f.write("\n")
            print(k, json.dumps(sub), f"wall {time.time() - t0:.1f}s", flush=True)
            continue
        if args.graph:
            entry = table[str(k)]
            assert entry["points_sha256"] == datagen.sha256_points(x)
            row_ptr, col_idx = o.graph(x, eps, n_threads=args.threads)
            entry["graph_sha256"] = graph_digest(row_ptr, col_idx)
            entry["graph_nnz"] = int(row_ptr[-1])
            del row_ptr, col_idx
            with open(OUT, "w") as f:
                json.dump(table, f, indent=1, sort_keys=True)
                f.write("\n")
            print(k, entry["graph_nnz"], f"wall {time.time() - t0:.1f}s",
                  flush=True)
            continue
        labels, counts, fit_s = o.fit(x, eps, min_pts, n_threads=args.threads)
        entry = {
            "name": w.name, "n": w.n, "d": w.d, "eps": w.eps,
            "min_pts": w.min_pts,
            "points_sha256": datagen.sha256_points(x),
            "labels_sha256": digest(labels.astype("<i4")),
            "counts_sha256": digest(counts.astype("<i4")),
            **summary(labels, counts, min_pts),
            "oracle_fit_seconds": round(fit_s, 3),
            "oracle_threads": args.threads or os.cpu_count(),
            "host": platform.processor() or platform.machine(),
        }
        table[str(k)] = entry
        with open(OUT, "w") as f:
            json.dump(table, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(entry), f"wall {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    main()

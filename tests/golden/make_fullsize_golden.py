"""Write the whole 3pCF histograms of the two largest workloads from the oracle.

    python tests/golden/make_fullsize_golden.py C5 C3 [--threads T] [--parts P]

For each workload it regenerates the points from the workload's seed (``workloads``), builds the
oracle's neighbour graph with forward rows only (each row keeps the neighbours above its label;
the oracle's merge-walk reads nothing else), and runs the oracle's 3pCF count over the hub
labels in P parts (hubs i with i % P == part), adding the integer histograms.  Each part is kept
in a scratch folder while the run goes on, so an interrupted run resumes where it stopped.

Outputs, beside this script:
* ``<key>_counts.npy``: uint64 [C(nb+2,3)], the configurations in lexicographic order;
* ``<key>_counts.json``: workload, sizes, the SHA-256 of the generated coordinates, the bin
  edges, totals and timings, and the command.

Only ``oracle/`` computes anything here; nothing from the library is imported.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import tempfile
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def say(*a):
    print(time.strftime("%H:%M:%S"), *a, flush=True)


def make(key: str, threads: int, parts: int, parts_dir: str) -> None:
    cfg = workloads.get(key)
    t0 = time.time()
    xyz, _ = cfg.generate()
    sha = workloads.coords_sha256(xyz)
    edges = cfg.edges_sq()
    say(key, cfg.name, "points", xyz.shape[0], "sha256", sha[:16], f"{time.time() - t0:.1f} s")

    t0 = time.time()
    g = oracle.Graph(xyz, edges, nthreads=threads, forward_only=True)
    build_s = time.time() - t0
    say(key, "oracle graph", g.nnz, "forward edges", f"{build_s:.1f} s")

    ncfg = oracle.num_configs(3, cfg.nbins)
    total = np.zeros(ncfg, np.uint64)
    walks = 0
    count_s = 0.0
    pdir = os.path.join(parts_dir, f"{key}_{sha[:16]}_p{parts}")
    os.makedirs(pdir, exist_ok=True)
    for part in range(parts):
        f = os.path.join(pdir, f"part{part:04d}.npz")
        if os.path.exists(f):
            z = np.load(f)
            c, wk, dt = z["counts"], int(z["walks"]), float(z["seconds"])
        else:
            t0 = time.time()
            c, _, _, wk = g.count_3pcf(hub_stride=parts, hub_offset=part, nthreads=threads)
            dt = time.time() - t0
            np.savez(f + ".tmp.npz", counts=c, walks=wk, seconds=dt)
            os.replace(f + ".tmp.npz", f)
        total += c
        walks += wk
        count_s += dt
        say(key, f"part {part + 1}/{parts}", "triangles", int(c.sum()), f"{dt:.1f} s")

    np.save(os.path.join(HERE, f"{key}_counts.npy"), total)
    meta = {
        "workload": key,
        "name": cfg.name,
        "n_points": int(xyz.shape[0]),
        "kind": cfg.kind,
        "seed": cfg.seed,
        "r_max": cfg.r,
        "nbins": cfg.nbins,
        "edges_sq": [int(x) for x in edges],
        "coords_sha256": sha,
        "undirected_edges": int(g.nnz),
        "merge_walks": int(walks),
        "triangles": int(total.sum()),
        "configurations": int(ncfg),
        "oracle_threads": threads,
        "oracle_build_s": round(build_s, 1),
        "oracle_count_s": round(count_s, 1),
        "command": "python tests/golden/make_fullsize_golden.py " + key,
    }
    with open(os.path.join(HERE, f"{key}_counts.json"), "w") as fh:
        json.dump(meta, fh, indent=1)
        fh.write("\n")
    say(key, "written", meta["triangles"], "triangles")


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("keys", nargs="+", choices=["C3", "C5"])
    ap.add_argument("--threads", type=int, default=0, help="oracle threads (0: all cores)")
    ap.add_argument("--parts", type=int, default=64, help="hub parts, each saved as it ends")
    ap.add_argument("--parts-dir", default=os.path.join(tempfile.gettempdir(), "gtc_golden_parts"))
    a = ap.parse_args()
    for key in a.keys:
        make(key, a.threads, a.parts, a.parts_dir)


if __name__ == "__main__":
    main()

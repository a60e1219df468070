"""Benchmark of the graph 3pCF hot path on one MI355X.

One step = the whole path on one synthetic workload: build the neighbour graph on the GPU (cell
list, pair search, CSR emit, degree statistics, hub order, and for a tiled workload the hub
windows and their tiles), count the binned triangles (weighted when the workload has weights),
and release the graph.  Inputs (coordinates, weights) are in HBM before the timed region starts.

The default workload is the BAO-scale one (4M uniform points, ~9e9 directed edges, 30 bins) in
its hub-tiled mode: 4 GiB hub windows of the 18 GB CSR, the CSR held in pinned host memory and
the windows streamed to the GPU per tile (GRAMSCI v2 §III.5.3).  The same line reports the
resident and the re-emitted-window modes of the same workload, timed in the same process.

Prints one JSON line: triplets/s for the whole step (value), hub-spoke merge-walks/s, the
enumeration kernel's roofline (algorithmic bytes, and the HBM bytes of a stored counter run),
and the CPU oracle timed on a bounded sample of the same workload on this host's cores.

    python bench.py [--config C3] [--steps 5] [--warmup 1] [--gpus 1] [--no-cpu-baseline]

With --config C4 (the parity 4pCF workload) a step builds the graph and counts the binned
tetrahedra with their even and odd channels instead; the line then reports tetrahedra/s and the
4-clique kernel's VALU-issue roofline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
# LDS: 128 B per clock per CU, 256 CUs, 2.4 GHz
LDS_PEAK_GBS = 128 * 256 * 2.4


def lds_bytes(spoke_elements: int, triangles: int, weighted: bool, unsorted: bool = False) -> float:
    """Algorithmic LDS bytes of one enumeration launch: a hub-map probe per spoke element (1 B
    entry; 4 B weighted), and per triangle the two rank-table reads (8 B; none with the histogram
    over the unsorted bin triple) and the 32-bit counter update (read and write, 8 B); weighted
    triangles add the spoke's weight (8 B), the third weight (8 B) and two 64-bit limb updates
    (32 B)."""
    per_elem = 4.0 if weighted else 1.0
    per_tri = (0.0 if unsorted else 8.0) + 8.0 + (8.0 + 8.0 + 32.0 if weighted else 0.0)
    return per_elem * spoke_elements + per_tri * triangles
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_triplet_traffic.txt")
TRIPLET_VALU_FILE = os.path.join(ROOT, "profiles", "k_triplet_valu.txt")
VALU_FILE = os.path.join(ROOT, "profiles", "k_clique4_valu.txt")
# VALU issue: a wave64 instruction takes a 16-lane SIMD 4 clocks, 4 SIMDs per CU, so one wave
# instruction per clock per CU: 256 CUs at 2.4 GHz (G wave-instructions/s)
VALU_PEAK_GINST = 256 * 2.4


def kernel_fingerprint(kernel: str = "k_triplet") -> str | None:
    """A kernel's machine-code fingerprint written by the build (sha256 of the gfx950
    instructions of all its instantiations), or None without a build."""
    try:
        with open(os.path.join(ROOT, "graph_triangle_counting_amd", f"{kernel}.fingerprint")) as fh:
            return fh.read().strip() or None
    except OSError:
        return None


def measured_valu(key: str):
    """VALU wave-instructions per k_clique4 launch from the committed rocprofv3 counter run
    (SQ_INSTS_VALU), or None when that run predates the current kernel's machine code."""
    try:
        fp = kernel_fingerprint("k_clique4")
        if fp is None:
            return None
        with open(VALU_FILE) as fh:
            for line in fh:
                if line.startswith("#") or not line.strip():
                    continue
                k, f, v = line.split()
                if k == key and f == fp:
                    return float(v)
    except OSError:
        pass
    return None


def measured_traffic(key: str, launch_mode: int, path: str = TRAFFIC_FILE):
    """HBM bytes per k_triplet count (all tile launches of one count) from the committed
    rocprofv3 counter runs (FETCH_SIZE + WRITE_SIZE, scaled by the copy calibration), keyed by
    workload and mode, or None when those runs predate the current kernel's machine code or were
    taken with another kernel variant (launch mode bits 0-2).  With path=TRIPLET_VALU_FILE, the
    same for the VALU wave-instructions per count (SQ_INSTS_VALU)."""
    try:
        fp = kernel_fingerprint()
        if fp is None:
            return None
        with open(path) as fh:
            for line in fh:
                if line.startswith("#") or not line.strip():
                    continue
                k, f, mode, b = line.split()
                if k == key and f == fp and int(mode) == (launch_mode & 7):
                    return float(b)
    except OSError:
        pass
    return None

# CPU-baseline sample per workload: (sub-box side as a fraction of the grid, hub stride)
CPU_SAMPLE = {"C1": (1.0, 1), "C2": (1.0, 1), "C3": (1 / 3, 16), "C4": (1.0, 2), "C5": (1 / 3, 4)}

# The mode each workload names: (hub-window budget in CSR bytes, where the CSR is kept).  The
# BAO-scale and the large mixed workloads stream their CSR in hub windows; the others are resident.
GIB = 1 << 30
DEFAULT_MODE = {"C3": (4 * GIB, "host"), "C5": (2 * GIB, "host")}


def traffic_key(key: str, tile_bytes: int, csr_mode: str) -> str:
    """Key of a stored counter run: the workload, plus the mode when it is tiled
    (e.g. C3-host-4GiB)."""
    if tile_bytes <= 0:
        return key
    size = f"{tile_bytes // GIB}GiB" if tile_bytes % GIB == 0 else f"{tile_bytes}B"
    return f"{key}-{csr_mode}-{size}"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="C3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--tile-bytes", type=int, default=-1,
                    help="hub-window budget in CSR bytes (0: one resident window; default: the "
                         "workload's own mode, 4 GiB host-streamed windows for C3, 2 GiB for C5)")
    ap.add_argument("--no-modes", action="store_true",
                    help="tiled workloads: skip timing the resident and re-emitted-window modes")
    ap.add_argument("--mode-steps", type=int, default=3,
                    help="timed steps of each compared mode (after one warm-up)")
    ap.add_argument("--host-csr", action="store_true",
                    help="out-of-core: keep the CSR in pinned host memory, stream windows "
                         "(same as --csr-mode host)")
    ap.add_argument("--csr-mode", choices=["device", "host", "rebuild"], default=None,
                    help="where the CSR is kept: device memory, pinned host memory (windows "
                         "uploaded per tile) or nowhere (windows emitted again per tile); the "
                         "last two need --tile-bytes")
    ap.add_argument("--s4", action="store_true",
                    help="4pCF workloads: S4 configurations instead of sorted 6-tuples")
    ap.add_argument("--weighted", action="store_true",
                    help="4pCF workloads: the weighted count (exact class sums), weights uniform in "
                         "[0.5, 1.5) drawn with seed 7")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (HBM counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the counter has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import graph_triangle_counting_amd as gtc
    import workloads

    cfg = workloads.get(args.config)
    if args.tile_bytes < 0:
        if cfg.order == 3 and cfg.key in DEFAULT_MODE and not args.csr_mode and not args.host_csr:
            args.tile_bytes, args.csr_mode = DEFAULT_MODE[cfg.key]
        else:
            args.tile_bytes = 0
    if cfg.order == 4:
        bench_4pcf(args, cfg)
        return
    log(f"[bench] generating {cfg.key} {cfg.name} n={cfg.n}")
    xyz_np, w_np = cfg.generate()
    edges = cfg.edges_sq()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    csr_mode = args.csr_mode or ("host" if args.host_csr else "device")
    xyz = torch.from_numpy(xyz_np).to(dev)
    w = None if w_np is None else torch.from_numpy(w_np).to(dev)
    torch.cuda.synchronize()

    def run(tile_bytes, mode, warmup, steps, tag):
        def step():
            g = gtc.Graph(xyz, edges, tile_bytes=tile_bytes, csr_mode=mode)
            c, ws, st = g.count_3pcf(w)
            gst = g.stats()
            g.close()
            return st, gst

        for k in range(warmup):
            st, gst = step()
            log(f"[bench] {tag} warmup {k}: build {gst['build_ms']:.2f} ms, kernel "
                f"{st['kernel_ms']:.2f} ms, count {st['count_ms']:.2f} ms, T={st['triangles']}")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rec = {"kernel_ms": [], "build_ms": [], "count_ms": [], "h2d_ms": [], "T": [], "q": []}
        for k in range(steps):
            st, gst = step()
            rec["kernel_ms"].append(st["kernel_ms"])
            rec["build_ms"].append(gst["build_ms"])
            rec["count_ms"].append(st["count_ms"])
            rec["h2d_ms"].append(st["h2d_ms"])
            rec["T"].append(st["triangles"])
            rec["q"].append(st["q_alg_bytes"])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        assert len(set(rec["T"])) == 1, "triangle counts differ between steps"
        avg = {k: sum(v) / len(v) for k, v in rec.items() if k not in ("T", "q")}
        log(f"[bench] {tag} {steps} steps: {1e3 * elapsed / steps:.2f} ms/step, build "
            f"{avg['build_ms']:.2f} ms, kernel {avg['kernel_ms']:.3f} ms, count "
            f"{avg['count_ms']:.2f} ms, T={rec['T'][0]}, E={st['edges']}, windows "
            f"{st['windows']}, tiles {st['tiles']}, h2d {avg['h2d_ms']:.1f} ms")
        return st, rec, avg, elapsed

    tag = csr_mode if args.tile_bytes > 0 else "resident"
    st, rec, avg, elapsed = run(args.tile_bytes, csr_mode, args.warmup, args.steps, tag)
    ms_step = 1e3 * elapsed / args.steps
    T = rec["T"][0]
    value = T * args.steps / elapsed
    k_avg = avg["kernel_ms"]
    achieved = rec["q"][0] / (k_avg * 1e-3) / 1e9

    modes = None
    if args.tile_bytes > 0 and not args.no_modes:
        modes = {tag: {"ms_per_step": ms_step, "build_ms": avg["build_ms"],
                       "count_ms": avg["count_ms"], "kernel_ms": k_avg,
                       "h2d_ms": avg["h2d_ms"], "windows": st["windows"], "tiles": st["tiles"]}}
        others = [("resident", 0, "device")]
        for m in ("rebuild", "host"):
            if m != csr_mode:
                others.append((m, args.tile_bytes, m))
        for name, tb, m in others:
            mst, mrec, mavg, mel = run(tb, m, 1, args.mode_steps, name)
            assert mrec["T"][0] == T, f"{name} mode counts a different triangle total"
            modes[name] = {"ms_per_step": 1e3 * mel / args.mode_steps,
                           "build_ms": mavg["build_ms"], "count_ms": mavg["count_ms"],
                           "kernel_ms": mavg["kernel_ms"], "h2d_ms": mavg["h2d_ms"],
                           "windows": mst["windows"], "tiles": mst["tiles"]}
        res = modes["resident"]["ms_per_step"]
        for m in modes.values():
            m["vs_resident"] = m["ms_per_step"] / res

    tkey = traffic_key(cfg.key, args.tile_bytes, csr_mode)
    traffic = measured_traffic(tkey, st["launch_mode"])
    ach = achievable_hbm_gbs()
    log(f"[bench] device copy reaches {ach['copy']:.0f} GB/s, a 1 GiB sum reads {ach['read']:.0f} GB/s")
    traffic_gbs = None if traffic is None else traffic / (k_avg * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "traffic_gbs": traffic_gbs,
                "frac_traffic": None if traffic_gbs is None else traffic_gbs / HBM_PEAK_GBS,
                "traffic_from": None if traffic is None else
                f"stored rocprofv3 counter run {os.path.relpath(TRAFFIC_FILE, ROOT)} "
                f"[{tkey}], FETCH_SIZE + WRITE_SIZE scaled by a plain copy, k_triplet machine "
                f"code {kernel_fingerprint()}, launch mode {st['launch_mode'] & 7}; not measured "
                f"in this run",
                "achievable": ach["best"], "frac_achievable": achieved / ach["best"],
                "achievable_from": {"copy_gbs": ach["copy"], "read_gbs": ach["read"],
                                    "kernels": "1 GiB device-to-device copy (read + written "
                                               "bytes); 1 GiB streaming read (gtc_hbm_read_rate)"},
                "kernel": "k_triplet", "kernel_ms": k_avg, "q_alg_bytes": rec["q"][0],
                "launch": {"waves_per_wg": st["launch_waves"], "workgroups": st["launch_blocks"],
                           "lds_bytes": st["launch_lds_bytes"]}}

    valu_insts = measured_traffic(tkey, st["launch_mode"], TRIPLET_VALU_FILE)
    valu = None if valu_insts is None else {
        "achieved": valu_insts / (k_avg * 1e-3) / 1e9, "peak": VALU_PEAK_GINST,
        "unit": "G VALU wave-instructions/s",
        "frac": valu_insts / (k_avg * 1e-3) / 1e9 / VALU_PEAK_GINST, "insts": valu_insts,
        "from": f"stored rocprofv3 counter run {os.path.relpath(TRIPLET_VALU_FILE, ROOT)} [{tkey}], "
                f"SQ_INSTS_VALU, k_triplet machine code {kernel_fingerprint()}, launch mode "
                f"{st['launch_mode'] & 7}; not measured in this run",
        "kernel": "k_triplet"}

    lds_b = lds_bytes(st["spoke_elements"], T, cfg.weighted, bool(st["launch_mode"] & 2))
    lds = {"achieved": lds_b / (k_avg * 1e-3) / 1e9, "peak": LDS_PEAK_GBS, "unit": "GB/s",
           "frac": lds_b / (k_avg * 1e-3) / 1e9 / LDS_PEAK_GBS, "bytes": lds_b,
           "kernel": "k_triplet"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, xyz_np, w_np, args.cpu_threads)

    out = {
        "metric": "triplets counted/sec and hub-spoke merge-walks/sec (3pCF), 1 MI355X",
        "value": value,
        "unit": "triplets/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int64+f64" if cfg.weighted else "int64",
        "data": "synthetic",
        "config": {"workload": f"{cfg.key} {cfg.name}", "n_points": cfg.n, "kind": cfg.kind,
                   "r_max": cfg.r, "nbins": cfg.nbins, "weighted": cfg.weighted,
                   "mean_degree_target": cfg.target_degree, "edges": st["edges"],
                   "triangles": T, "merge_walks": st["edges"],
                   "merge_walks_enumerated": st["merge_walks"], "tile_bytes": args.tile_bytes,
                   "csr_mode": csr_mode, "windows": st["windows"], "tiles": st["tiles"]},
        "merge_walks_per_s": st["edges"] * args.steps / elapsed,
        "merge_walks_note": "one walk per forward edge (E+); merge_walks_enumerated leaves out "
                            "the walks of hubs that cannot close a triangle (fewer than two "
                            "forward neighbours, or spokes with no forward neighbours)",
        "kernel_triplets_per_s": T / (k_avg * 1e-3),
        "build_ms": avg["build_ms"],
        "count_ms": avg["count_ms"],
        "h2d_ms": avg["h2d_ms"],
        "modes": modes,
        "roofline": roofline,
        "valu": valu,
        "lds": lds,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_4pcf(args, cfg):
    """The parity 4pCF path: build, the 4-clique count (even and odd channels) over sorted bin
    6-tuples, or S4 configurations (--s4), unweighted or with exact weighted class sums
    (--weighted), release."""
    import numpy as np
    import torch

    import graph_triangle_counting_amd as gtc
    import workloads
    log(f"[bench] generating {cfg.key} {cfg.name} n={cfg.n}")
    xyz_np, _ = cfg.generate()
    edges = cfg.edges_sq()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    csr_mode = args.csr_mode or ("host" if args.host_csr else "device")
    xyz = torch.from_numpy(xyz_np).to(dev)
    w_np = workloads.rng_for(7).uniform(0.5, 1.5, xyz_np.shape[0]) if args.weighted else None
    w = None if w_np is None else torch.from_numpy(np.ascontiguousarray(w_np)).to(dev)
    torch.cuda.synchronize()

    def step():
        g = gtc.Graph(xyz, edges, tile_bytes=args.tile_bytes, csr_mode=csr_mode)
        if w is None:
            st = g.count_4pcf_parity(s4=args.s4)[-1]
        else:
            st = g.count_4pcf_weighted(w, s4=args.s4)[-1]
        gst = g.stats()
        g.close()
        return st, gst

    for k in range(args.warmup):
        st, gst = step()
        log(f"[bench] warmup {k}: build {gst['build_ms']:.2f} ms, kernel {st['kernel_ms']:.2f} ms, "
            f"tetrahedra {st['cliques4']}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    kms, bms, ncl = [], [], []
    for k in range(args.steps):
        st, gst = step()
        kms.append(st["kernel_ms"])
        bms.append(gst["build_ms"])
        ncl.append(st["cliques4"])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert len(set(ncl)) == 1, "tetrahedron counts differ between steps"
    K = ncl[0]
    k_avg = sum(kms) / len(kms)
    log(f"[bench] {args.steps} steps: {1e3 * elapsed / args.steps:.2f} ms/step, build "
        f"{sum(bms) / len(bms):.2f} ms, kernel {k_avg:.3f} ms, tetrahedra {K}, windows "
        f"{gst['windows']}, tiles {st['tiles']}")
    variant = cfg.key + ("-s4" if args.s4 else "") + ("-w" if args.weighted else "")
    valu = measured_valu(variant) if args.tile_bytes == 0 else None
    achieved = None if valu is None else valu / (k_avg * 1e-3) / 1e9
    roofline = {"bound": "alu", "achieved": achieved, "peak": VALU_PEAK_GINST,
                "unit": "G VALU wave-instructions/s",
                "frac": None if achieved is None else achieved / VALU_PEAK_GINST, "traffic": None,
                "valu_insts_per_launch": valu,
                "valu_insts_per_tetrahedron": None if valu is None else valu / K,
                "kernel": "k_clique4", "kernel_ms": k_avg,
                "kernel_tetrahedra_per_s": K / (k_avg * 1e-3),
                "launch": {"waves_per_wg": st["launch_waves"], "workgroups": st["launch_blocks"],
                           "lds_bytes": st["launch_lds_bytes"]}}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_4pcf(cfg, xyz_np, args.cpu_threads, args.s4, w_np)
    out = {
        "metric": "4-cliques (tetrahedra) counted/sec with the even/odd parity split (4pCF), "
                  "1 MI355X",
        "value": K * args.steps / elapsed,
        "unit": "tetrahedra/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32+f64",
        "data": "synthetic",
        "config": {"workload": f"{cfg.key} {cfg.name}", "n_points": cfg.n, "kind": cfg.kind,
                   "r_max": cfg.r, "nbins": cfg.nbins,
                   "configurations": "S4" if args.s4 else "sorted 6-tuples",
                   "weighted": bool(args.weighted),
                   "edges": st["edges"], "tetrahedra": K, "tile_bytes": args.tile_bytes,
                   "csr_mode": csr_mode, "windows": gst["windows"], "tiles": st["tiles"]},
        "build_ms": sum(bms) / len(bms),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_4pcf(cfg, xyz, threads, s4=False, w=None):
    """The oracle's parity 4pCF, as it is, on every stride-th hub of the same point set (weighted:
    the whole set, the oracle's weighted count takes no hub stride)."""
    import numpy as np

    import oracle
    _, stride = CPU_SAMPLE[cfg.key]
    nthreads = threads or (os.cpu_count() or 1)
    try:
        nthreads = min(nthreads, len(os.sched_getaffinity(0)))
    except AttributeError:
        pass
    log(f"[bench] cpu baseline: oracle 4pCF on {xyz.shape[0]} points, hub stride {stride}, "
        f"{nthreads} threads")
    t0 = time.perf_counter()
    g = oracle.Graph(xyz, cfg.edges_sq(), nthreads=nthreads)
    tb = time.perf_counter() - t0
    t0 = time.perf_counter()
    if w is None:
        ev, _, ncl = g.count_4pcf_parity(hub_stride=stride, nthreads=nthreads, s4=s4)
    else:
        stride = 1
        ev = g.count_4pcf_weighted(w, s4=s4, nthreads=nthreads)[0]
        ncl = int(np.asarray(ev, dtype=np.uint64).sum())
    tc = time.perf_counter() - t0
    assert int(np.asarray(ev, dtype=np.uint64).sum()) == ncl
    return {"value": ncl / tc, "unit": "tetrahedra/s", "cores": nthreads, "kind": "oracle",
            "sample": f"full point set ({xyz.shape[0]} points); tetrahedra of every {stride}-th "
                      f"hub label ({ncl} tetrahedra); count phase {tc:.2f} s, graph build "
                      f"{tb:.2f} s",
            "tetrahedra": ncl, "count_s": tc, "build_s": tb}


def achievable_hbm_gbs(nbytes: int = 1 << 30, reps: int = 5) -> dict:
    """HBM rates two plain kernels reach on this GPU, best of reps, HIP events on their stream: a
    device-to-device copy (bytes read + written per second) and the library's streaming-read
    probe over 1 GiB.  The larger is the measured ceiling beside the vendor peak."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(7)
    dst = torch.empty_like(src)

    def best(fn):
        fn()
        t = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            t = min(t, e0.elapsed_time(e1) * 1e-3)
        return t

    import graph_triangle_counting_amd as gtc
    copy = 2.0 * nbytes / best(lambda: dst.copy_(src)) / 1e9
    read = gtc.hbm_read_rate(src, reps)
    del src, dst
    torch.cuda.empty_cache()
    return {"copy": copy, "read": read, "best": max(copy, read)}


def copy_calibration(nbytes: int):
    """A plain device copy of a known size: what FETCH_SIZE / WRITE_SIZE read for it scales the
    counters of the enumeration kernel to bytes."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4, "copies": 3}), flush=True)


def cpu_baseline(cfg, xyz, w, threads):
    """The oracle, as it is, on a bounded sample of the same workload, on this host's cores."""
    import numpy as np

    import oracle
    frac, stride = CPU_SAMPLE[cfg.key]
    if frac < 1.0:
        xyz, w = cfg.crop(xyz, w, frac)
    nthreads = threads or (os.cpu_count() or 1)
    try:
        nthreads = min(nthreads, len(os.sched_getaffinity(0)))
    except AttributeError:
        pass
    log(f"[bench] cpu baseline: oracle on {xyz.shape[0]} points, hub stride {stride}, "
        f"{nthreads} threads")
    t0 = time.perf_counter()
    g = oracle.Graph(xyz, cfg.edges_sq(), nthreads=nthreads)
    tb = time.perf_counter() - t0
    t0 = time.perf_counter()
    c, _, _, walks = g.count_3pcf(w, hub_stride=stride, nthreads=nthreads)
    tc = time.perf_counter() - t0
    T = int(np.asarray(c, dtype=np.uint64).sum())
    # one core: the same count on every (16 stride)-th hub of the sample, about a second
    t0 = time.perf_counter()
    c1, _, _, walks1 = g.count_3pcf(w, hub_stride=16 * stride, nthreads=1)
    t1 = time.perf_counter() - t0
    T1 = int(np.asarray(c1, dtype=np.uint64).sum())
    serial = {"value": T1 / t1, "unit": "triplets/s", "cores": 1,
              "sample": f"triangles of every {16 * stride}-th hub label of the same sample "
                        f"({T1} triangles, {t1:.2f} s)"}
    sample = (f"{'full point set' if frac >= 1 else f'central sub-box of side {frac:.3f} L, full density'}"
              f" ({xyz.shape[0]} points); triangles of every {stride}-th hub label"
              f"{' (all hubs)' if stride == 1 else ''}; count phase {tc:.2f} s, graph build "
              f"{tb:.2f} s")
    return {"value": T / tc, "unit": "triplets/s", "cores": nthreads, "kind": "oracle",
            "sample": sample, "merge_walks_per_s": walks / tc, "triangles": T,
            "count_s": tc, "build_s": tb, "serial": serial}


if __name__ == "__main__":
    main()

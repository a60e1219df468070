"""Command line: the 3pCF / 4pCF estimators on catalogue files (GRAMSCI v2 §II.2's compute_3pcf /
compute_4pcf, as a command).

    python -m graph_triangle_counting_amd 3pcf --data D.npy --randoms R.npy \
        --rmin 1 --rmax 30 --nbins 6 --out result.npz
    python -m graph_triangle_counting_amd 4pcf --data D.npy --randoms R.npy \
        --rmin 20 --rmax 65 --nbins 4 --out result.npz

Catalogues are .npy arrays of float positions [n, 3] (any unit), weights .npy [n] (optional,
default 1).  Positions are mapped onto the integer grid of the library: x_grid = rint((x - lo) *
scale), lo the smallest coordinate over both catalogues and scale = (2^20 - 1) / the largest
extent, and radii r_grid = r * scale; bin b holds the integer squared grid distances d^2 with
ceil(r_b_grid^2) <= d^2 < ceil(r_{b+1}_grid^2), r_b equally spaced from rmin to rmax.  The grid
step 1 / scale is the resolution of the measurement.  The output .npz holds the estimator arrays
(zeta, NNN, RRR, bins, r1..r3 for the 3pCF; zeta_even, zeta_odd, zeta_conn, xi, bins, r1..r6,
realizable for the 4pCF), radii in the input unit, and the grid scale.
"""
from __future__ import annotations

import argparse
import sys

import numpy as np

GRID = 1 << 20


def grid_map(pos_data: np.ndarray, pos_rand: np.ndarray):
    """(lo, scale) mapping both catalogues onto [0, 2^20) with one common scale."""
    allp = np.concatenate([pos_data.reshape(-1, 3), pos_rand.reshape(-1, 3)])
    if not np.all(np.isfinite(allp)):
        raise ValueError("positions must be finite")
    lo = allp.min(axis=0)
    extent = float((allp.max(axis=0) - lo).max())
    scale = (GRID - 1) / extent if extent > 0 else 1.0
    return lo, scale


def to_grid(pos: np.ndarray, lo: np.ndarray, scale: float) -> np.ndarray:
    g = np.rint((np.asarray(pos, np.float64).reshape(-1, 3) - lo) * scale)
    return np.clip(g, 0, GRID - 1).astype(np.int32)


def edges_sq(rmin: float, rmax: float, nbins: int, scale: float) -> np.ndarray:
    """Integer squared edges of nbins bins equally spaced in r from rmin to rmax, grid units."""
    if not (0 <= rmin < rmax) or nbins < 1:
        raise ValueError("need 0 <= rmin < rmax and nbins >= 1")
    r = (rmin + np.arange(nbins + 1) * (rmax - rmin) / nbins) * scale
    e = np.ceil(r * r).astype(np.int64)
    if np.any(np.diff(e) <= 0):
        raise ValueError("bins narrower than the grid resolution")
    return e


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m graph_triangle_counting_amd",
                                 description="3pCF / 4pCF estimators on one MI355X")
    ap.add_argument("statistic", choices=["3pcf", "4pcf"])
    ap.add_argument("--data", required=True, help=".npy float positions [n, 3]")
    ap.add_argument("--data-weights", default=None, help=".npy weights [n] (default 1)")
    ap.add_argument("--randoms", required=True, help=".npy float positions [n, 3]")
    ap.add_argument("--random-weights", default=None, help=".npy weights [n] (default 1)")
    ap.add_argument("--rmin", type=float, required=True)
    ap.add_argument("--rmax", type=float, required=True)
    ap.add_argument("--nbins", type=int, required=True)
    ap.add_argument("--out", required=True, help="output .npz")
    ap.add_argument("--tile-bytes", type=int, default=0,
                    help="hub-window budget in CSR bytes (0: automatic)")
    ap.add_argument("--csr-mode", choices=["device", "host", "rebuild"], default=None)
    args = ap.parse_args(argv)

    import torch

    import graph_triangle_counting_amd as gtc

    pd = np.load(args.data, allow_pickle=False)
    pr = np.load(args.randoms, allow_pickle=False)
    wd = None if args.data_weights is None else np.load(args.data_weights, allow_pickle=False)
    wr = None if args.random_weights is None else np.load(args.random_weights, allow_pickle=False)
    lo, scale = grid_map(pd, pr)
    e = edges_sq(args.rmin, args.rmax, args.nbins, scale)
    dev = torch.device("cuda", torch.cuda.current_device())
    xd = torch.from_numpy(to_grid(pd, lo, scale)).to(dev)
    xr = torch.from_numpy(to_grid(pr, lo, scale)).to(dev)
    td = None if wd is None else torch.from_numpy(np.asarray(wd, np.float64)).to(dev)
    tr = None if wr is None else torch.from_numpy(np.asarray(wr, np.float64)).to(dev)
    kw = dict(edges_sq=e, tile_bytes=args.tile_bytes, csr_mode=args.csr_mode)
    out = {"edges_sq": e, "grid_scale": np.float64(scale), "grid_origin": lo}
    if args.statistic == "3pcf":
        r = gtc.compute_3pcf(xd, td, xr, tr, **kw)
        out.update(zeta=r.zeta, NNN=r.NNN, RRR=r.RRR, bins=r.bins,
                   r1=r.r1 / scale, r2=r.r2 / scale, r3=r.r3 / scale)
    else:
        r = gtc.compute_4pcf(xd, td, xr, tr, **kw)
        out.update(zeta_even=r.zeta_even, zeta_odd=r.zeta_odd, zeta_conn=r.zeta_conn, xi=r.xi,
                   bins=r.bins, realizable=r.realizable,
                   **{f"r{k + 1}": getattr(r, f"r{k + 1}") / scale for k in range(6)})
    np.savez(args.out, **out)
    print(f"{args.statistic}: {len(r.bins)} configurations, grid step {1 / scale:.6g}, "
          f"kernel {r.stats['kernel_ms']:.1f} ms -> {args.out}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

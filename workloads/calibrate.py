"""Pick the integer r_max of each workload so the realised mean neighbour count is closest to the
target, then print the values to freeze into ``workloads.CONFIGS``.

The mean degree is 2E/N with E the number of unordered pairs at squared distance < r^2 (distinct
points, integer coordinates, exact integer test).  Large configurations are measured on a fixed
random sample of hubs (exact neighbour counts for each sampled hub), which pins the mean to well
under 0.5 %.  Usage:  python -m workloads.calibrate [C1 C2 ...]
"""
from __future__ import annotations

import sys

import numpy as np
from scipy.spatial import cKDTree

from workloads import CONFIGS, rng_for


def mean_degree(tree: cKDTree, xyz: np.ndarray, hubs: np.ndarray, r: int) -> float:
    """Mean over ``hubs`` of the exact number of other points with squared distance < r^2.

    Squared distances are integers, so d^2 < r^2 is the same as d <= sqrt(r^2 - 1/2); the float
    distance error (~1e-16 relative) is far below that half-unit margin.
    """
    rq = float(np.sqrt(r * r - 0.5))
    tot = 0
    for chunk in np.array_split(hubs, max(1, hubs.size // 4000)):
        tot += int(tree.query_ball_point(xyz[chunk].astype(np.float64), rq,
                                         return_length=True).sum()) - chunk.size  # minus self
    return tot / hubs.size


def calibrate(key: str, sample: int = 20_000) -> tuple[int, float]:
    cfg = CONFIGS[key]
    xyz, _ = cfg.generate()
    tree = cKDTree(xyz.astype(np.float64))
    hubs = np.arange(xyz.shape[0]) if xyz.shape[0] <= sample else \
        np.sort(rng_for(1000 + cfg.seed).choice(xyz.shape[0], sample, replace=False))
    # bracket on r (degree is monotone in r): start below the uniform-density estimate, double up
    n = xyz.shape[0]
    lo = max(1, int((cfg.target_degree / (n * 4.0 / 3.0 * np.pi)) ** (1 / 3) * (1 << 20) / 8))
    while mean_degree(tree, xyz, hubs, lo) >= cfg.target_degree and lo > 1:
        lo //= 2
    hi = lo * 2
    while mean_degree(tree, xyz, hubs, hi) < cfg.target_degree:
        lo, hi = hi, hi * 2
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if mean_degree(tree, xyz, hubs, mid) < cfg.target_degree:
            lo = mid
        else:
            hi = mid
    dlo, dhi = mean_degree(tree, xyz, hubs, lo), mean_degree(tree, xyz, hubs, hi)
    r, d = (lo, dlo) if abs(dlo - cfg.target_degree) <= abs(dhi - cfg.target_degree) else (hi, dhi)
    return r, d


if __name__ == "__main__":
    keys = sys.argv[1:] or list(CONFIGS)
    for k in keys:
        r, d = calibrate(k)
        print(f"{k}: r={r} mean_degree~{d:.2f} (target {CONFIGS[k].target_degree})", flush=True)

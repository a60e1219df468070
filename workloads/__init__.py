"""Seeded synthetic point sets for the graph 3pCF / 4pCF counter.

This module only makes inputs: integer coordinates on the 2^20 grid, optional weights and the
integer squared bin edges of a configuration.  It holds none of the counting arithmetic, so the
oracle and the HIP path can both draw their inputs from it without sharing any computation.

The pages measure on survey catalogues and N-body mocks that are not available here (GRAMSCI v2,
"Fast Graph-based Higher-Order Clustering Statistics on the GPU", §IV.1 test catalogue, §V DESI
DR1 LRG, §IV.9 Quijote halos).  The configurations below stand in for them: uniform points for the
quasi-uniform test mock, and Neyman-Scott clustered points for the heavy high-multiplicity tail
that makes survey data slow (§V.2, the closing cost note).

Coordinates are ``int32`` arrays of shape ``(n, 3)`` with every value in ``[0, 2**20)``.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

GRID = 1 << 20  # side of the integer coordinate grid


def rng_for(seed: int) -> np.random.Generator:
    """PCG64 generator for a configuration seed."""
    return np.random.Generator(np.random.PCG64(seed))


def uniform_points(rng: np.random.Generator, n: int) -> np.ndarray:
    """n points drawn uniformly from the integer grid [0, 2^20)^3."""
    return rng.integers(0, GRID, size=(n, 3), dtype=np.int64).astype(np.int32)


def neyman_scott_points(rng: np.random.Generator, n: int, parents: int,
                        sigma: float) -> np.ndarray:
    """Neyman-Scott clustered points on the integer grid.

    ``parents`` cluster centres are uniform in the continuous box [0, 2^20)^3.  Each of the ``n``
    children picks a parent uniformly at random (so children per parent are multinomial), takes a
    Gaussian offset of standard deviation ``sigma`` grid units on each axis and is rounded half to
    even onto the grid.  A child that lands outside [0, 2^20) on any axis draws a fresh offset
    (same parent) until it lands inside.
    """
    centres = rng.random((parents, 3)) * GRID
    owner = rng.integers(0, parents, size=n)
    out = np.empty((n, 3), dtype=np.int64)
    todo = np.arange(n)
    while todo.size:
        pos = np.rint(centres[owner[todo]] + rng.normal(0.0, sigma, size=(todo.size, 3)))
        ok = np.all((pos >= 0) & (pos < GRID), axis=1)
        out[todo[ok]] = pos[ok].astype(np.int64)
        todo = todo[~ok]
    return out.astype(np.int32)


def uniform_weights(rng: np.random.Generator, n: int, lo: float = 0.5,
                    hi: float = 1.5) -> np.ndarray:
    """fp64 weights uniform in [lo, hi)."""
    return lo + (hi - lo) * rng.random(n)


def linear_edges_sq(r: int, nbins: int) -> np.ndarray:
    """Integer squared bin edges for ``nbins`` bins equally spaced in r on [0, r).

    e_b = ceil(b^2 r^2 / nbins^2) for b = 0..nbins, so for an integer squared distance d2,
    d2 >= e_b holds exactly when sqrt(d2) >= b r / nbins.  e_0 = 0 and e_nbins = r^2.
    """
    b = np.arange(nbins + 1, dtype=object)
    e = [(int(x) * int(x) * r * r + nbins * nbins - 1) // (nbins * nbins) for x in b]
    return np.array(e, dtype=np.int64)


def coords_sha256(xyz: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(xyz, dtype=np.int32).tobytes()).hexdigest()


@dataclass(frozen=True)
class Config:
    """One benchmark / parity workload."""
    key: str
    name: str
    kind: str            # "uniform" | "neyman_scott" | "mixed"
    n: int
    seed: int
    target_degree: float  # target mean number of neighbours 2E/N
    nbins: int
    r: int               # integer r_max (grid units), calibrated to target_degree and frozen
    order: int = 3       # 3 -> 3pCF, 4 -> parity 4pCF
    weighted: bool = False
    parents: int = 20_000
    sigma_frac: float = 0.002
    notes: str = field(default="")

    @property
    def sigma(self) -> float:
        return self.sigma_frac * GRID

    def edges_sq(self) -> np.ndarray:
        return linear_edges_sq(self.r, self.nbins)

    def generate(self, n: int | None = None):
        """Return (xyz int32 [n,3], weights fp64 [n] or None) for this configuration.

        ``n`` overrides the point count while keeping the generator; it is used to make scaled-down
        variants, never for the configuration itself.
        """
        n = self.n if n is None else n
        rng = rng_for(self.seed)
        if self.kind == "uniform":
            xyz = uniform_points(rng, n)
        elif self.kind == "neyman_scott":
            xyz = neyman_scott_points(rng, n, self.parents, self.sigma)
        elif self.kind == "mixed":
            half = n // 2
            a = uniform_points(rng, half)
            b = neyman_scott_points(rng, n - half, self.parents, self.sigma)
            xyz = np.concatenate([a, b])
        else:
            raise ValueError(self.kind)
        xyz = xyz[rng.permutation(n)]
        w = uniform_weights(rng, n) if self.weighted else None
        return np.ascontiguousarray(xyz, dtype=np.int32), w

    def crop(self, xyz: np.ndarray, w, frac_side: float, corner=(0.5, 0.5, 0.5)):
        """Points of (xyz, w) inside an axis-aligned sub-box with side ``frac_side * 2^20``,
        centred at ``corner`` (fractions of the grid).  Keeps the full density, so rows have the
        same lengths as in the full workload.
        """
        side = int(frac_side * GRID)
        lo = np.array([int(c * GRID) - side // 2 for c in corner], dtype=np.int64)
        lo = np.clip(lo, 0, GRID - side)
        sel = np.all((xyz >= lo) & (xyz < lo + side), axis=1)
        return np.ascontiguousarray(xyz[sel]), (None if w is None else np.ascontiguousarray(w[sel]))


# r values are frozen after calibration by workloads/calibrate.py (realised mean degree printed
# there).  They are inputs of the workloads, chosen once.
CONFIGS = {
    "C1": Config("C1", "3pcf_uniform_n4096_nb10", "uniform", 4096, 1, 20.0, 10, r=115150,
                 notes="uniform, unweighted, small case the oracle finishes in well under a second"),
    "C2": Config("C2", "3pcf_ns_weighted_n1M_nb20", "neyman_scott", 1_000_000, 2, 100.0, 20, r=24310,
                 weighted=True, notes="Neyman-Scott 20k parents, sigma 0.002 L, fp64 weights"),
    "C3": Config("C3", "3pcf_uniform_n4M_m2250_nb30", "uniform", 4_000_000, 3, 2250.0, 30, r=54771,
                 notes="BAO-like scale, ~9e9 directed edges"),
    "C4": Config("C4", "4pcf_parity_ns_n500k_nb8", "neyman_scott", 500_000, 4, 40.0, 8, r=20366,
                 order=4, notes="parity-split 4pCF on clustered points"),
    "C5": Config("C5", "3pcf_mixed_n16M_m300_nb16", "mixed", 16_000_000, 5, 300.0, 16, r=11997,
                 notes="50% uniform + 50% Neyman-Scott; CSR larger than one hub tile"),
}


def get(key: str) -> Config:
    return CONFIGS[key]

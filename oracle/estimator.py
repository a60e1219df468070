"""Oracle of the data-minus-random estimators (GRAMSCI v2 §II.1, §III.3, §IV).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.  The composition is written out from the
pages' definitions, on top of the oracle's counts:

* radial bins equally spaced in r from r_min to r_max (§IV), as integer squared edges
  e_b = ceil(r_b^2) computed with exact rational arithmetic;
* one neighbour graph over the data followed by the randoms;
* signed, normalised weights (§II.1): w / sum_D w on data, -w / sum_R w on randoms, the sums
  correctly rounded (``math.fsum``); the random normalisation alone (0 on data) for the
  denominators;
* zeta = NNN / RRR (3pCF), zeta_even / zeta_odd = NNNN_even / NNNN_odd over RRRR, the internal
  xi = (signed pair sum) / RR (§III.3), the connected 4pCF zeta_even - disc(xi) (Eq. (4), (5)).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from oracle import Graph, disconnected_4pcf_s4


def linear_edges_sq(r_min: int, r_max: int, nbins: int) -> np.ndarray:
    """e_b = ceil(r_b^2) for r_b = r_min + b (r_max - r_min) / nbins (exact rationals)."""
    out = []
    for b in range(nbins + 1):
        r = Fraction(r_min) + Fraction(b * (r_max - r_min), nbins)
        out.append(math.ceil(r * r))
    return np.array(out, dtype=np.int64)


def estimator_weights(nd: int, w_data, nr: int, w_rand):
    """(signed weights, random-only weights) over data then randoms."""
    wd = np.ones(nd) if w_data is None else np.asarray(w_data, dtype=np.float64)
    wr = np.ones(nr) if w_rand is None else np.asarray(w_rand, dtype=np.float64)
    sd = math.fsum(wd.tolist())
    sr = math.fsum(wr.tolist())
    signed = np.concatenate([wd / sd if nd else wd, -(wr / sr)])
    rand = np.concatenate([np.zeros(nd), wr / sr])
    return signed, rand


def _ratio(a, b):
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.asarray(a, dtype=np.float64) / np.asarray(b, dtype=np.float64)


def compute_3pcf(xyz_data, w_data, xyz_rand, w_rand, edges_sq):
    """(zeta, NNN, RRR) per configuration."""
    xd = np.asarray(xyz_data, dtype=np.int32).reshape(-1, 3)
    xr = np.asarray(xyz_rand, dtype=np.int32).reshape(-1, 3)
    signed, rand = estimator_weights(len(xd), w_data, len(xr), w_rand)
    g = Graph(np.concatenate([xd, xr]), edges_sq)
    _, nnn, _, _ = g.count_3pcf(signed)
    _, rrr, _, _ = g.count_3pcf(rand)
    return _ratio(nnn, rrr), nnn, rrr


def compute_4pcf(xyz_data, w_data, xyz_rand, w_rand, edges_sq):
    """(zeta_even, zeta_odd, zeta_conn, xi) per S4 configuration (xi per bin)."""
    xd = np.asarray(xyz_data, dtype=np.int32).reshape(-1, 3)
    xr = np.asarray(xyz_rand, dtype=np.int32).reshape(-1, 3)
    signed, rand = estimator_weights(len(xd), w_data, len(xr), w_rand)
    g = Graph(np.concatenate([xd, xr]), edges_sq)
    nb = g.nbins
    _, _, ne, no, _ = g.count_4pcf_weighted(signed, s4=True)
    _, _, rr4, _, _ = g.count_4pcf_weighted(rand, s4=True)
    _, nn, _ = g.count_2pcf(signed)
    _, rr, _ = g.count_2pcf(rand)
    xi = _ratio(nn, rr)
    ze = _ratio(ne, rr4)
    zo = _ratio(no, rr4)
    return ze, zo, ze - disconnected_4pcf_s4(nb, xi), xi

"""Brute-force definitions for tiny point sets: every pair, every triple, every 4-set.

These pin the oracle.  They share no code with it: pairwise squared distances come from NumPy,
triangles and tetrahedra from exhaustive loops over index combinations, configuration ranks from
``itertools.combinations_with_replacement`` (which yields nondecreasing tuples in lexicographic
order), and weighted sums from exact rational arithmetic (``fractions.Fraction``).
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np


def sq_dists(xyz: np.ndarray) -> np.ndarray:
    x = xyz.astype(np.int64)
    d = x[:, None, :] - x[None, :, :]
    return (d * d).sum(axis=2)


def adjacency(xyz: np.ndarray, edges) -> tuple[np.ndarray, np.ndarray]:
    """(A bool [n,n], B int [n,n]) with A[i,j] iff i != j and e_0 <= d^2 < e_nb, B the bin."""
    e = np.asarray(edges, dtype=np.int64)
    d2 = sq_dists(xyz)
    n = xyz.shape[0]
    a = (d2 >= e[0]) & (d2 < e[-1]) & ~np.eye(n, dtype=bool)
    b = np.searchsorted(e, d2, side="right") - 1
    return a, b


def config_index(nbins: int, k: int) -> dict:
    return {t: r for r, t in enumerate(itertools.combinations_with_replacement(range(nbins), k))}


def triangles(xyz: np.ndarray, edges, w=None, hubs=None):
    """Every pairwise-adjacent triple once (only those whose smallest label is in ``hubs``, when
    given).  Returns (counts, weighted_fl, weighted_exact) where weighted_fl sums
    fl(fl(w1*w2)*w3) (weights ascending) exactly and rounds once, and weighted_exact is the
    correctly rounded exact real sum of w_i w_j w_k."""
    a, b = adjacency(xyz, edges)
    nb = len(edges) - 1
    idx = config_index(nb, 3)
    counts = np.zeros(len(idx), np.uint64)
    acc_fl = [Fraction(0)] * len(idx)
    acc_ex = [Fraction(0)] * len(idx)
    n = xyz.shape[0]
    hubset = None if hubs is None else {int(h) for h in hubs}
    for i, j, k in itertools.combinations(range(n), 3):
        if hubset is not None and i not in hubset:
            continue
        if a[i, j] and a[i, k] and a[j, k]:
            c = idx[tuple(sorted((int(b[i, j]), int(b[i, k]), int(b[j, k]))))]
            counts[c] += 1
            if w is not None:
                w1, w2, w3 = sorted((float(w[i]), float(w[j]), float(w[k])))
                acc_fl[c] += Fraction((w1 * w2) * w3)
                acc_ex[c] += Fraction(w[i]) * Fraction(w[j]) * Fraction(w[k])
    if w is None:
        return counts, None, None
    return counts, np.array([float(x) for x in acc_fl]), np.array([float(x) for x in acc_ex])


def _det3(m) -> int:
    return (m[0][0] * (m[1][1] * m[2][2] - m[1][2] * m[2][1])
            - m[0][1] * (m[1][0] * m[2][2] - m[1][2] * m[2][0])
            + m[0][2] * (m[1][0] * m[2][1] - m[1][1] * m[2][0]))


def chirality(pts) -> int:
    """Sign of the signed volume with vertices ordered by their summed squared edge lengths;
    0 if two such sums tie or the volume is zero.  ``pts`` are four integer 3-vectors."""
    p = [tuple(int(c) for c in q) for q in pts]
    key = [sum(sum((p[v][t] - p[u][t]) ** 2 for t in range(3)) for u in range(4)) for v in range(4)]
    order = sorted(range(4), key=lambda v: key[v])
    if len(set(key)) < 4:
        return 0
    o = [p[v] for v in order]
    m = [[o[r + 1][t] - o[0][t] for t in range(3)] for r in range(3)]
    v = _det3(m)
    return (v > 0) - (v < 0)


def cliques4(xyz: np.ndarray, edges):
    """Every pairwise-adjacent 4-set once: (even uint64[n_cfg], odd int64[n_cfg])."""
    a, b = adjacency(xyz, edges)
    nb = len(edges) - 1
    idx = config_index(nb, 6)
    even = np.zeros(len(idx), np.uint64)
    odd = np.zeros(len(idx), np.int64)
    n = xyz.shape[0]
    for q in itertools.combinations(range(n), 4):
        if all(a[u, v] for u, v in itertools.combinations(q, 2)):
            c = idx[tuple(sorted(int(b[u, v]) for u, v in itertools.combinations(q, 2)))]
            even[c] += 1
            odd[c] += chirality([xyz[v] for v in q])
    return even, odd


def s4_canonical(t) -> tuple:
    """Smallest relabelling of a 6-tuple of edge bins (edge order 01, 02, 03, 12, 13, 23)."""
    B = [[None] * 4 for _ in range(4)]
    for (u, v), x in zip(itertools.combinations(range(4), 2), t):
        B[u][v] = B[v][u] = x
    return min(tuple(B[p[u]][p[v]] for u, v in itertools.combinations(range(4), 2))
               for p in itertools.permutations(range(4)))


def s4_index(nbins: int) -> dict:
    """Canonical 6-tuple -> rank (lexicographic), over every orbit of nbins^6 tuples."""
    canon = sorted({s4_canonical(t) for t in itertools.product(range(nbins), repeat=6)})
    return {t: r for r, t in enumerate(canon)}


def cliques4_s4(xyz: np.ndarray, edges):
    """Every pairwise-adjacent 4-set once, binned by S4 configuration."""
    a, b = adjacency(xyz, edges)
    nb = len(edges) - 1
    idx = s4_index(nb)
    even = np.zeros(len(idx), np.uint64)
    odd = np.zeros(len(idx), np.int64)
    n = xyz.shape[0]
    for q in itertools.combinations(range(n), 4):
        if all(a[u, v] for u, v in itertools.combinations(q, 2)):
            c = idx[s4_canonical([int(b[u, v]) for u, v in itertools.combinations(q, 2)])]
            even[c] += 1
            odd[c] += chirality([xyz[v] for v in q])
    return even, odd


def pairs(xyz: np.ndarray, edges, w=None):
    """Every adjacent pair once: (counts uint64 [nb], exact weighted sums of fl(w_i w_j) as
    Fractions or None)."""
    from fractions import Fraction
    a, b = adjacency(xyz, edges)
    nb = len(edges) - 1
    counts = np.zeros(nb, np.uint64)
    acc = [Fraction(0)] * nb
    n = xyz.shape[0]
    for i in range(n):
        for j in range(i + 1, n):
            if a[i, j]:
                counts[b[i, j]] += 1
                if w is not None:
                    acc[b[i, j]] += Fraction(float(w[i]) * float(w[j]))  # one rounded product
    return counts, (acc if w is not None else None)


def disconnected_s4(t, xi) -> float:
    """Eq. (4) for one 6-tuple of edge bins (edge order of itertools.combinations(range(4), 2)):
    the sum over the three splits of the four vertices into two pairs."""
    e = {pair: x for pair, x in zip(itertools.combinations(range(4), 2), t)}
    total = 0.0
    for p, q in (((0, 1), (2, 3)), ((0, 2), (1, 3)), ((0, 3), (1, 2))):
        total += xi[e[p]] * xi[e[q]]
    return total


def cliques4_weighted(xyz: np.ndarray, edges, w, s4: bool = False, s: int | None = None):
    """Exact sums over every pairwise-adjacent 4-set of p = ((w1 w2) w3) w4 (weights ascending, each
    product rounded to a double) and of chirality * p: (even, odd) lists of Fractions.  With s, each
    p is first quantised to round_half_even(p * 2^s) / 2^s."""
    from fractions import Fraction
    a, b = adjacency(xyz, edges)
    nb = len(edges) - 1
    idx = s4_index(nb) if s4 else config_index(nb, 6)
    ev = [Fraction(0)] * len(idx)
    od = [Fraction(0)] * len(idx)
    n = xyz.shape[0]
    for q in itertools.combinations(range(n), 4):
        if all(a[u, v] for u, v in itertools.combinations(q, 2)):
            bins = [int(b[u, v]) for u, v in itertools.combinations(q, 2)]
            c = idx[s4_canonical(bins) if s4 else tuple(sorted(bins))]
            v = sorted(float(w[x]) for x in q)
            p = Fraction(((v[0] * v[1]) * v[2]) * v[3])
            if s is not None:
                p = Fraction(round(p * 2**s), 2**s)  # Fraction rounding: half to even
            ev[c] += p
            od[c] += chirality([xyz[x] for x in q]) * p
    return ev, od


def estimator_by_type(xd, wd, xr, wr, edges, order: int):
    """The Szapudi-Szalay / Landy-Szalay numerators written by catalogue type, in exact rationals:
    for each clique of the union graph (order 2: pairs, 3: triangles, 4: tetrahedra) with k random
    vertices, T_k += prod(w) / (S_D^(order-k) S_R^k); the numerator is sum_k (-1)^k T_k (for order
    3: DDD - 3 DDR + 3 DRR - RRR with each term normalised), the denominator T_order taken over the
    all-random cliques alone.  Order 4 also sums the chirality-signed terms.  Configurations: bins
    (order 2), sorted triples (3), S4 canonical tuples (4).  Returns (num, den, absum[, odd]) as
    lists of Fractions, absum the sum of |term| over every clique (for rounding bounds)."""
    xyz = np.concatenate([np.asarray(xd, np.int64).reshape(-1, 3),
                          np.asarray(xr, np.int64).reshape(-1, 3)])
    nd = len(xd)
    w = [Fraction(float(x)) for x in wd] + [Fraction(float(x)) for x in wr]
    sd = sum(w[:nd], Fraction(0))
    sr = sum(w[nd:], Fraction(0))
    a, b = adjacency(xyz, edges)
    nb = len(edges) - 1
    if order == 2:
        idx = {(x,): x for x in range(nb)}
    elif order == 3:
        idx = config_index(nb, 3)
    else:
        idx = s4_index(nb)
    num = [Fraction(0)] * len(idx)
    den = [Fraction(0)] * len(idx)
    ab = [Fraction(0)] * len(idx)
    odd = [Fraction(0)] * len(idx)
    for q in itertools.combinations(range(len(xyz)), order):
        if not all(a[u, v] for u, v in itertools.combinations(q, 2)):
            continue
        bins = [int(b[u, v]) for u, v in itertools.combinations(q, 2)]
        if order == 4:
            c = idx[s4_canonical(bins)]
        else:
            c = idx[tuple(sorted(bins))]
        k = sum(1 for v in q if v >= nd)
        t = Fraction(1)
        for v in q:
            t *= w[v]
        t /= sd ** (order - k) * sr ** k
        sgn = -1 if k % 2 else 1
        num[c] += sgn * t
        ab[c] += abs(t)
        if k == order:
            den[c] += t
        if order == 4:
            odd[c] += sgn * chirality([xyz[v] for v in q]) * t
    if order == 4:
        return num, den, ab, odd
    return num, den, ab

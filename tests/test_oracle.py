"""Pins for the CPU oracle, each against something other than the oracle itself: brute force over
every triple / 4-set, exact rational sums, closed forms, library routines (scipy sparse products,
networkx) and invariances that the definitions imply.  CPU only.
"""
from __future__ import annotations

import itertools
from math import comb

import numpy as np
import pytest

import brute
import oracle
from workloads import GRID, linear_edges_sq, rng_for

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def small_cloud(seed, n, box, nclump=0):
    """n points in a small box (so many are neighbours), optionally with coincident points."""
    rng = rng_for(seed)
    lo = rng.integers(0, GRID - box + 1)
    xyz = lo + rng.integers(0, box, size=(n, 3))
    if nclump:
        xyz[rng.integers(0, n, nclump)] = xyz[0]
    return np.ascontiguousarray(xyz.astype(np.int32))


def rank3(nb):
    return brute.config_index(nb, 3)


def rank6(nb):
    return brute.config_index(nb, 6)


# ------------------------------------------------------------------ graph vs brute force

@pytest.mark.parametrize("seed,n,box,nb", [(1, 40, 2000, 1), (2, 90, 3000, 4), (3, 120, (1 << 20) - 1, 7),
                                           (4, 70, 600, 3)])
def test_graph_matches_brute_force(seed, n, box, nb):
    xyz = small_cloud(seed, n, box, nclump=3)
    edges = linear_edges_sq(box // 2 + 7, nb)
    g = oracle.Graph(xyz, edges)
    rp, col, b = g.export()
    a, bb = brute.adjacency(xyz, edges)
    for i in range(n):
        row = col[rp[i]:rp[i + 1]]
        assert np.all(np.diff(row) > 0), "rows must be strictly ascending (Eq. 1)"
        np.testing.assert_array_equal(row, np.nonzero(a[i])[0])
        np.testing.assert_array_equal(b[rp[i]:rp[i + 1]], bb[i, row])


def test_graph_exact_boundaries():
    # points at squared distance exactly e_b land in bin b; exactly r^2 is not a neighbour
    edges = np.array([0, 100, 400, 900], np.int64)
    base = np.array([5000, 5000, 5000])
    pts = [base, base + [10, 0, 0], base + [0, 20, 0], base + [0, 0, 30], base + [0, 0, 29]]
    xyz = np.array(pts, np.int32)
    g = oracle.Graph(xyz, edges)
    rp, col, b = g.export()
    row0 = dict(zip(col[rp[0]:rp[1]].tolist(), b[rp[0]:rp[1]].tolist()))
    assert row0 == {1: 1, 2: 2, 4: 2}  # d2=100 -> bin 1, 400 -> bin 2, 900 excluded, 841 -> bin 2


# ------------------------------------------------------------------ 3pCF vs brute force

@pytest.mark.parametrize("seed,n,box,nb", [(11, 30, 1500, 1), (12, 80, 2500, 3), (13, 120, 4000, 6),
                                           (14, 60, 800, 10)])
def test_3pcf_matches_brute_force(seed, n, box, nb):
    xyz = small_cloud(seed, n, box, nclump=2)
    edges = linear_edges_sq(box // 2, nb)
    w = 0.5 + rng_for(seed + 100).random(n)
    cnt_b, wfl_b, wex_b = brute.triangles(xyz, edges, w)
    g = oracle.Graph(xyz, edges)
    cnt, wsum, s, walks = g.count_3pcf(w)
    np.testing.assert_array_equal(cnt, cnt_b)
    np.testing.assert_array_equal(wsum, wfl_b)  # same products, exact sum, one rounding
    np.testing.assert_allclose(wsum, wex_b, rtol=1e-15, atol=0)
    assert s == 55
    assert walks == g.nnz // 2
    cnt2, _, _, _ = g.count_3pcf(None, nthreads=1)
    np.testing.assert_array_equal(cnt2, cnt_b)


@pytest.mark.parametrize("seed,n,box,nb", [(15, 70, 2000, 3), (16, 110, 3500, 6)])
def test_forward_graph_matches_brute_force(seed, n, box, nb):
    # forward rows (neighbours above the row's label) are the upper half of the brute adjacency,
    # and the 3pCF / 4pCF / 2pCF counts on them are the brute-force ones
    xyz = small_cloud(seed, n, box, nclump=3)
    edges = linear_edges_sq(box // 2, nb)
    w = 0.5 + rng_for(seed + 300).random(n)
    gf = oracle.Graph(xyz, edges, forward_only=True)
    rp, col, b = gf.export()
    a, bb = brute.adjacency(xyz, edges)
    assert gf.nnz == int(a.sum()) // 2
    for i in range(n):
        want = np.nonzero(a[i])[0]
        want = want[want > i]
        np.testing.assert_array_equal(col[rp[i]:rp[i + 1]], want)
        np.testing.assert_array_equal(b[rp[i]:rp[i + 1]], bb[i, want])
    cnt_b, wfl_b, _ = brute.triangles(xyz, edges, w)
    cnt, wsum, _, walks = gf.count_3pcf(w)
    np.testing.assert_array_equal(cnt, cnt_b)
    np.testing.assert_array_equal(wsum, wfl_b)
    assert walks == gf.nnz
    ev_b, od_b = brute.cliques4(xyz, edges)
    ev, od, _ = gf.count_4pcf_parity()
    np.testing.assert_array_equal(ev, ev_b)
    np.testing.assert_array_equal(od, od_b)
    pc_b = brute.pairs(xyz, edges)[0]
    np.testing.assert_array_equal(gf.count_2pcf()[0], pc_b)


def test_hub_offsets_partition_the_count_by_smallest_label():
    # hub_stride / hub_offset select the triangles whose smallest label is offset mod stride
    xyz = small_cloud(17, 90, 2600, nclump=2)
    edges = linear_edges_sq(1300, 5)
    g = oracle.Graph(xyz, edges, forward_only=True)
    full = g.count_3pcf()[0]
    tot = np.zeros_like(full)
    for off in range(3):
        part = g.count_3pcf(hub_stride=3, hub_offset=off)[0]
        want = brute.triangles(xyz, edges, hubs=range(off, 90, 3))[0]
        np.testing.assert_array_equal(part, want)
        tot += part
    np.testing.assert_array_equal(tot, full)
    with pytest.raises(ValueError):
        g.count_3pcf(hub_stride=3, hub_offset=3)


def test_3pcf_signed_weights_match_brute_force():
    # signed weights as in the data-minus-random estimator (§II.1); products are exact at this scale
    xyz = small_cloud(21, 70, 2500)
    edges = linear_edges_sq(1300, 4)
    rng = rng_for(22)
    w = np.where(rng.random(70) < 0.5, -1.0, 1.0) * (0.25 + rng.random(70))
    cnt_b, wfl_b, _ = brute.triangles(xyz, edges, w)
    g = oracle.Graph(xyz, edges)
    cnt, wsum, s, _ = g.count_3pcf(w)
    np.testing.assert_array_equal(cnt, cnt_b)
    np.testing.assert_array_equal(wsum, wfl_b)


# ------------------------------------------------------------------ 4pCF vs brute force

@pytest.mark.parametrize("seed,n,box,nb", [(31, 24, 1500, 1), (32, 32, 2500, 2), (33, 36, 3000, 4)])
def test_4pcf_matches_brute_force(seed, n, box, nb):
    xyz = small_cloud(seed, n, box, nclump=0)
    edges = linear_edges_sq(box * 3 // 4, nb)
    even_b, odd_b = brute.cliques4(xyz, edges)
    g = oracle.Graph(xyz, edges)
    even, odd, ncl = g.count_4pcf_parity()
    np.testing.assert_array_equal(even, even_b)
    np.testing.assert_array_equal(odd, odd_b)
    assert ncl == int(even_b.sum())
    assert ncl > 0


# ------------------------------------------------------------------ closed forms

def test_clique_closed_form():
    # K points within a tiny ball: every pair is a neighbour in bin 0 -> C(K,3) / C(K,4)
    k = 25
    rng = rng_for(41)
    xyz = (500000 + rng.integers(0, 40, size=(k, 3))).astype(np.int32)
    edges = np.array([0, 10_000, 40_000], np.int64)
    g = oracle.Graph(xyz, edges)
    cnt, _, _, _ = g.count_3pcf()
    assert cnt[rank3(2)[(0, 0, 0)]] == comb(k, 3) and cnt.sum() == comb(k, 3)
    even, odd, _ = g.count_4pcf_parity()
    assert even[rank6(2)[(0,) * 6]] == comb(k, 4) and even.sum() == comb(k, 4)


def regular_tetra(a):
    return np.array([[0, 0, 0], [a, a, 0], [a, 0, a], [0, a, a]], np.int64)


def test_regular_tetrahedra_closed_form():
    # K isolated regular tetrahedra (all six d^2 = 2a^2): 4K triangles and K cliques in the
    # (b,b,b) / (b,)*6 configuration; every vertex key ties, so the odd channel is zero.
    a, k, nb = 1000, 12, 5
    edges = linear_edges_sq(2000, nb)  # r = 2000 > a*sqrt(2) = 1414
    b = int(np.searchsorted(edges, 2 * a * a, side="right") - 1)
    units = [regular_tetra(a) + [50_000 * (t + 1), 50_000, 70_000] for t in range(k)]
    xyz = np.concatenate(units).astype(np.int32)
    g = oracle.Graph(xyz, edges)
    cnt, _, _, _ = g.count_3pcf()
    assert cnt[rank3(nb)[(b, b, b)]] == 4 * k and cnt.sum() == 4 * k
    even, odd, _ = g.count_4pcf_parity()
    assert even[rank6(nb)[(b,) * 6]] == k and even.sum() == k
    assert np.all(odd == 0)


def test_isolated_pairs_have_no_triangles():
    # the pages' isolated-pair regression case (§IV.8): pairs far apart -> zero triangles
    xyz = np.array([[t * 10_000, 0, 0] for t in range(50)] + [[t * 10_000 + 5, 0, 0] for t in range(50)],
                   np.int32)
    g = oracle.Graph(xyz, linear_edges_sq(100, 3))
    assert g.nnz == 100
    cnt, _, _, _ = g.count_3pcf()
    assert cnt.sum() == 0


SCALENE = np.array([[0, 0, 0], [1000, 0, 0], [130, 1700, 0], [410, 520, 2300]], np.int64)


def proper_rotations():
    """The 24 proper rotations of the cube (signed permutation matrices with det +1)."""
    out = []
    for perm in itertools.permutations(range(3)):
        for signs in itertools.product((1, -1), repeat=3):
            m = np.zeros((3, 3), np.int64)
            for r, c in enumerate(perm):
                m[r, c] = signs[r]
            if round(np.linalg.det(m)) == 1:
                out.append(m)
    return out


def test_parity_injection_count_level_identity():
    # §IV.9: isolated scalene tetrahedra, n_l of one handedness and n_r mirrored; the odd channel
    # at the injected configuration is exactly +-(n_l - n_r), the even channel n_l + n_r.
    rots = proper_rotations()
    mirror = np.diag([-1, 1, 1])
    n_l, n_r = 17, 6
    units = []
    rng = rng_for(51)
    for t in range(n_l + n_r):
        rot = rots[int(rng.integers(len(rots)))]
        shape = SCALENE @ rot.T
        if t >= n_l:
            shape = shape @ mirror.T
        units.append(shape - shape.min(axis=0) + [40_000 * (t + 1), 200_000, 300_000])
    xyz = np.concatenate(units).astype(np.int32)
    nb = 6
    edges = linear_edges_sq(3200, nb)
    g = oracle.Graph(xyz, edges)
    even, odd, ncl = g.count_4pcf_parity()
    assert ncl == n_l + n_r
    c = int(np.nonzero(even)[0][0])
    assert even[c] == n_l + n_r and even.sum() == n_l + n_r
    assert abs(int(odd[c])) == n_l - n_r and int(odd.sum()) == int(odd[c])
    s = brute.chirality(SCALENE)
    assert s != 0 and int(odd[c]) == s * (n_l - n_r)


# ------------------------------------------------------------------ library cross-checks

def uniform_graph(seed=61, n=3000, box=200_000, r=20_000, nb=8):
    rng = rng_for(seed)
    xyz = (300_000 + rng.integers(0, box, size=(n, 3))).astype(np.int32)
    return xyz, linear_edges_sq(r, nb)


def test_total_equals_trace_a_cubed():
    # the histogram total is the number of triangles = trace(A^3)/6 (scipy sparse products)
    import scipy.sparse as sp
    xyz, edges = uniform_graph()
    g = oracle.Graph(xyz, edges)
    rp, col, _ = g.export()
    a = sp.csr_matrix((np.ones(col.size, np.int64), col, rp), shape=(g.n, g.n))
    t = int((a @ a).multiply(a).sum()) // 6
    cnt, _, _, _ = g.count_3pcf()
    assert int(cnt.sum()) == t and t > 1000
    # and = sum over undirected edges of common neighbours / 3
    deg = g.forward_degrees()
    assert int(deg.sum()) == g.nnz // 2


def test_totals_match_networkx():
    import networkx as nx
    xyz, edges = uniform_graph(seed=62, n=700, box=120_000, r=22_000)
    g = oracle.Graph(xyz, edges)
    rp, col, _ = g.export()
    G = nx.Graph()
    G.add_nodes_from(range(g.n))
    for i in range(g.n):
        G.add_edges_from((i, int(j)) for j in col[rp[i]:rp[i + 1]] if j > i)
    tri = sum(nx.triangles(G).values()) // 3
    k4 = sum(1 for c in nx.enumerate_all_cliques(G) if len(c) == 4)
    cnt, _, _, _ = g.count_3pcf()
    even, _, ncl = g.count_4pcf_parity()
    assert int(cnt.sum()) == tri and int(even.sum()) == k4 == ncl and k4 > 100


# ------------------------------------------------------------------ invariances

def cluster_set(seed=71, n=900):
    rng = rng_for(seed)
    centres = 200_000 + rng.integers(0, 400_000, size=(30, 3))
    xyz = centres[rng.integers(0, 30, n)] + rng.normal(0, 4000, size=(n, 3))
    return np.clip(np.rint(xyz), 0, GRID - 1).astype(np.int32)


def all_outputs(xyz, edges, w):
    g = oracle.Graph(xyz, edges)
    cnt, ws, _, _ = g.count_3pcf(w)
    even, odd, _ = g.count_4pcf_parity()
    return cnt, ws, even, odd


def test_relabelling_invariance():
    xyz = cluster_set()
    edges = linear_edges_sq(9000, 6)
    w = 0.5 + rng_for(72).random(xyz.shape[0])
    base = all_outputs(xyz, edges, w)
    perm = rng_for(73).permutation(xyz.shape[0])
    other = all_outputs(np.ascontiguousarray(xyz[perm]), edges, w[perm])
    for x, y in zip(base, other):
        np.testing.assert_array_equal(x, y)
    assert base[3].any(), "need a non-zero odd channel for this check to mean anything"


def test_mirror_and_axis_symmetries():
    xyz = cluster_set(74)
    edges = linear_edges_sq(9000, 6)
    cnt, _, even, odd = all_outputs(xyz, edges, None)
    assert np.abs(odd).sum() > 0
    mirrored = xyz.copy()
    mirrored[:, 0] = GRID - 1 - mirrored[:, 0]
    c2, _, e2, o2 = all_outputs(mirrored, edges, None)
    np.testing.assert_array_equal(c2, cnt)
    np.testing.assert_array_equal(e2, even)
    np.testing.assert_array_equal(o2, -odd)
    swapped = np.ascontiguousarray(xyz[:, [1, 0, 2]])
    _, _, e3, o3 = all_outputs(swapped, edges, None)
    np.testing.assert_array_equal(e3, even)
    np.testing.assert_array_equal(o3, -odd)
    cyc = np.ascontiguousarray(xyz[:, [1, 2, 0]])
    _, _, e4, o4 = all_outputs(cyc, edges, None)
    np.testing.assert_array_equal(e4, even)
    np.testing.assert_array_equal(o4, odd)


def test_translation_and_scaling():
    xyz = cluster_set(75)
    edges = linear_edges_sq(9000, 6)
    cnt, _, even, odd = all_outputs(xyz, edges, None)
    shift = np.array([1234, -5678, 91011])
    moved = xyz.astype(np.int64) + shift
    assert moved.min() >= 0 and moved.max() < GRID
    c2, _, e2, o2 = all_outputs(moved.astype(np.int32), edges, None)
    np.testing.assert_array_equal(c2, cnt)
    np.testing.assert_array_equal(e2, even)
    np.testing.assert_array_equal(o2, odd)
    half = (xyz // 2 * 2).astype(np.int64)  # even coordinates, then scale up by 2 with edges x4
    ch, _, eh, oh = all_outputs((half // 2).astype(np.int32), edges, None)
    cd, _, ed, od = all_outputs(half.astype(np.int32), edges * 4, None)
    np.testing.assert_array_equal(ch, cd)
    np.testing.assert_array_equal(eh, ed)
    np.testing.assert_array_equal(oh, od)


def test_constant_weights():
    xyz = cluster_set(76, 600)
    edges = linear_edges_sq(9000, 5)
    g = oracle.Graph(xyz, edges)
    cnt, w1, _, _ = g.count_3pcf(np.ones(g.n))
    np.testing.assert_array_equal(w1, cnt.astype(np.float64))
    _, w2, s, _ = g.count_3pcf(np.full(g.n, 2.0))
    np.testing.assert_array_equal(w2, 8.0 * cnt.astype(np.float64))
    _, wz, _, _ = g.count_3pcf(np.zeros(g.n))
    assert np.all(wz == 0)


def test_exact_sums_are_the_rounded_weighted_output():
    xyz = cluster_set(77, 500)
    edges = linear_edges_sq(9000, 4)
    w = 0.5 + rng_for(78).random(xyz.shape[0])
    g = oracle.Graph(xyz, edges)
    cnt, sums, s = g.count_3pcf_exact(w)
    _, wsum, s2, _ = g.count_3pcf(w)
    assert s == s2 == 55
    for c in range(cnt.size):
        assert wsum[c] == float(sums[c]) * 2.0 ** -s  # Python int -> float is correctly rounded


def test_hub_stride_partitions_by_smallest_label():
    xyz, edges = uniform_graph(seed=79, n=1500)
    g = oracle.Graph(xyz, edges)
    full, _, _, walks = g.count_3pcf()
    part, _, _, w2 = g.count_3pcf(hub_stride=3)
    assert np.all(part <= full) and 0 < part.sum() < full.sum() and 0 < w2 < walks


@pytest.mark.parametrize("seed,n,box,nb", [(81, 60, 2000, 3), (82, 110, 3500, 6)])
def test_hub_counts_match_brute_force(seed, n, box, nb):
    # the graph-free per-hub definition, summed over every hub, is the brute-force 3pCF
    xyz = small_cloud(seed, n, box, nclump=2)
    edges = linear_edges_sq(box // 2, nb)
    w = 0.5 + rng_for(seed + 100).random(n)
    cnt_b, wfl_b, _ = brute.triangles(xyz, edges, w)
    cnt, wsum, s = oracle.count_3pcf_hubs(xyz, edges, np.arange(n), w)
    np.testing.assert_array_equal(cnt, cnt_b)
    np.testing.assert_array_equal(wsum, wfl_b)
    assert s == 55


def test_hub_counts_agree_with_the_merge_walk_on_hub_subsets():
    # two independent routes to the triangles of a hub subset: the merge-walk over the graph (hubs
    # with label % 3 == 0) and the pair test from coordinates; subsets of hubs add up
    xyz, edges = uniform_graph(seed=83, n=1500)
    w = 0.5 + rng_for(84).random(xyz.shape[0])
    g = oracle.Graph(xyz, edges)
    part, wpart, s0, _ = g.count_3pcf(w, hub_stride=3)
    hubs = np.arange(0, xyz.shape[0], 3)
    cnt, wsum, s = oracle.count_3pcf_hubs(xyz, edges, hubs, w)
    np.testing.assert_array_equal(cnt, part)
    np.testing.assert_array_equal(wsum, wpart)
    assert s == s0
    rng = rng_for(85)
    perm = rng.permutation(hubs)
    a, wa, _ = oracle.count_3pcf_hubs(xyz, edges, perm[: perm.size // 3], w)
    b, wb, _ = oracle.count_3pcf_hubs(xyz, edges, perm[perm.size // 3:], w)
    np.testing.assert_array_equal(a + b, cnt)


def test_hub_counts_reject_bad_hub_lists():
    xyz, edges = uniform_graph(seed=86, n=200)
    for hubs in ([0, 5, 5], [-1], [200]):
        with pytest.raises(ValueError):
            oracle.count_3pcf_hubs(xyz, edges, hubs)
    cnt, _, _ = oracle.count_3pcf_hubs(xyz, edges, [])
    assert cnt.sum() == 0


# ------------------------------------------------------------------ S4 configurations (§III.3)

def test_s4_configuration_counts_are_the_orbit_counts():
    # Burnside over S4 acting on the 6 edges of K4 (cycle types 1^6, 6 x 1^2 2^2, 3 x 1^2 2^2,
    # 8 x 3^2, 6 x 2 4): (k^6 + 9 k^4 + 14 k^2) / 24
    for k in range(1, 9):
        assert oracle.num_configs_s4(k) == (k**6 + 9 * k**4 + 14 * k**2) // 24
    assert oracle.num_configs_s4(4) == 276 and oracle.num_configs_s4(8) == 12496  # [G] §V.2


@pytest.mark.parametrize("nb", [1, 2, 3])
def test_s4_canonical_tuples(nb):
    got = [tuple(r) for r in oracle.config_bins_s4(nb)]
    assert got == list(brute.s4_index(nb))  # same orbits, same lexicographic order


def test_s4_realizable_mask_matches_the_pages():
    # [G] §V.2: 4 linear bins on 20 < r < 65 leave 178 of 276 configurations realizable.  In
    # quarter units the edges 80, 125, 170, 215, 260 are integers; the test is scale-free.
    edges = np.array([80, 125, 170, 215, 260], np.int64) ** 2
    mask = oracle.config_realizable_s4(4, edges)
    assert mask.size == 276 and int(mask.sum()) == 178
    rank = {tuple(r): i for i, r in enumerate(oracle.config_bins_s4(4))}
    assert mask[rank[(0, 0, 0, 0, 0, 2)]] == 0  # five edges near 26 and one near 48
    for b in range(4):
        assert mask[rank[(b,) * 6]] == 1  # regular tetrahedra


@pytest.mark.parametrize("seed,n,box,nb", [(41, 26, 1500, 1), (42, 32, 2500, 2), (43, 36, 3000, 3)])
def test_4pcf_s4_matches_brute_force(seed, n, box, nb):
    xyz = small_cloud(seed, n, box, nclump=2)
    edges = linear_edges_sq(box // 2, nb)
    e_b, o_b = brute.cliques4_s4(xyz, edges)
    e, o, ncl = oracle.Graph(xyz, edges).count_4pcf_parity(s4=True)
    np.testing.assert_array_equal(e, e_b)
    np.testing.assert_array_equal(o, o_b)
    assert ncl == int(e_b.sum())


def test_4pcf_s4_folds_onto_sorted_tuples():
    # every S4 configuration lies in exactly one sorted-6-tuple class
    xyz, edges = uniform_graph(seed=44, n=3000, r=30_000, nb=4)
    g = oracle.Graph(xyz, edges)
    e4, o4, _ = g.count_4pcf_parity(s4=True)
    es, os_, _ = g.count_4pcf_parity()
    cls = {t: r for r, t in enumerate(itertools.combinations_with_replacement(range(4), 6))}
    fe = np.zeros_like(es)
    fo = np.zeros_like(os_)
    for c, t in enumerate(oracle.config_bins_s4(4)):
        k = cls[tuple(sorted(int(x) for x in t))]
        fe[k] += e4[c]
        fo[k] += o4[c]
    np.testing.assert_array_equal(fe, es)
    np.testing.assert_array_equal(fo, os_)
    assert es.sum() > 0


@pytest.mark.parametrize("s4", [False, True])
@pytest.mark.parametrize("seed,n,box,nb", [(45, 30, 2000, 2), (46, 36, 3000, 3)])
def test_4pcf_weighted_matches_brute_force(seed, n, box, nb, s4):
    xyz = small_cloud(seed, n, box, nclump=2)
    edges = linear_edges_sq(box // 2, nb)
    rng = rng_for(seed + 100)
    w = np.where(rng.random(n) < 0.3, -1.0, 1.0) * (0.5 + rng.random(n))  # signed weights
    import math
    a = float(np.abs(w).max())
    s_want = 57 - math.frexp(((a * a) * a) * a)[1]
    ev_b, od_b = brute.cliques4_weighted(xyz, edges, w, s4, s=s_want)
    g = oracle.Graph(xyz, edges)
    e, o, ew, ow, s = g.count_4pcf_weighted(w, s4=s4)
    assert s == s_want
    np.testing.assert_array_equal(ew, [float(x) for x in ev_b])  # exact quantised sums
    np.testing.assert_array_equal(ow, [float(x) for x in od_b])
    # against the unquantised products: each term moves by at most 2^-(s+1)
    ev_x, od_x = brute.cliques4_weighted(xyz, edges, w, s4)
    ncl = max(int(e.sum()), 1)
    np.testing.assert_allclose(ew, [float(x) for x in ev_x], rtol=0, atol=ncl * 2.0 ** -s)
    np.testing.assert_allclose(ow, [float(x) for x in od_x], rtol=0, atol=ncl * 2.0 ** -s)
    e0, o0, _ = g.count_4pcf_parity(s4=s4)
    np.testing.assert_array_equal(e, e0)
    np.testing.assert_array_equal(o, o0)
    assert e.sum() > 0


def test_4pcf_weighted_constant_weights():
    xyz, edges = uniform_graph(seed=47, n=2000, r=30_000, nb=4)
    g = oracle.Graph(xyz, edges)
    e, o, ew, ow, _ = g.count_4pcf_weighted(np.ones(2000))
    np.testing.assert_array_equal(ew, e.astype(np.float64))
    np.testing.assert_array_equal(ow, o.astype(np.float64))
    _, _, ew2, ow2, _ = g.count_4pcf_weighted(np.full(2000, 2.0))
    np.testing.assert_array_equal(ew2, 16.0 * e)
    np.testing.assert_array_equal(ow2, 16.0 * o)


# ------------------------------------------------------------------ 2pCF, disconnected 4pCF (§III.3)

@pytest.mark.parametrize("seed,n,box,nb", [(51, 60, 2000, 3), (52, 120, 4000, 7)])
def test_2pcf_matches_brute_force(seed, n, box, nb):
    xyz = small_cloud(seed, n, box, nclump=3)
    edges = linear_edges_sq(box // 2, nb)
    w = 0.5 + rng_for(seed + 100).random(n)
    cnt_b, acc_b = brute.pairs(xyz, edges, w)
    g = oracle.Graph(xyz, edges)
    cnt, wsum, s = g.count_2pcf(w)
    np.testing.assert_array_equal(cnt, cnt_b)
    np.testing.assert_array_equal(wsum, [float(x) for x in acc_b])  # exact sum, one rounding
    assert int(cnt.sum()) == g.nnz // 2
    assert s == 55  # max |w| near 1.49: M = fl(a * a) in [2, 4), s = 57 - 2
    c1, w1, _ = g.count_2pcf(np.ones(n))
    np.testing.assert_array_equal(w1, c1.astype(np.float64))


def test_2pcf_signed_weights_are_the_landy_szalay_numerator():
    # data weights 1/N_D and random weights -1/N_R: sum of w_i w_j over pairs = DD/N_D^2
    # - DR/(N_D N_R) + RR/N_R^2 per bin (DR counted once per data-random pair)
    rng = rng_for(53)
    nd, nr = 90, 130
    xyz = small_cloud(54, nd + nr, 3000)
    edges = linear_edges_sq(1500, 5)
    w = np.concatenate([np.full(nd, 1.0 / nd), np.full(nr, -1.0 / nr)])
    cnt, wsum, _ = oracle.Graph(xyz, edges).count_2pcf(w)
    a, b = brute.adjacency(xyz, edges)
    dd = np.zeros(5); dr = np.zeros(5); rr = np.zeros(5)
    for i in range(nd + nr):
        for j in range(i + 1, nd + nr):
            if a[i, j]:
                (dd if j < nd else (dr if i < nd else rr))[b[i, j]] += 1
    np.testing.assert_allclose(wsum, dd / nd**2 - dr / (nd * nr) + rr / nr**2, rtol=1e-13, atol=1e-16)


def test_disconnected_4pcf_matches_the_pair_splits():
    rng = rng_for(55)
    for nb in (1, 3, 4):
        xi = rng.normal(size=nb)
        disc = oracle.disconnected_4pcf_s4(nb, xi)
        bins = oracle.config_bins_s4(nb)
        want = np.array([brute.disconnected_s4(t, xi) for t in bins])
        np.testing.assert_allclose(disc, want, rtol=1e-15, atol=1e-15)
        # a relabelled tuple of the same configuration gives the same value (S4 invariance)
        for t in bins[:20]:
            for p in rng.permutation(list(itertools.permutations(range(4))))[:5]:
                B = np.zeros((4, 4), int)
                for (u, v), x in zip(itertools.combinations(range(4), 2), t):
                    B[u, v] = B[v, u] = x
                t2 = [B[p[u], p[v]] for u, v in itertools.combinations(range(4), 2)]
                assert brute.disconnected_s4(t2, xi) == pytest.approx(brute.disconnected_s4(t, xi), abs=1e-15)
    np.testing.assert_allclose(oracle.disconnected_4pcf_s4(4, np.full(4, 0.3)), 3 * 0.09, rtol=1e-15)


def test_degenerate_inputs():
    edges = linear_edges_sq(1000, 3)
    for n in (0, 1, 2):
        xyz = np.zeros((n, 3), np.int32)
        g = oracle.Graph(xyz, edges)
        cnt, _, _, _ = g.count_3pcf()
        even, odd, _ = g.count_4pcf_parity()
        assert cnt.sum() == 0 and even.sum() == 0
    with pytest.raises(ValueError):
        oracle.Graph(np.array([[GRID, 0, 0]], np.int32), edges)
    with pytest.raises(ValueError):
        oracle.Graph(np.zeros((3, 3), np.int32), np.array([0, 5, 5], np.int64))


def test_coplanar_tetrahedra_have_no_chirality():
    # §III.2: zero signed volume -> zero weight in the odd channel, even channel unaffected.
    # Scalene planar quadrilaterals (distinct vertex keys), several orientations.
    planar = np.array([[0, 0, 0], [1000, 0, 0], [130, 1700, 0], [900, 1300, 0]], np.int64)
    assert len({sum(int(((planar[v] - planar[u]) ** 2).sum()) for u in range(4)) for v in range(4)}) == 4
    units = []
    for t, rot in enumerate(proper_rotations()[:10]):
        shape = planar @ rot.T
        units.append(shape - shape.min(axis=0) + [60_000 * (t + 1), 300_000, 300_000])
    xyz = np.concatenate(units).astype(np.int32)
    g = oracle.Graph(xyz, linear_edges_sq(3000, 4))
    even, odd, ncl = g.count_4pcf_parity()
    assert ncl == 10 and even.sum() == 10 and np.all(odd == 0)


# ------------------------------------------------------------------ estimators (§II.1, §III.3)

from fractions import Fraction  # noqa: E402

from oracle import estimator as est  # noqa: E402


@pytest.mark.parametrize("rmin,rmax,nb", [(0, 1000, 3), (7, 31, 4), (1, 100, 16), (3, 4, 1),
                                          (50_000, 1 << 21, 255)])
def test_linear_edges_sq_bins_are_equal_in_r(rmin, rmax, nb):
    # an integer squared distance d2 lies in bin b exactly when r_b <= sqrt(d2) < r_{b+1},
    # r_b = rmin + b (rmax - rmin) / nb: compare with that inequality in integers,
    # (d2 nb^2 >= (rmin nb + b (rmax - rmin))^2), at and around every edge
    e = est.linear_edges_sq(rmin, rmax, nb)
    for b in range(nb + 1):
        rb_nb = rmin * nb + b * (rmax - rmin)
        for d2 in {max(int(e[b]) + k, 0) for k in (-2, -1, 0, 1)}:
            assert (d2 >= e[b]) == (d2 * nb * nb >= rb_nb * rb_nb)
    if rmin == 0:
        np.testing.assert_array_equal(e, linear_edges_sq(rmax, nb))


def estimator_set(seed, nd, nr, box):
    rng = rng_for(seed)
    xd = small_cloud(seed + 1, nd, box // 3)
    lo = xd.min(axis=0) - box // 3
    xr = np.ascontiguousarray((lo + rng.integers(0, box, size=(nr, 3))).clip(0, GRID - 1)
                              .astype(np.int32))
    wd = rng.uniform(0.5, 2.0, nd)
    wr = rng.uniform(0.5, 2.0, nr)
    return xd, wd, xr, wr


def _close(got, want, absum, tol=1e-13):
    for c, (g, x, a) in enumerate(zip(got, want, absum)):
        assert abs(Fraction(float(g)) - x) <= tol * a + Fraction(1, 2**1074), c


@pytest.mark.parametrize("seed,nd,nr,nb,rmin", [(81, 14, 18, 3, 100), (82, 10, 20, 2, 0)])
def test_3pcf_estimator_is_the_szapudi_szalay_combination(seed, nd, nr, nb, rmin):
    xd, wd, xr, wr = estimator_set(seed, nd, nr, 1800)
    edges = est.linear_edges_sq(rmin, 1200, nb)
    zeta, nnn, rrr = est.compute_3pcf(xd, wd, xr, wr, edges)
    num, den, ab = brute.estimator_by_type(xd, wd, xr, wr, edges, 3)
    assert sum(1 for x in den if x) >= 3
    _close(nnn, num, ab)
    _close(rrr, den, den)
    for c in range(len(num)):
        if den[c]:
            assert zeta[c] == pytest.approx(float(num[c] / den[c]), rel=1e-11, abs=1e-11 * float(ab[c] / den[c]))
        else:
            assert not np.isfinite(zeta[c])


@pytest.mark.parametrize("seed,nd,nr,nb", [(83, 10, 14, 2), (84, 8, 16, 3)])
def test_4pcf_estimator_is_the_signed_combination(seed, nd, nr, nb):
    xd, wd, xr, wr = estimator_set(seed, nd, nr, 1500)
    edges = est.linear_edges_sq(50, 1100, nb)
    ze, zo, zc, xi = est.compute_4pcf(xd, wd, xr, wr, edges)
    num, den, ab, odd = brute.estimator_by_type(xd, wd, xr, wr, edges, 4)
    pnum, pden, pab = brute.estimator_by_type(xd, wd, xr, wr, edges, 2)
    assert sum(1 for x in den if x) >= 3 and any(odd)
    xi_want = [float(n / d) for n, d in zip(pnum, pden)]
    np.testing.assert_allclose(xi, xi_want, rtol=1e-12)
    bins = oracle.config_bins_s4(nb)
    for c in range(len(num)):
        if den[c]:
            scale = float(ab[c] / den[c])
            assert ze[c] == pytest.approx(float(num[c] / den[c]), abs=1e-11 * scale)
            assert zo[c] == pytest.approx(float(odd[c] / den[c]), abs=1e-11 * scale)
            assert zc[c] == pytest.approx(float(num[c] / den[c]) - brute.disconnected_s4(bins[c], xi_want),
                                          abs=1e-11 * (scale + 3 * max(map(abs, xi_want)) ** 2))
        else:
            assert not np.isfinite(ze[c])


def test_estimators_vanish_when_data_are_the_randoms():
    # D = R with unit weights: every clique with a data vertex has a twin with the random copy
    # (same positions, twins at distance 0 < r_min never adjacent) and the opposite sign, and the
    # normalised weights all have one magnitude, so every product rounds the same whatever the
    # order and signs of its factors, and the sums cancel exactly
    x = small_cloud(86, 24, 600)
    edges = est.linear_edges_sq(20, 500, 3)
    zeta, nnn, rrr = est.compute_3pcf(x, None, x, None, edges)
    assert rrr.max() > 0
    np.testing.assert_array_equal(nnn, 0.0)
    ze, zo, zc, xi = est.compute_4pcf(x[:18], None, x[:18], None, edges)
    np.testing.assert_array_equal(xi, 0.0)
    fin = np.isfinite(ze)
    assert fin.sum() > 3
    np.testing.assert_array_equal(ze[fin], 0.0)
    np.testing.assert_array_equal(zo[fin], 0.0)
    np.testing.assert_array_equal(zc[fin], 0.0)


def test_estimator_weights_are_normalised():
    rng = rng_for(87)
    wd, wr = rng.uniform(0.1, 3, 50), rng.uniform(0.1, 3, 70)
    s, r = est.estimator_weights(50, wd, 70, wr)
    assert Fraction(sum(map(Fraction, s[:50]))) == pytest.approx(1, abs=1e-15)
    assert Fraction(sum(map(Fraction, s[50:]))) == pytest.approx(-1, abs=1e-15)
    assert (r[:50] == 0).all() and np.array_equal(r[50:], -s[50:])


# ------------------------------------------------------------------ generated point sets

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), n=st.integers(0, 60), box=st.integers(1, 3000),
       nb=st.integers(1, 6), clump=st.integers(0, 6))
def test_generated_sets_match_brute_force(seed, n, box, nb, clump):
    # arbitrary small clouds (coincident points, tiny boxes, edges at exact distances): the
    # oracle's graph, triangles and tetrahedra with parity equal the exhaustive definitions
    xyz = small_cloud(seed, n, box, min(clump, n))
    r = max(1, box // 2)
    edges = linear_edges_sq(r, nb) if r * r >= nb * nb else linear_edges_sq(nb, nb)
    g = oracle.Graph(xyz, edges)
    a, _ = brute.adjacency(xyz, edges)
    assert g.nnz == int(a.sum())
    c, _, _, _ = g.count_3pcf()
    bc, _, _ = brute.triangles(xyz, edges)
    np.testing.assert_array_equal(c, bc)
    if n <= 30:
        e, o, _ = g.count_4pcf_parity()
        be, bo = brute.cliques4(xyz, edges)
        np.testing.assert_array_equal(e, be)
        np.testing.assert_array_equal(o, bo)

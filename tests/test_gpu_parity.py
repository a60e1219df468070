"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Unweighted counts, even and odd channels: bit-exact.  Weighted sums: bit-exact as well (both sides
sum the same fixed-point products exactly and round once); the stated bar is 1e-12 relative per
configuration, which bit-exactness implies.
"""
from __future__ import annotations

import functools
import itertools

import numpy as np
import pytest

import graph_triangle_counting_amd as gtc
import oracle
import workloads
from gpu_common import (clustered, edge_set_from_gpu, edge_set_from_oracle, hip_3pcf, hip_4pcf,
                        host_internal_order, to_gpu, uniform)
from workloads import GRID, linear_edges_sq, rng_for

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ graph

@pytest.mark.parametrize("kind,seed,n,r,nb", [
    ("uniform", 1, 3000, 60_000, 5),
    ("clustered", 2, 6000, 9_000, 7),
    ("uniform", 3, 700, 600_000, 3),     # two cells per axis (g < 3 path)
    ("clustered", 4, 5000, 300, 2),      # tiny radius: grid capped, cells much larger than r
])
def test_graph_matches_oracle(gpu_available, kind, seed, n, r, nb):
    say("graph", kind, seed, n, r, nb)
    xyz = uniform(seed, n) if kind == "uniform" else clustered(seed, n, 40, 3000)
    edges = linear_edges_sq(r, nb)
    g = gtc.Graph(to_gpu(xyz), edges)
    got = edge_set_from_gpu(g)
    st = g.stats()
    g.close()
    want = edge_set_from_oracle(oracle.Graph(xyz, edges))
    assert st["edges"] == want.shape[0]
    np.testing.assert_array_equal(got, want)


def test_graph_split_layout_exports_the_same_edges(gpu_available, monkeypatch):
    # a label array plus a bin array (the layout of graphs above 2^24 points) holds the same graph
    xyz = clustered(5, 8000, 40, 3000)
    edges = linear_edges_sq(9_000, 6)
    want = edge_set_from_oracle(oracle.Graph(xyz, edges))
    monkeypatch.setenv("GTC_CSR_LAYOUT", "split")
    g = gtc.Graph(to_gpu(xyz), edges)
    got = edge_set_from_gpu(g)
    g.close()
    np.testing.assert_array_equal(got, want)


# ------------------------------------------------------------------ 3pCF

CASES_3 = [
    ("uniform", 11, 2000, 90_000, 1, False),
    ("uniform", 12, 20_000, 40_000, 10, True),
    ("clustered", 13, 30_000, 12_000, 20, True),
    ("clustered", 14, 12_000, 4_000, 30, False),
    ("uniform", 15, 5000, 150_000, 64, True),
]


@pytest.mark.parametrize("kind,seed,n,r,nb,weighted", CASES_3)
def test_3pcf_matches_oracle(gpu_available, kind, seed, n, r, nb, weighted):
    say("3pcf", kind, seed, n, r, nb, weighted)
    xyz = uniform(seed, n) if kind == "uniform" else clustered(seed, n, 60, 2500)
    edges = linear_edges_sq(r, nb)
    w = 0.5 + rng_for(seed + 1000).random(n) if weighted else None
    c, ws, st = hip_3pcf(xyz, edges, w)
    oc, ows, s, walks = oracle.Graph(xyz, edges).count_3pcf(w)
    np.testing.assert_array_equal(c, oc)
    assert st["triangles"] == int(oc.sum()) and oc.sum() > 0
    if weighted:
        assert st["weight_scale"] == s
        np.testing.assert_array_equal(ws, ows)


@pytest.mark.parametrize("layout", ["packed", "split"])
@pytest.mark.parametrize("mode", ["flat", "banded"])
@pytest.mark.parametrize("kind,seed,n,r,nb", [
    ("uniform", 16, 20_000, 40_000, 1),
    ("clustered", 17, 30_000, 12_000, 7),
    ("uniform", 18, 12_000, 60_000, 16),
    ("uniform", 20, 12_000, 60_000, 30),
    ("clustered", 21, 30_000, 12_000, 32),
])
def test_3pcf_unsorted_histogram(gpu_available, monkeypatch, layout, mode, kind, seed, n, r, nb):
    # the histogram over the unsorted bin triple (nb^3 bins, folded onto ranks at each exchange)
    # gives the oracle's counts in both walk modes and layouts
    say("3pcf unsorted", mode, layout, kind, seed, n, r, nb)
    monkeypatch.setenv("GTC_TRIPLET_MODE", mode)
    monkeypatch.setenv("GTC_TRIPLET_HIST", "unsorted")
    if layout == "split":
        monkeypatch.setenv("GTC_CSR_LAYOUT", "split")
    xyz = uniform(seed, n) if kind == "uniform" else clustered(seed, n, 60, 2500)
    edges = linear_edges_sq(r, nb)
    c, _, st = hip_3pcf(xyz, edges)
    assert st["launch_mode"] & 3 == (1 if mode == "banded" else 0) | 2
    oc, _, _, _ = oracle.Graph(xyz, edges).count_3pcf()
    np.testing.assert_array_equal(c, oc)
    assert oc.sum() > 0


@pytest.mark.parametrize("mode", ["flat", "banded"])
@pytest.mark.parametrize("copies", ["1", "2"])
def test_3pcf_unsorted_histogram_copies(gpu_available, monkeypatch, mode, copies):
    # the unsorted histogram in one copy, or two (odd lanes add to the second; both are folded
    # onto ranks at each exchange)
    say("3pcf copies", mode, copies)
    monkeypatch.setenv("GTC_TRIPLET_MODE", mode)
    monkeypatch.setenv("GTC_TRIPLET_HIST", "unsorted")
    monkeypatch.setenv("GTC_TRIPLET_COPIES", copies)
    monkeypatch.setenv("GTC_TRIPLET_FLUSH_AT", "5000")
    xyz = clustered(23, 30_000, 60, 2500)
    edges = linear_edges_sq(12_000, 16)
    c, _, st = hip_3pcf(xyz, edges)
    assert st["launch_mode"] & 2
    oc, _, _, _ = oracle.Graph(xyz, edges).count_3pcf()
    np.testing.assert_array_equal(c, oc)
    assert oc.sum() > 0


@pytest.mark.parametrize("mode", ["flat", "banded"])
@pytest.mark.parametrize("copies", ["1", "2"])
def test_3pcf_weighted_histogram_copies(gpu_available, monkeypatch, mode, copies):
    # the weighted LDS histogram with one copy of its counts and low limbs, or two (odd lanes add
    # to the second; the exchanges sum both), with frequent exchanges
    say("3pcf weighted copies", mode, copies)
    monkeypatch.setenv("GTC_TRIPLET_MODE", mode)
    monkeypatch.setenv("GTC_TRIPLET_COPIES", copies)
    monkeypatch.setenv("GTC_TRIPLET_FLUSH_AT", "5000")
    xyz = clustered(24, 20_000, 60, 2500)
    edges = linear_edges_sq(12_000, 16)
    w = 0.5 + rng_for(1024).random(20_000)
    c, ws, st = hip_3pcf(xyz, edges, w)
    assert st["launch_mode"] & 1 == (1 if mode == "banded" else 0)
    oc, ows, _, _ = oracle.Graph(xyz, edges).count_3pcf(w)
    assert oc.sum() > 100 * 5000
    np.testing.assert_array_equal(c, oc)
    np.testing.assert_array_equal(ws, ows)


@pytest.mark.parametrize("layout", ["packed", "split"])
@pytest.mark.parametrize("deep,seed,nb", [("0", 20, 30), ("1", 18, 16), ("1", 22, 30)])
def test_3pcf_deep_load_pipeline(gpu_available, monkeypatch, layout, deep, seed, nb):
    # the banded unsorted-histogram walk with twice the loads in flight per lane (chosen by itself
    # when the histogram leaves room for 16 waves per CU; forced both ways here)
    say("3pcf deep", deep, layout, seed, nb)
    monkeypatch.setenv("GTC_TRIPLET_MODE", "banded")
    monkeypatch.setenv("GTC_TRIPLET_HIST", "unsorted")
    monkeypatch.setenv("GTC_TRIPLET_DEEP", deep)
    if layout == "split":
        monkeypatch.setenv("GTC_CSR_LAYOUT", "split")
    xyz = uniform(seed, 12_000)
    edges = linear_edges_sq(60_000, nb)
    c, _, st = hip_3pcf(xyz, edges)
    assert st["launch_mode"] == 3 | (4 if deep == "1" else 0)
    oc, _, _, _ = oracle.Graph(xyz, edges).count_3pcf()
    np.testing.assert_array_equal(c, oc)
    assert oc.sum() > 0


@pytest.mark.parametrize("hist", ["sorted", "unsorted"])
@pytest.mark.parametrize("weighted", [False, True])
def test_3pcf_frequent_histogram_exchanges(gpu_available, monkeypatch, hist, weighted):
    # waves exchange the LDS histogram every few hundred hits while the others keep adding to it:
    # every increment still reaches the global counts exactly once
    if hist == "unsorted" and weighted:
        pytest.skip("the unsorted histogram is unweighted only")
    say("3pcf exchanges", hist, weighted)
    monkeypatch.setenv("GTC_TRIPLET_HIST", hist)
    monkeypatch.setenv("GTC_TRIPLET_FLUSH_AT", "300")
    xyz = clustered(19, 20_000, 60, 2500)
    edges = linear_edges_sq(10_000, 12)
    w = 0.5 + rng_for(1019).random(20_000) if weighted else None
    c, ws, st = hip_3pcf(xyz, edges, w)
    assert bool(st["launch_mode"] & 2) == (hist == "unsorted")
    oc, ows, _, _ = oracle.Graph(xyz, edges).count_3pcf(w)
    assert oc.sum() > 100 * 300
    np.testing.assert_array_equal(c, oc)
    if weighted:
        np.testing.assert_array_equal(ws, ows)


@pytest.mark.parametrize("layout", ["packed", "split"])
@pytest.mark.parametrize("mode", ["flat", "banded"])
@pytest.mark.parametrize("kind,seed,n,r,nb,weighted", CASES_3[1:4])
def test_3pcf_walk_modes(gpu_available, monkeypatch, layout, mode, kind, seed, n, r, nb, weighted):
    # the two spoke walks (one map over the hub domain / one map per key run), on both CSR layouts
    # (label and bin in one word / a label array and a bin array), agree with the oracle
    say("3pcf mode", mode, layout, kind, seed, n, r, nb, weighted)
    monkeypatch.setenv("GTC_TRIPLET_MODE", mode)
    if layout == "split":
        monkeypatch.setenv("GTC_CSR_LAYOUT", "split")
    xyz = uniform(seed, n) if kind == "uniform" else clustered(seed, n, 60, 2500)
    edges = linear_edges_sq(r, nb)
    w = 0.5 + rng_for(seed + 1000).random(n) if weighted else None
    c, ws, st = hip_3pcf(xyz, edges, w)
    assert st["launch_mode"] & 1 == (1 if mode == "banded" else 0)
    oc, ows, s, _ = oracle.Graph(xyz, edges).count_3pcf(w)
    np.testing.assert_array_equal(c, oc)
    if weighted:
        np.testing.assert_array_equal(ws, ows)


@pytest.mark.parametrize("r,weighted", [(1_100_000, False), (1_100_000, True), (700_000, True),
                                        (350_000, False), (350_000, True)])
def test_3pcf_coarse_grids(gpu_available, monkeypatch, r, weighted):
    # grids of one, two and three cells per axis: with fewer than three the flat walk's domain is
    # one key run and the other four are empty (a zero entry each in the map); most pairs are
    # edges, so nearly every bin triple is hit
    say("3pcf coarse grid", r, weighted)
    monkeypatch.setenv("GTC_TRIPLET_MODE", "flat")
    n = 600
    xyz = uniform(23, n)
    edges = linear_edges_sq(r, 7)
    w = 0.5 + rng_for(1023).random(n) if weighted else None
    c, ws, st = hip_3pcf(xyz, edges, w)
    assert st["launch_mode"] & 1 == 0
    oc, ows, _, _ = oracle.Graph(xyz, edges).count_3pcf(w)
    assert oc.sum() > 100_000
    np.testing.assert_array_equal(c, oc)
    if weighted:
        np.testing.assert_array_equal(ws, ows)


def test_3pcf_hub_subsets(gpu_available):
    # counts of hub subsets add up to the full count, match the per-hub oracle in the graph's
    # internal order, and reject repeated or out-of-range labels
    import torch
    n = 20_000
    xyz = clustered(61, n, 60, 2500)
    edges = linear_edges_sq(12_000, 12)
    w = 0.5 + rng_for(62).random(n)
    g = gtc.Graph(to_gpu(xyz), edges)
    wt = torch.from_numpy(w).cuda()
    # hub labels are internal labels: the oracle takes the points in the order the cell list
    # defines, computed on the host, which the build must have produced
    perm = host_internal_order(xyz, edges)
    np.testing.assert_array_equal(g.perm(), perm)
    full, wfull, _ = g.count_3pcf(wt)
    full = full.cpu().numpy().view(np.uint64)
    parts = np.array_split(rng_for(63).permutation(n), 3)
    tot = np.zeros_like(full)
    for part in parts:
        c, _, st = g.count_3pcf_hubs(part, wt)
        tot += c.cpu().numpy().view(np.uint64)
    np.testing.assert_array_equal(tot, full)
    sample = parts[0][:300]
    c, ws, st = g.count_3pcf_hubs(sample, wt)
    oc, ows, _ = oracle.count_3pcf_hubs(xyz[perm], edges, sample, w[perm])
    np.testing.assert_array_equal(c.cpu().numpy().view(np.uint64), oc)
    np.testing.assert_array_equal(ws.cpu().numpy(), ows)
    assert st["triangles"] == int(oc.sum())
    for bad in ([1, 2, 2], [-1], [n]):
        with pytest.raises(gtc.GtcError) as ei:
            g.count_3pcf_hubs(bad)
        assert ei.value.status == gtc.GTC_E_INVALID
    c, _, _ = g.count_3pcf_hubs([])
    assert int(c.sum()) == 0
    g.close()
    gt = gtc.Graph(to_gpu(xyz), edges, tile_bytes=1 << 16)
    with pytest.raises(gtc.GtcError) as ei:
        gt.count_3pcf_hubs([0])
    assert ei.value.status == gtc.GTC_E_UNSUPPORTED
    gt.close()


@pytest.mark.parametrize("layout", ["packed", "split"])
@pytest.mark.parametrize("kind,seed,n,r,nb", [("clustered", 71, 30_000, 12_000, 12),
                                              ("uniform", 72, 20_000, 40_000, 30)])
def test_2pcf_matches_oracle(gpu_available, monkeypatch, layout, kind, seed, n, r, nb):
    import torch
    if layout == "split":
        monkeypatch.setenv("GTC_CSR_LAYOUT", "split")
    xyz = uniform(seed, n) if kind == "uniform" else clustered(seed, n, 60, 2500)
    edges = linear_edges_sq(r, nb)
    rng = rng_for(seed + 1)
    # signed weights of the data-minus-random estimator: data +1/N_D, randoms -1/N_R
    nd = n // 3
    w = np.where(np.arange(n) < nd, 1.0 / nd, -1.0 / (n - nd)) * (0.5 + rng.random(n))
    g = gtc.Graph(to_gpu(xyz), edges)
    c, ws, st = g.count_2pcf(torch.from_numpy(w).cuda())
    c0, _, _ = g.count_2pcf()
    g.close()
    og = oracle.Graph(xyz, edges)
    oc, ows, s = og.count_2pcf(w)
    np.testing.assert_array_equal(c.cpu().numpy().view(np.uint64), oc)
    np.testing.assert_array_equal(c0.cpu().numpy().view(np.uint64), oc)
    np.testing.assert_array_equal(ws.cpu().numpy(), ows)
    assert st["weight_scale"] == s and int(oc.sum()) == og.nnz // 2


@pytest.mark.parametrize("csr_mode", ["device", "host", "rebuild"])
def test_2pcf_on_tiled_graphs(gpu_available, csr_mode):
    import torch
    xyz = clustered(73, 25_000, 60, 2500)
    edges = linear_edges_sq(12_000, 10)
    w = 0.5 + rng_for(74).random(25_000)
    oc, ows, _ = oracle.Graph(xyz, edges).count_2pcf(w)
    g = gtc.Graph(to_gpu(xyz), edges, tile_bytes=4 * int(oc.sum()) // 5, csr_mode=csr_mode)
    assert g.stats()["windows"] > 1
    c, ws, _ = g.count_2pcf(torch.from_numpy(w).cuda())
    g.close()
    np.testing.assert_array_equal(c.cpu().numpy().view(np.uint64), oc)
    np.testing.assert_array_equal(ws.cpu().numpy(), ows)


def test_3pcf_c1_full(gpu_available):
    cfg = workloads.get("C1")
    xyz, w = cfg.generate()
    say("C1", xyz.shape)
    c, _, st = hip_3pcf(xyz, cfg.edges_sq())
    oc, _, _, _ = oracle.Graph(xyz, cfg.edges_sq()).count_3pcf()
    np.testing.assert_array_equal(c, oc)


def test_3pcf_c2_full_weighted(gpu_available):
    cfg = workloads.get("C2")
    xyz, w = cfg.generate()
    say("C2", xyz.shape)
    c, ws, st = hip_3pcf(xyz, cfg.edges_sq(), w)
    say("C2 gpu done", st["triangles"], st["kernel_ms"])
    oc, ows, s, _ = oracle.Graph(xyz, cfg.edges_sq()).count_3pcf(w)
    np.testing.assert_array_equal(c, oc)
    np.testing.assert_array_equal(ws, ows)
    rel = np.abs(ws - ows) / np.maximum(np.abs(ows), 1e-300)
    assert np.all(rel <= 1e-12)


def test_3pcf_signed_weights(gpu_available):
    xyz = clustered(21, 8000, 30, 3000)
    edges = linear_edges_sq(9000, 6)
    rng = rng_for(22)
    w = np.where(rng.random(8000) < 0.5, -1.0, 1.0) * (0.1 + rng.random(8000))
    c, ws, st = hip_3pcf(xyz, edges, w)
    oc, ows, s, _ = oracle.Graph(xyz, edges).count_3pcf(w)
    np.testing.assert_array_equal(c, oc)
    assert st["weight_scale"] == s
    np.testing.assert_array_equal(ws, ows)


def test_3pcf_edge_cases(gpu_available):
    edges = linear_edges_sq(5000, 4)
    for n in (0, 1, 2):
        say("tiny n", n)
        c, _, st = hip_3pcf(np.zeros((n, 3), np.int32), edges)
        assert c.sum() == 0 and st["edges"] == (n * (n - 1)) // 2
    # all points coincident: every pair in bin 0, C(n,3) triangles
    say("coincident")
    xyz = np.full((300, 3), 777, np.int32)
    c, _, st = hip_3pcf(xyz, edges)
    assert c[0] == 300 * 299 * 298 // 6 and c.sum() == c[0]
    # grid corners and the maximum coordinate
    say("corners")
    pts = np.array([[0, 0, 0], [GRID - 1] * 3, [GRID - 1, 0, 0], [0, GRID - 1, 0], [3, 4, 0],
                    [GRID - 2, GRID - 1, GRID - 3], [GRID - 1, GRID - 4, GRID - 1]], np.int32)
    c, _, _ = hip_3pcf(pts, linear_edges_sq(10, 3))
    oc, _, _, _ = oracle.Graph(pts, linear_edges_sq(10, 3)).count_3pcf()
    np.testing.assert_array_equal(c, oc)
    # no edges at all
    say("no edges")
    c, _, st = hip_3pcf(uniform(5, 1000), linear_edges_sq(2, 1))
    assert c.sum() == 0 and st["edges"] == 0
    # 255 bins
    say("255 bins")
    xyz = clustered(6, 3000, 10, 2000)
    e = linear_edges_sq(6000, 255)
    c, _, _ = hip_3pcf(xyz, e)
    oc, _, _, _ = oracle.Graph(xyz, e).count_3pcf()
    np.testing.assert_array_equal(c, oc)


def test_3pcf_bad_coordinates_rejected(gpu_available):
    xyz = uniform(7, 100)
    xyz[17, 1] = GRID
    with pytest.raises(gtc.GtcError) as ei:
        gtc.Graph(to_gpu(xyz), linear_edges_sq(1000, 2))
    assert ei.value.status == gtc.GTC_E_INVALID


def test_3pcf_repeatable_and_label_invariant(gpu_available):
    xyz = clustered(8, 20_000, 50, 2500)
    edges = linear_edges_sq(10_000, 12)
    w = 0.5 + rng_for(9).random(xyz.shape[0])
    a = hip_3pcf(xyz, edges, w)
    b = hip_3pcf(xyz, edges, w)
    perm = rng_for(10).permutation(xyz.shape[0])
    c = hip_3pcf(np.ascontiguousarray(xyz[perm]), edges, w[perm])
    for x in (b, c):
        np.testing.assert_array_equal(a[0], x[0])
        np.testing.assert_array_equal(a[1], x[1])


def test_internal_labels_are_deterministic(gpu_available):
    # internal labels: cell-sorted, ties in original order (§8 a2), the same on every build
    xyz = clustered(11, 30_000, 20, 1500)  # dense cells: many ties per cell
    edges = linear_edges_sq(8_000, 6)
    g1 = gtc.Graph(to_gpu(xyz), edges)
    g2 = gtc.Graph(to_gpu(xyz), edges)
    e1, e2 = g1.export(), g2.export()
    s1, s2 = g1.stats(), g2.stats()
    g1.close()
    g2.close()
    for a, b in zip(e1, e2):
        np.testing.assert_array_equal(a, b)
    for k in ("max_out_degree", "spoke_elements", "edges"):
        assert s1[k] == s2[k]
    perm = e1[3]
    # the build's cells (side ceil(r_max), at most ~2n cells and 512 per axis): internal order
    # sorts by cell key, ties by original index
    want, key = host_internal_order(xyz, edges, return_keys=True)
    np.testing.assert_array_equal(perm, want)
    assert np.unique(key).size < xyz.shape[0] // 2  # dense cells: many ties to break


def test_3pcf_nonfinite_weight_rejected(gpu_available):
    import torch
    xyz = uniform(11, 500)
    g = gtc.Graph(to_gpu(xyz), linear_edges_sq(100_000, 3))
    w = torch.ones(500, dtype=torch.float64, device="cuda")
    w[3] = float("nan")
    with pytest.raises(gtc.GtcError) as ei:
        g.count_3pcf(w)
    assert ei.value.status == gtc.GTC_E_INVALID
    g.close()


# ------------------------------------------------------------------ 4pCF

CASES_4 = [
    ("clustered", 31, 4000, 6000, 1),
    ("clustered", 32, 20_000, 8000, 4),
    ("uniform", 33, 8000, 70_000, 8),
    ("clustered", 34, 15_000, 3000, 16),
]


def points_4(kind, seed, n):
    return uniform(seed, n) if kind == "uniform" else clustered(seed, n, 50, 2000)


@functools.lru_cache(maxsize=None)
def oracle_4pcf(kind, seed, n, r, nb, s4=False):
    """The oracle's counts for one case, computed once per test session (both CSR layouts and
    the later tests of the same case compare against the same arrays)."""
    return oracle.Graph(points_4(kind, seed, n), linear_edges_sq(r, nb)).count_4pcf_parity(s4=s4)


@pytest.mark.parametrize("layout", ["packed", "split"])
@pytest.mark.parametrize("kind,seed,n,r,nb", CASES_4)
def test_4pcf_matches_oracle(gpu_available, monkeypatch, layout, kind, seed, n, r, nb):
    say("4pcf", layout, kind, seed, n, r, nb)
    if layout == "split":
        monkeypatch.setenv("GTC_CSR_LAYOUT", "split")
    xyz = points_4(kind, seed, n)
    edges = linear_edges_sq(r, nb)
    e, o, st = hip_4pcf(xyz, edges)
    oe, oo, ncl = oracle_4pcf(kind, seed, n, r, nb)
    np.testing.assert_array_equal(e, oe)
    np.testing.assert_array_equal(o, oo)
    assert st["cliques4"] == ncl and ncl > 0


@pytest.mark.parametrize("kind,seed,n,r,nb", CASES_4)
def test_4pcf_s4_matches_oracle(gpu_available, kind, seed, n, r, nb):
    # S4 configurations (six edge bins up to vertex relabelling), even and odd channels
    say("4pcf s4", kind, seed, n, r, nb)
    xyz = points_4(kind, seed, n)
    edges = linear_edges_sq(r, nb)
    g = gtc.Graph(to_gpu(xyz), edges)
    e, o, st = g.count_4pcf_parity(s4=True)
    es, os_, _ = g.count_4pcf_parity()
    g.close()
    e = e.cpu().numpy().view(np.uint64)
    o = o.cpu().numpy()
    oe, oo, ncl = oracle_4pcf(kind, seed, n, r, nb, s4=True)
    np.testing.assert_array_equal(e, oe)
    np.testing.assert_array_equal(o, oo)
    assert st["cliques4"] == ncl and ncl > 0
    # folding S4 configurations onto sorted 6-tuples gives the sorted-tuple counts
    cls = {t: r for r, t in enumerate(itertools.combinations_with_replacement(range(nb), 6))}
    fe = np.zeros(len(cls), np.uint64)
    for c, t in enumerate(gtc.config_bins_s4(nb)):
        fe[cls[tuple(sorted(int(x) for x in t))]] += e[c]
    np.testing.assert_array_equal(fe, es.cpu().numpy().view(np.uint64))


def test_4pcf_c4_full(gpu_available):
    # full C4 in both configuration schemes from one oracle pass: S4 counts compared directly,
    # sorted-tuple counts through the folding of S4 configurations onto sorted 6-tuples
    cfg = workloads.get("C4")
    xyz, _ = cfg.generate()
    nb = cfg.nbins
    say("C4", xyz.shape)
    g = gtc.Graph(to_gpu(xyz), cfg.edges_sq())
    es, os_, st = g.count_4pcf_parity()
    e4, o4, st4 = g.count_4pcf_parity(s4=True)
    g.close()
    say("C4 gpu done", st["cliques4"], st["kernel_ms"], "s4", st4["kernel_ms"])
    oe, oo, ncl = oracle.Graph(xyz, cfg.edges_sq()).count_4pcf_parity(s4=True)
    np.testing.assert_array_equal(e4.cpu().numpy().view(np.uint64), oe)
    np.testing.assert_array_equal(o4.cpu().numpy(), oo)
    cls = {t: r for r, t in enumerate(itertools.combinations_with_replacement(range(nb), 6))}
    fe = np.zeros(len(cls), np.uint64)
    fo = np.zeros(len(cls), np.int64)
    for c, t in enumerate(oracle.config_bins_s4(nb)):
        k = cls[tuple(sorted(int(x) for x in t))]
        fe[k] += oe[c]
        fo[k] += oo[c]
    np.testing.assert_array_equal(es.cpu().numpy().view(np.uint64), fe)
    np.testing.assert_array_equal(os_.cpu().numpy(), fo)
    assert st["cliques4"] == st4["cliques4"] == ncl
    assert np.abs(oo).sum() > 0


def test_4pcf_mirror_negates_odd(gpu_available):
    xyz = clustered(35, 10_000, 40, 2000)
    edges = linear_edges_sq(7000, 5)
    e, o, _ = hip_4pcf(xyz, edges)
    m = xyz.copy()
    m[:, 2] = GRID - 1 - m[:, 2]
    e2, o2, _ = hip_4pcf(m, edges)
    np.testing.assert_array_equal(e, e2)
    np.testing.assert_array_equal(o, -o2)
    assert np.abs(o).sum() > 0


def plane_points(seed: int, n: int, span: int, off_frac: float) -> np.ndarray:
    """Lattice points of the plane 7x + 8y + 9z = const (basis (8, -7, 0), (9, 0, -7)) around the
    grid centre; a fraction off_frac moved off it by +-(-1, 1, 0), one lattice step of that normal.
    Most quadruples are coplanar or nearly so, with hub-relative triple products whose fp64 terms
    exceed 2^53: plain fp64 rounding gets some of their signs wrong."""
    rng = rng_for(seed)
    s = rng.integers(-span, span + 1, size=n)
    t = rng.integers(-span, span + 1, size=n)
    p = np.stack([GRID // 2 + 8 * s + 9 * t, GRID // 2 - 7 * s, GRID // 2 - 7 * t], 1)
    k = rng.choice([-1, 0, 1], size=n, p=[off_frac / 2, 1 - off_frac, off_frac / 2])
    p = np.unique(p + k[:, None] * np.array([-1, 1, 0]), axis=0)
    assert p.min() >= 0 and p.max() < GRID
    return p.astype(np.int32)


def test_4pcf_handedness_of_nearly_flat_tetrahedra(gpu_available):
    # coplanar and nearly coplanar quadruples at large separations: the handedness must be the
    # exact sign (zero for coplanar ones), as in the oracle's integer arithmetic
    xyz = plane_points(37, 200, 30_000, 0.3)
    edges = linear_edges_sq(450_000, 4)
    say("4pcf flat", xyz.shape)
    e, o, st = hip_4pcf(xyz, edges)
    oe, oo, ncl = oracle.Graph(xyz, edges).count_4pcf_parity()
    np.testing.assert_array_equal(e, oe)
    np.testing.assert_array_equal(o, oo)
    assert st["cliques4"] == ncl and ncl > 100_000
    assert np.abs(oo).sum() > 0 and np.abs(oo).sum() < ncl  # both handed and flat ones


def test_4pcf_requires_coords(gpu_available):
    g = gtc.Graph(to_gpu(uniform(36, 200)), linear_edges_sq(200_000, 3), drop_coords=True)
    with pytest.raises(gtc.GtcError):
        g.count_4pcf_parity()
    g.close()


@pytest.mark.parametrize("order,tiny,huge", [(3, 2.0 ** -340, 1e150), (4, 2.0 ** -255, 1e100),
                                             (2, 2.0 ** -510, 1e200)])
def test_weights_beyond_the_exact_scale_are_refused(gpu_available, order, tiny, huge):
    # the exact sums scale every product by 2^s, s = 57 - e for max|w|^order = f 2^e: a max|w| so
    # small that 2^s passes the largest double, or so large that max|w|^order overflows, is
    # refused instead of summed into garbage
    import torch
    xyz = clustered(33, 4_000, 20, 3000)
    edges = linear_edges_sq(9_000, 4)
    g = gtc.Graph(to_gpu(xyz), edges)

    def run(a):
        w = torch.full((xyz.shape[0],), a, dtype=torch.float64, device="cuda")
        if order == 3:
            return g.count_3pcf(w)[1]
        if order == 4:
            return g.count_4pcf_weighted(w)[2]
        return g.count_2pcf(w)[1]

    for a in (tiny, -tiny, huge):
        with pytest.raises(gtc.GtcError) as ei:
            run(a)
        assert ei.value.status == gtc.GTC_E_UNSUPPORTED
    g.close()


def test_small_weights_within_the_exact_scale(gpu_available):
    # max|w| = 2^-300: the 3pCF scale is 2^956, still a double; the sums equal the oracle's
    xyz = clustered(34, 4_000, 20, 3000)
    edges = linear_edges_sq(9_000, 4)
    w = 2.0 ** -300 * (0.5 + rng_for(35).random(xyz.shape[0]))
    c, ws, st = hip_3pcf(xyz, edges, w)
    oc, ows, s, _ = oracle.Graph(xyz, edges).count_3pcf(w)
    assert st["weight_scale"] == s and 900 < s <= 1023
    np.testing.assert_array_equal(c, oc)
    np.testing.assert_array_equal(ws, ows)
    assert ws.max() > 0

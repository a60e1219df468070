"""GPU parity of the weighted 4pCF and of the data-minus-random estimators (compute_3pcf,
compute_4pcf) against the oracle on the same seeded inputs.

Every output is bit-exact: both sides sum the same fixed-point products exactly, round each sum
once, and divide the same doubles (the catalogue sums are correctly rounded on both sides).
Configurations without random cliques give NaN or infinity on both sides.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import graph_triangle_counting_amd as gtc
import oracle
from gpu_common import clustered, to_gpu, uniform
from oracle import estimator
from workloads import linear_edges_sq, rng_for

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def to_gpu_f64(w):
    import torch
    return None if w is None else torch.from_numpy(np.asarray(w, np.float64)).cuda()


# ------------------------------------------------------------------ weighted 4pCF

@pytest.mark.parametrize("s4", [False, True])
@pytest.mark.parametrize("kind,seed,n,r,nb,signed", [
    ("clustered", 41, 4000, 6000, 1, False),
    ("clustered", 42, 12_000, 8000, 4, True),
    ("uniform", 43, 8000, 70_000, 8, True),
    ("clustered", 44, 15_000, 3000, 16, True),
])
def test_4pcf_weighted_matches_oracle(gpu_available, s4, kind, seed, n, r, nb, signed):
    say("4pcf weighted", s4, kind, seed, n, r, nb, signed)
    xyz = uniform(seed, n) if kind == "uniform" else clustered(seed, n, 50, 2000)
    rng = rng_for(seed + 500)
    w = rng.uniform(0.25, 3.0, n) * (rng.choice([-1.0, 1.0], n) if signed else 1.0)
    edges = linear_edges_sq(r, nb)
    g = gtc.Graph(to_gpu(xyz), edges)
    e, o, ew, ow, st = g.count_4pcf_weighted(to_gpu_f64(w), s4=s4)
    e0, o0, _ = g.count_4pcf_parity(s4=s4)
    g.close()
    oe, oo, oew, oow, s = oracle.Graph(xyz, edges).count_4pcf_weighted(w, s4=s4)
    np.testing.assert_array_equal(e.cpu().numpy().view(np.uint64), oe)
    np.testing.assert_array_equal(o.cpu().numpy(), oo)
    np.testing.assert_array_equal(ew.cpu().numpy(), oew)
    np.testing.assert_array_equal(ow.cpu().numpy(), oow)
    assert st["weight_scale"] == s and st["cliques4"] == int(oe.sum()) > 0
    # the weighted kernel's counts are the unweighted kernel's
    np.testing.assert_array_equal(e.cpu().numpy(), e0.cpu().numpy())
    np.testing.assert_array_equal(o.cpu().numpy(), o0.cpu().numpy())


@pytest.mark.parametrize("kind,seed,n,r,nb", [("clustered", 46, 15_000, 6000, 8),
                                              ("uniform", 47, 8000, 70_000, 6)])
def test_4pcf_weighted_s4_cache_matches_global_sums(gpu_available, monkeypatch, kind, seed, n, r,
                                                    nb):
    # weighted S4 sums with the LDS cache of the sampled hot configurations equal those kept
    # wholly in global memory, bit for bit, counts included
    say("4pcf weighted s4 cache", kind, seed, n, r, nb)
    xyz = uniform(seed, n) if kind == "uniform" else clustered(seed, n, 50, 2000)
    w = rng_for(seed + 700).uniform(-2.0, 2.0, n)
    g = gtc.Graph(to_gpu(xyz), linear_edges_sq(r, nb))
    cached = [x.cpu().numpy() for x in g.count_4pcf_weighted(to_gpu_f64(w), s4=True)[:4]]
    monkeypatch.setenv("GTC_CONFIG_CACHE", "off")
    plain = [x.cpu().numpy() for x in g.count_4pcf_weighted(to_gpu_f64(w), s4=True)[:4]]
    g.close()
    for x, y in zip(cached, plain):
        np.testing.assert_array_equal(x, y)
    assert cached[0].view(np.uint64).sum() > 0 and np.abs(cached[3]).sum() > 0


@pytest.mark.parametrize("cache", ["on", "off"])
@pytest.mark.parametrize("s4", [False, True])
def test_4pcf_weighted_frequent_drains_match_oracle(gpu_available, monkeypatch, s4, cache):
    # the LDS count bins drained to global memory every few hundred tetrahedra of a wave give
    # the oracle's exact counts and sums (signed weights)
    say("4pcf weighted drains", s4, cache)
    monkeypatch.setenv("GTC_CLIQUE_FLUSH_AT", "300")
    monkeypatch.setenv("GTC_CONFIG_CACHE", cache)
    xyz = clustered(48, 8000, 50, 2000)
    w = rng_for(548).uniform(-2.0, 2.0, 8000)
    edges = linear_edges_sq(3000, 6)
    g = gtc.Graph(to_gpu(xyz), edges)
    e, o, ew, ow, _ = g.count_4pcf_weighted(to_gpu_f64(w), s4=s4)
    g.close()
    oe, oo, oew, oow, _ = oracle.Graph(xyz, edges).count_4pcf_weighted(w, s4=s4)
    np.testing.assert_array_equal(e.cpu().numpy().view(np.uint64), oe)
    np.testing.assert_array_equal(o.cpu().numpy(), oo)
    np.testing.assert_array_equal(ew.cpu().numpy(), oew)
    np.testing.assert_array_equal(ow.cpu().numpy(), oow)
    assert int(oe.sum()) > 300 * 64


def test_4pcf_weighted_rejects_non_finite_weights(gpu_available):
    xyz = clustered(45, 500, 10, 2000)
    w = np.ones(500)
    w[7] = np.inf
    g = gtc.Graph(to_gpu(xyz), linear_edges_sq(5000, 3))
    with pytest.raises(gtc.GtcError):
        g.count_4pcf_weighted(to_gpu_f64(w))
    g.close()


# ------------------------------------------------------------------ estimators

def catalogues(seed, nd, nr, lo=300_000, hi=420_000, unit=False):
    """Clustered data and uniform randoms over the same box, with weights in [0.5, 2)."""
    xd = clustered(seed, nd, max(nd // 100, 1), 1500, lo, hi)
    xr = uniform(seed + 1, nr, lo, hi)
    rng = rng_for(seed + 2)
    if unit:
        return xd, None, xr, None
    return xd, rng.uniform(0.5, 2.0, nd), xr, rng.uniform(0.5, 2.0, nr)


def hip_compute_3pcf(xd, wd, xr, wr, edges, **kw):
    return gtc.compute_3pcf(to_gpu(xd), to_gpu_f64(wd), to_gpu(xr), to_gpu_f64(wr),
                            edges_sq=edges, **kw)


def hip_compute_4pcf(xd, wd, xr, wr, edges, **kw):
    return gtc.compute_4pcf(to_gpu(xd), to_gpu_f64(wd), to_gpu(xr), to_gpu_f64(wr),
                            edges_sq=edges, **kw)


@pytest.mark.parametrize("seed,nd,nr,rmin,rmax,nb,unit", [
    (51, 3000, 6000, 400, 9000, 6, False),
    (52, 8000, 8000, 0, 6000, 12, True),
    (53, 500, 2500, 1000, 20_000, 3, False),
])
def test_compute_3pcf_matches_oracle(gpu_available, seed, nd, nr, rmin, rmax, nb, unit):
    say("compute_3pcf", seed, nd, nr, rmin, rmax, nb, unit)
    xd, wd, xr, wr = catalogues(seed, nd, nr, unit=unit)
    edges = estimator.linear_edges_sq(rmin, rmax, nb)
    r = hip_compute_3pcf(xd, wd, xr, wr, edges)
    z, nnn, rrr = estimator.compute_3pcf(xd, wd, xr, wr, edges)
    np.testing.assert_array_equal(r.NNN, nnn)
    np.testing.assert_array_equal(r.RRR, rrr)
    np.testing.assert_array_equal(r.zeta, z)
    assert np.isfinite(r.zeta).sum() > len(z) // 2
    np.testing.assert_array_equal(r.edges_sq, edges)
    np.testing.assert_array_equal(r.bins, gtc.config_bins(3, nb))
    c = 0.5 * (np.sqrt(edges[:-1].astype(float)) + np.sqrt(edges[1:].astype(float)))
    np.testing.assert_array_equal(r.r3, c[r.bins[:, 2]])
    # the equilateral 3pCF: the configurations (b, b, b)
    cfg = list(itertools.combinations_with_replacement(range(nb), 3))
    eq = r.equilateral()
    k = [cfg.index((b, b, b)) for b in range(nb)]
    np.testing.assert_array_equal(eq["zeta"], z[k])
    np.testing.assert_array_equal(eq["RRR"], rrr[k])
    np.testing.assert_array_equal(eq["r"], c)


@pytest.mark.parametrize("mode", ["host", "rebuild"])
def test_compute_3pcf_out_of_core_matches_resident(gpu_available, mode):
    say("compute_3pcf out of core", mode)
    xd, wd, xr, wr = catalogues(54, 6000, 9000)
    edges = estimator.linear_edges_sq(300, 7000, 5)
    a = hip_compute_3pcf(xd, wd, xr, wr, edges)
    b = hip_compute_3pcf(xd, wd, xr, wr, edges, tile_bytes=40_000, csr_mode=mode)
    assert b.stats["windows"] > 3
    np.testing.assert_array_equal(a.NNN, b.NNN)
    np.testing.assert_array_equal(a.RRR, b.RRR)
    np.testing.assert_array_equal(a.zeta, b.zeta)


@pytest.mark.parametrize("seed,nd,nr,rmin,rmax,nb,unit", [
    (61, 3000, 6000, 400, 7000, 4, False),
    (62, 5000, 5000, 0, 5000, 3, True),
    (63, 1500, 3000, 800, 9000, 2, False),
])
def test_compute_4pcf_matches_oracle(gpu_available, seed, nd, nr, rmin, rmax, nb, unit):
    say("compute_4pcf", seed, nd, nr, rmin, rmax, nb, unit)
    xd, wd, xr, wr = catalogues(seed, nd, nr, unit=unit)
    edges = estimator.linear_edges_sq(rmin, rmax, nb)
    r = hip_compute_4pcf(xd, wd, xr, wr, edges)
    ze, zo, zc, xi = estimator.compute_4pcf(xd, wd, xr, wr, edges)
    np.testing.assert_array_equal(r.xi, xi)
    np.testing.assert_array_equal(r.zeta_even, ze)
    np.testing.assert_array_equal(r.zeta_odd, zo)
    np.testing.assert_array_equal(r.zeta_conn, zc)
    assert np.isfinite(r.zeta_even).sum() > len(ze) // 3
    np.testing.assert_array_equal(r.bins, gtc.config_bins_s4(nb))
    np.testing.assert_array_equal(r.realizable, oracle.config_realizable_s4(nb, edges).astype(bool))


@pytest.mark.parametrize("mode", ["host", "rebuild"])
def test_compute_4pcf_out_of_core_matches_resident(gpu_available, mode):
    say("compute_4pcf out of core", mode)
    xd, wd, xr, wr = catalogues(67, 3000, 6000)
    edges = estimator.linear_edges_sq(400, 7000, 3)
    a = hip_compute_4pcf(xd, wd, xr, wr, edges)
    b = hip_compute_4pcf(xd, wd, xr, wr, edges, tile_bytes=30_000, csr_mode=mode)
    assert b.stats["windows"] > 3
    for x, y in ((a.zeta_even, b.zeta_even), (a.zeta_odd, b.zeta_odd), (a.zeta_conn, b.zeta_conn),
                 (a.xi, b.xi)):
        np.testing.assert_array_equal(x, y)


def test_estimators_vanish_when_data_are_the_randoms(gpu_available):
    # D = R with unit weights: every clique with a data vertex cancels against its random twin
    x = uniform(64, 3000, 300_000, 360_000)
    edges = estimator.linear_edges_sq(100, 8000, 3)
    r3 = hip_compute_3pcf(x, None, x, None, edges)
    assert r3.RRR.max() > 0
    np.testing.assert_array_equal(r3.NNN, 0.0)
    r4 = hip_compute_4pcf(x, None, x, None, edges)
    fin = np.isfinite(r4.zeta_even)
    assert fin.sum() > 5
    np.testing.assert_array_equal(r4.xi, 0.0)
    np.testing.assert_array_equal(r4.zeta_even[fin], 0.0)
    np.testing.assert_array_equal(r4.zeta_odd[fin], 0.0)


def test_estimators_without_data(gpu_available):
    # no data points, unit weights: NNN = -RRR (every triangle is all-random, sign (-1)^3; unit
    # weights keep the products' rounding independent of their order)
    _, _, xr, _ = catalogues(65, 10, 4000)
    xd = np.zeros((0, 3), np.int32)
    edges = estimator.linear_edges_sq(200, 9000, 4)
    r = hip_compute_3pcf(xd, None, xr, None, edges)
    fin = r.RRR > 0
    np.testing.assert_array_equal(r.NNN[fin], -r.RRR[fin])
    np.testing.assert_array_equal(r.zeta[fin], -1.0)
    z, _, _ = estimator.compute_3pcf(xd, None, xr, None, edges)
    np.testing.assert_array_equal(r.zeta, z)


def test_estimators_reject_bad_catalogues(gpu_available):
    xd, wd, xr, wr = catalogues(66, 200, 300)
    edges = estimator.linear_edges_sq(200, 9000, 4)
    bad = wd.copy()
    bad[3] = np.nan
    with pytest.raises(gtc.GtcError):
        hip_compute_3pcf(xd, bad, xr, wr, edges)
    zero = np.concatenate([np.ones(150), -np.ones(150)])
    with pytest.raises(gtc.GtcError):
        hip_compute_3pcf(xd, wd, xr, zero, edges)

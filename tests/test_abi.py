"""The C ABI on the CPU: the library loads, exports everything include/gtc.h declares, and rejects
bad arguments with GTC_E_INVALID before touching a GPU.  Configuration tables are checked against
itertools (nondecreasing tuples in lexicographic order)."""
import ctypes as C
import itertools
import subprocess
from math import comb

import numpy as np
import pytest

import graph_triangle_counting_amd as gtc


def test_library_exports_every_declared_function():
    declared = gtc.header_functions()
    assert len(declared) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", gtc.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    L = gtc.lib()
    for f in declared:
        assert hasattr(L, f)


def test_num_configs():
    for nb in (1, 2, 10, 30, 255):
        assert gtc.num_configs(3, nb) == comb(nb + 2, 3)
    for nb in (1, 4, 8, 16):
        assert gtc.num_configs(4, nb) == comb(nb + 5, 6)
    assert gtc.lib().gtc_num_configs(4, 17) == -1
    assert gtc.lib().gtc_num_configs(3, 0) == -1
    assert gtc.lib().gtc_num_configs(5, 3) == -1


@pytest.mark.parametrize("order,nb", [(3, 1), (3, 7), (3, 20), (4, 3), (4, 8)])
def test_config_bins_lexicographic(order, nb):
    k = 3 if order == 3 else 6
    want = np.array(list(itertools.combinations_with_replacement(range(nb), k)), np.int32)
    np.testing.assert_array_equal(gtc.config_bins(order, nb), want)


def _build(xyz_ptr, n, edges, nb, opt=None):
    L = gtc.lib()
    h = C.c_void_p()
    e = np.ascontiguousarray(edges, dtype=np.int64) if edges is not None else None
    rc = L.gtc_build_graph(xyz_ptr, n, e.ctypes.data_as(C.c_void_p) if e is not None else None,
                           nb, C.byref(opt) if opt else None, None, C.byref(h))
    return rc, h


def test_s4_configuration_tables_match_the_oracle():
    import oracle
    for nb in range(1, 17):
        assert gtc.num_configs_s4(nb) == (nb**6 + 9 * nb**4 + 14 * nb**2) // 24
    assert gtc.lib().gtc_num_configs_s4(17) == -1 and gtc.lib().gtc_num_configs_s4(0) == -1
    for nb in range(1, 7):
        np.testing.assert_array_equal(gtc.config_bins_s4(nb), oracle.config_bins_s4(nb))
    from workloads import linear_edges_sq
    cases = [(4, np.array([80, 125, 170, 215, 260], np.int64) ** 2),  # [G] §V.2: 178 of 276
             (4, linear_edges_sq(20_000, 4)), (5, linear_edges_sq(9_000, 5)),
             (8, linear_edges_sq(20_366, 8))]
    for nb, edges in cases:
        m = gtc.config_realizable_s4(nb, edges)
        np.testing.assert_array_equal(m, oracle.config_realizable_s4(nb, edges))
    assert int(gtc.config_realizable_s4(4, cases[0][1]).sum()) == 178


def _tetrahedron_by_construction(d):
    """Place a tetrahedron with edge lengths d[(u, v)] by trilateration: v0 at the origin, v1 on
    the x axis, v2 in the xy plane, v3 above it.  Returns z^2 of v3 (the squared height over the
    face v0 v1 v2, times nothing), or None when a face is no proper triangle."""
    for a, b, c in ((0, 1, 2), (0, 1, 3), (0, 2, 3), (1, 2, 3)):
        x, y, z = d[(a, b)], d[(a, c)], d[(b, c)]
        if not (x < y + z and y < x + z and z < x + y):
            return None
    p1 = d[(0, 1)]
    x2 = (d[(0, 2)] ** 2 - d[(1, 2)] ** 2 + p1 ** 2) / (2 * p1)
    y2 = np.sqrt(d[(0, 2)] ** 2 - x2 ** 2)
    x3 = (d[(0, 3)] ** 2 - d[(1, 3)] ** 2 + p1 ** 2) / (2 * p1)
    y3 = (d[(0, 3)] ** 2 - d[(2, 3)] ** 2 + x2 ** 2 + y2 ** 2 - 2 * x2 * x3) / (2 * y2)
    return d[(0, 3)] ** 2 - x3 ** 2 - y3 ** 2


@pytest.mark.parametrize("nb,rmax", [(2, 12_000), (3, 20_000), (3, 700)])
def test_realizable_mask_by_construction(nb, rmax):
    # an independent check of the library's realizability mask at 2 and 3 bins: the bin-centre
    # edge lengths of each configuration (midpoint in r of each bin) are realised by placing the
    # four vertices one by one; a configuration is realizable when every face is a proper
    # triangle and the last vertex lies off the plane of the first three
    from workloads import linear_edges_sq
    edges = linear_edges_sq(rmax, nb)
    r = np.sqrt(edges.astype(np.float64))
    centre = (r[:-1] + r[1:]) / 2
    bins = gtc.config_bins_s4(nb)
    mask = gtc.config_realizable_s4(nb, edges)
    order = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]
    n_real = 0
    for t, m in zip(bins, mask):
        d = {e: centre[b] for e, b in zip(order, t)}
        z2 = _tetrahedron_by_construction(d)
        want = z2 is not None and z2 > 0
        if z2 is not None:
            assert abs(z2) > 1e-9 * centre.max() ** 2, "near-degenerate case: pick other edges"
        assert bool(m) == want, (t, z2)
        n_real += want
    assert 0 < n_real < len(bins)


def test_disconnected_and_connected_4pcf_match_the_oracle():
    import oracle
    rng = np.random.default_rng(7)
    for nb in (1, 4, 8):
        xi = rng.normal(size=nb)
        d = gtc.disconnected_4pcf_s4(nb, xi)
        np.testing.assert_array_equal(d, oracle.disconnected_4pcf_s4(nb, xi))
        zeta = rng.normal(size=d.size)
        np.testing.assert_array_equal(gtc.connected_4pcf_s4(nb, zeta, xi), zeta - d)
    assert gtc.lib().gtc_disconnected_4pcf_s4(17, None, None) == gtc.GTC_E_INVALID


def test_build_rejects_bad_arguments_without_gpu():
    fake = C.c_void_p(0x1000)  # never dereferenced: every case fails before any device work
    cases = [
        (None, 10, [0, 5, 10], 2),            # null coordinates with n > 0
        (fake, -1, [0, 5, 10], 2),            # negative n
        (fake, 1 << 31, [0, 5, 10], 2),       # n too large
        (fake, 10, None, 2),                  # null edges
        (fake, 10, [0, 5, 10], 0),            # nbins 0
        (fake, 10, [0] + list(range(1, 257)), 256),  # nbins > 255
        (fake, 10, [-1, 5, 10], 2),           # negative first edge
        (fake, 10, [0, 5, 5], 2),             # not strictly increasing
        (fake, 10, [0, 10, 5], 2),
        (fake, 10, [0, 5, 3 * (1 << 40) + 2], 2),  # beyond the largest squared distance
    ]
    for ptr, n, edges, nb in cases:
        rc, h = _build(ptr, n, edges, nb)
        assert rc == gtc.GTC_E_INVALID, (n, edges, nb)
        assert not h.value
        assert gtc.lib().gtc_last_error()
    rc, _ = _build(fake, 10, [0, 5, 10], 2, gtc.Options(-5, 0, 0))
    assert rc == gtc.GTC_E_INVALID
    for mode in (1, 2):  # out-of-core modes need a window budget
        rc, _ = _build(fake, 10, [0, 5, 10], 2, gtc.Options(0, mode, 0))
        assert rc == gtc.GTC_E_INVALID
    for mode in (-1, 3):
        rc, _ = _build(fake, 10, [0, 5, 10], 2, gtc.Options(100, mode, 0))
        assert rc == gtc.GTC_E_INVALID
    rc, _ = _build(fake, 10, [0, 5, 10], 2, gtc.Options(100, 2, 1))  # rebuild needs coordinates
    assert rc == gtc.GTC_E_INVALID
    L = gtc.lib()
    assert L.gtc_build_graph(fake, 10, None, 2, None, None, None) == gtc.GTC_E_INVALID


def test_count_rejects_bad_arguments_without_gpu():
    L = gtc.lib()
    st = gtc.Stats()
    fake = C.c_void_p(0x1000)
    assert L.gtc_count_3pcf(None, None, fake, None, C.byref(st), None) == gtc.GTC_E_INVALID
    assert L.gtc_count_4pcf_parity(None, fake, fake, C.byref(st), None) == gtc.GTC_E_INVALID
    assert L.gtc_graph_export(None, None, None, None, None) == gtc.GTC_E_INVALID
    assert L.gtc_graph_stats(None, C.byref(st)) == gtc.GTC_E_INVALID
    L.gtc_graph_free(None)  # no-op
    assert L.gtc_config_bins(3, 5, None) == gtc.GTC_E_INVALID
    for code in (0, -1, -2, -3, -4, -5):
        assert L.gtc_status_string(code)


def test_python_binding_requires_gpu_tensors():
    import torch
    with pytest.raises(TypeError):
        gtc.Graph(torch.zeros((4, 3), dtype=torch.int32), [0, 10])


def _plan(row_ptr, tile_bytes, entry_bytes=5):
    L = gtc.lib()
    rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
    n = rp.size - 1
    out = np.zeros(n + 2, np.int64)
    W = L.gtc_plan_windows(rp.ctypes.data_as(C.c_void_p), n, tile_bytes, entry_bytes,
                           out.ctypes.data_as(C.c_void_p))
    return W, out[:W + 1]


def test_plan_windows_partitions_rows_greedily():
    L = gtc.lib()
    rng = np.random.default_rng(5)
    for trial in range(40):
        n = int(rng.integers(1, 400))
        deg = rng.integers(0, 60, n)
        deg[rng.integers(0, n, 3)] = 500  # a few rows longer than small budgets
        rp = np.concatenate([[0], np.cumsum(deg)])
        budget = int(rng.integers(1, 5 * 800))
        eb = 4 if trial % 2 else 5  # packed entries, or label + bin arrays
        W, b = _plan(rp, budget, eb)
        assert W >= 1 and b[0] == 0 and b[-1] == n and np.all(np.diff(b) > 0)
        for k in range(W):
            rows = b[k + 1] - b[k]
            size = eb * (rp[b[k + 1]] - rp[b[k]])
            assert size <= budget or rows == 1, (trial, k)
            if b[k + 1] < n:  # greedy: one more row would not fit
                assert eb * (rp[b[k + 1] + 1] - rp[b[k]]) > budget
    W, b = _plan(np.zeros(1, np.int64), 100)
    assert W == 1 and list(b) == [0, 0]
    assert L.gtc_plan_windows(None, 3, 10, 5, None) == gtc.GTC_E_INVALID
    bad = np.array([0, 5, 3], np.int64)
    out = np.zeros(4, np.int64)
    assert L.gtc_plan_windows(bad.ctypes.data_as(C.c_void_p), 2, 10, 5,
                              out.ctypes.data_as(C.c_void_p)) == gtc.GTC_E_INVALID
    good = np.array([0, 5, 7], np.int64)
    assert L.gtc_plan_windows(good.ctypes.data_as(C.c_void_p), 2, 10, 0,
                              out.ctypes.data_as(C.c_void_p)) == gtc.GTC_E_INVALID


def test_graph_windows_rejects_a_null_graph():
    L = gtc.lib()
    out = np.zeros(4, np.int64)
    assert L.gtc_graph_windows(None, None, None, 0) == gtc.GTC_E_INVALID
    assert L.gtc_graph_windows(None, out.ctypes.data_as(C.c_void_p), None, 4) == gtc.GTC_E_INVALID


@pytest.mark.parametrize("rmin,rmax,nb", [(0, 1000, 3), (7, 31, 4), (1, 100, 16), (3, 4, 1),
                                          (50_000, 1 << 21, 255), (0, 1 << 21, 7)])
def test_linear_edges_sq_matches_the_oracle(rmin, rmax, nb):
    from oracle import estimator
    np.testing.assert_array_equal(gtc.linear_edges_sq(rmin, rmax, nb),
                                  estimator.linear_edges_sq(rmin, rmax, nb))


def test_linear_edges_sq_rejects_bad_ranges():
    for args in ((-1, 10, 2), (10, 10, 2), (0, (1 << 21) + 1, 2), (0, 10, 0), (0, 10, 256),
                 (0, 3, 8)):  # the last: 8 bins on [0, 3) repeat an integer edge
        with pytest.raises(gtc.GtcError):
            gtc.linear_edges_sq(*args)


def test_estimators_reject_bad_arguments_without_gpu():
    L = gtc.lib()
    fake = C.c_void_p(0x1000)  # never dereferenced: every case fails before any device work
    e = np.array([0, 5, 10], np.int64).ctypes.data_as(C.c_void_p)
    out = np.zeros(64)
    o = out.ctypes.data_as(C.c_void_p)
    st = gtc.Stats()
    c3 = lambda xd, nd, xr, nr, nb, z: L.gtc_compute_3pcf(xd, nd, None, xr, nr, None, e, nb, None,
                                                          z, None, None, C.byref(st), None)
    assert c3(fake, 4, fake, 0, 2, o) == gtc.GTC_E_INVALID   # no randoms
    assert c3(None, 4, fake, 4, 2, o) == gtc.GTC_E_INVALID   # data coordinates missing
    assert c3(fake, -1, fake, 4, 2, o) == gtc.GTC_E_INVALID  # negative n_data
    assert c3(fake, 4, fake, 4, 2, None) == gtc.GTC_E_INVALID  # no output
    assert c3(fake, 4, fake, 4, 0, o) == gtc.GTC_E_INVALID   # nbins 0
    assert c3(fake, 1 << 30, fake, 1 << 30, 2, o) == gtc.GTC_E_INVALID  # n >= 2^31
    c4 = lambda nb, opt, z: L.gtc_compute_4pcf(fake, 4, None, fake, 4, None, e, nb, opt, z, z,
                                               None, None, C.byref(st), None)
    assert c4(17, None, o) == gtc.GTC_E_INVALID  # beyond the 4pCF's 16 bins
    assert c4(2, None, None) == gtc.GTC_E_INVALID
    assert c4(2, C.byref(gtc.Options(0, 0, 1)), o) == gtc.GTC_E_INVALID  # coordinates dropped


@pytest.mark.parametrize("order,s4,nb", [(3, False, 1), (3, False, 7), (3, False, 255), (4, False, 1),
                                         (4, False, 8), (4, False, 16), (4, True, 1), (4, True, 5),
                                         (4, True, 8)])
def test_equilateral_configs_point_at_all_equal_tuples(order, s4, nb):
    ranks = gtc.equilateral_configs(order, nb, s4)
    k = 3 if order == 3 else 6
    if nb <= 16 and not s4:  # against itertools' lexicographic nondecreasing tuples
        tuples = list(itertools.combinations_with_replacement(range(nb), k))
        assert [tuples[r] for r in ranks] == [(b,) * k for b in range(nb)]
    bins = gtc.config_bins_s4(nb) if s4 else gtc.config_bins(order, nb)
    np.testing.assert_array_equal(bins[ranks], np.repeat(np.arange(nb), k).reshape(nb, k))
    assert np.all(np.diff(ranks) > 0)


def test_equilateral_configs_reject_bad_arguments():
    L = gtc.lib()
    out = np.zeros(300, np.int64).ctypes.data_as(C.c_void_p)
    for order, s4, nb in ((2, 0, 4), (3, 1, 4), (3, 0, 0), (3, 0, 256), (4, 0, 17), (4, 1, 0)):
        assert L.gtc_equilateral_configs(order, s4, nb, out) == gtc.GTC_E_INVALID
    assert L.gtc_equilateral_configs(3, 0, 4, None) == gtc.GTC_E_INVALID


def test_hbm_read_rate_rejects_bad_arguments_without_gpu():
    L = gtc.lib()
    g = C.c_double(0)
    fake = C.c_void_p(0x1000)
    assert L.gtc_hbm_read_rate(None, 1024, 1, C.byref(g), None) == gtc.GTC_E_INVALID
    assert L.gtc_hbm_read_rate(C.c_void_p(0x1004), 1024, 1, C.byref(g), None) == gtc.GTC_E_INVALID
    assert L.gtc_hbm_read_rate(fake, 8, 1, C.byref(g), None) == gtc.GTC_E_INVALID
    assert L.gtc_hbm_read_rate(fake, 1024, 0, C.byref(g), None) == gtc.GTC_E_INVALID
    assert L.gtc_hbm_read_rate(fake, 1024, 1, None, None) == gtc.GTC_E_INVALID


def test_tiles_cover_every_walk_and_tetrahedron_once():
    # Windows from the library's planner over a real forward CSR (the oracle's graph, labels
    # ascending), tiles enumerated as the count loops do: 3pCF (h, s), h <= s <= smax(h); 4pCF
    # (h, c1, c2), h <= c1 <= c2 <= smax(h), smax(h) the window of the largest spoke label of
    # window h.  Every walk (i, j) and every tetrahedron i < a < b < c must fall in exactly one
    # enumerated tile: (win i, win j), and (win i, win a, win b).
    import itertools
    import oracle
    from workloads import linear_edges_sq, rng_for
    rng = rng_for(93)
    xyz = (rng.integers(0, 40_000, (700, 3))).astype(np.int32)
    og = oracle.Graph(xyz, linear_edges_sq(9_000, 3))
    rp_full, col_full, _ = og.export()
    n = og.n
    fwd = [[int(k) for k in col_full[rp_full[i]:rp_full[i + 1]] if k > i] for i in range(n)]
    rp = np.concatenate([[0], np.cumsum([len(r) for r in fwd])]).astype(np.int64)
    for budget in (4 * 40, 4 * 200, 4 * int(rp[-1]) // 7):
        W, b = _plan(rp, budget, 4)
        win = np.searchsorted(b, np.arange(n), side="right") - 1
        smax = [max([win[r[-1]] for r in fwd[b[h]:b[h + 1]] if r] + [h]) for h in range(W)]
        tiles3 = {(h, s) for h in range(W) for s in range(h, smax[h] + 1)}
        tiles4 = {(h, c1, c2) for h in range(W) for c1 in range(h, smax[h] + 1)
                  for c2 in range(c1, smax[h] + 1)}
        nwalk = ncl = 0
        for i in range(n):
            for j in fwd[i]:
                assert (win[i], win[j]) in tiles3
                nwalk += 1
            adj = set(fwd[i])
            for a, bb in itertools.combinations(fwd[i], 2):
                if bb not in fwd[a]:
                    continue
                for c in fwd[bb]:
                    if c in adj and c in fwd[a]:
                        assert (win[i], win[a], win[bb]) in tiles4
                        ncl += 1
        assert W > 2 and nwalk == rp[-1] and ncl > 0

"""The command line (python -m graph_triangle_counting_amd): the grid mapping on the CPU, and one
run per statistic on the GPU against the library called directly on the same grid points."""
from __future__ import annotations

import numpy as np
import pytest

from graph_triangle_counting_amd import __main__ as cli
from workloads import rng_for


def test_grid_map_covers_the_grid_with_one_scale():
    rng = rng_for(91)
    d = rng.uniform(-50, 250, (400, 3))
    r = rng.uniform(-60, 240, (900, 3))
    lo, scale = cli.grid_map(d, r)
    gd, gr = cli.to_grid(d, lo, scale), cli.to_grid(r, lo, scale)
    allg = np.concatenate([gd, gr])
    assert allg.min() == 0 and allg.max() == (1 << 20) - 1
    # distances scale by one factor (to the grid's rounding)
    i, j = 3, 700
    a, b = np.concatenate([d, r])[i], np.concatenate([d, r])[j]
    ga, gb = allg[i].astype(float), allg[j].astype(float)
    assert abs(np.linalg.norm(ga - gb) / scale - np.linalg.norm(a - b)) <= 2.0 / scale
    with pytest.raises(ValueError):
        cli.grid_map(np.full((2, 3), np.nan), r)


def test_edges_are_equal_bins_in_r():
    scale = 1000.0
    e = cli.edges_sq(2.0, 30.0, 7, scale)
    rb = (2.0 + np.arange(8) * 4.0) * scale
    np.testing.assert_array_equal(e, np.ceil(rb * rb).astype(np.int64))
    for b in range(8):  # an integer squared distance is in bin b iff its root reaches r_b
        for d2 in (int(e[b]) - 1, int(e[b])):
            assert (d2 >= e[b]) == (np.sqrt(d2) >= rb[b] - 1e-9)
    for bad in ((5.0, 5.0, 3), (-1.0, 5.0, 3), (0.0, 5.0, 0)):
        with pytest.raises(ValueError):
            cli.edges_sq(*bad, scale)
    with pytest.raises(ValueError):  # bins finer than the grid
        cli.edges_sq(0.0, 1e-6, 50, 1.0)


@pytest.mark.gpu
@pytest.mark.parametrize("stat", ["3pcf", "4pcf"])
def test_cli_matches_the_library(gpu_available, tmp_path, stat):
    import torch

    import graph_triangle_counting_amd as gtc
    rng = rng_for(92)
    centres = rng.uniform(0, 100, (30, 3))
    d = centres[rng.integers(0, 30, 3000)] + rng.normal(0, 1.0, (3000, 3))
    r = rng.uniform(0, 100, (6000, 3))
    wd = rng.uniform(0.5, 2.0, 3000)
    for name, a in (("d", d), ("r", r), ("wd", wd)):
        np.save(tmp_path / f"{name}.npy", a)
    out = tmp_path / "out.npz"
    rmin, rmax, nb = (0.5, 6.0, 5) if stat == "3pcf" else (0.5, 4.0, 3)
    assert cli.main([stat, "--data", str(tmp_path / "d.npy"), "--randoms", str(tmp_path / "r.npy"),
                     "--data-weights", str(tmp_path / "wd.npy"), "--rmin", str(rmin), "--rmax",
                     str(rmax), "--nbins", str(nb), "--out", str(out)]) == 0
    res = np.load(out)
    lo, scale = cli.grid_map(d, r)
    e = cli.edges_sq(rmin, rmax, nb, scale)
    np.testing.assert_array_equal(res["edges_sq"], e)
    xd = torch.from_numpy(cli.to_grid(d, lo, scale)).cuda()
    xr = torch.from_numpy(cli.to_grid(r, lo, scale)).cuda()
    wt = torch.from_numpy(wd).cuda()
    if stat == "3pcf":
        ref = gtc.compute_3pcf(xd, wt, xr, None, edges_sq=e)
        np.testing.assert_array_equal(res["zeta"], ref.zeta)
        np.testing.assert_array_equal(res["RRR"], ref.RRR)
        np.testing.assert_allclose(res["r3"], ref.r3 / scale)
        assert np.isfinite(res["zeta"]).sum() > 5
    else:
        ref = gtc.compute_4pcf(xd, wt, xr, None, edges_sq=e)
        np.testing.assert_array_equal(res["zeta_even"], ref.zeta_even)
        np.testing.assert_array_equal(res["zeta_conn"], ref.zeta_conn)
        np.testing.assert_array_equal(res["xi"], ref.xi)
        assert res["realizable"].dtype == bool and np.isfinite(res["zeta_even"]).sum() > 5

"""GPU: the hub-window tile loop gives exactly the resident counts and the oracle's counts, with
the CSR in device memory, in pinned host memory (windows uploaded per tile), or nowhere (windows
emitted again per tile)."""
from __future__ import annotations

import numpy as np
import pytest

import graph_triangle_counting_amd as gtc
import oracle
import workloads
from gpu_common import clustered, edge_set_from_gpu, hip_3pcf, hip_4pcf, to_gpu, uniform
from workloads import linear_edges_sq, rng_for

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


CASES = [
    ("clustered", 41, 30_000, 12_000, 12, True),
    ("uniform", 42, 20_000, 45_000, 8, False),
]


@pytest.mark.parametrize("layout", ["packed", "split"])
@pytest.mark.parametrize("csr_mode", ["device", "host", "rebuild"])
@pytest.mark.parametrize("kind,seed,n,r,nb,weighted", CASES)
def test_tiled_equals_resident_and_oracle(gpu_available, monkeypatch, kind, seed, n, r, nb,
                                          weighted, csr_mode, layout):
    if layout == "split":
        monkeypatch.setenv("GTC_CSR_LAYOUT", "split")
    xyz = uniform(seed, n) if kind == "uniform" else clustered(seed, n, 60, 2500)
    edges = linear_edges_sq(r, nb)
    w = 0.5 + rng_for(seed + 7).random(n) if weighted else None
    c0, w0, st0 = hip_3pcf(xyz, edges, w)
    oc, ow, _, _ = oracle.Graph(xyz, edges).count_3pcf(w)
    np.testing.assert_array_equal(c0, oc)
    csr_bytes = 5 * st0["edges"]
    for frac in (1 / 2, 1 / 7, 1 / 40):
        tb = max(1, int(csr_bytes * frac))
        say("tiles", kind, seed, "csr_mode", csr_mode, layout, "tile_bytes", tb)
        c, ws, st = hip_3pcf(xyz, edges, w, tile_bytes=tb, csr_mode=csr_mode)
        assert st["windows"] > 1 and st["tiles"] >= st["windows"]
        np.testing.assert_array_equal(c, c0)
        if weighted:
            np.testing.assert_array_equal(ws, w0)
            np.testing.assert_array_equal(ws, ow)
        if csr_mode != "device":
            assert st["h2d_ms"] > 0


def test_tiled_graph_exports_the_same_edges(gpu_available):
    xyz = clustered(43, 8000, 30, 3000)
    edges = linear_edges_sq(9000, 5)
    g0 = gtc.Graph(to_gpu(xyz), edges)
    want = edge_set_from_gpu(g0)
    tb = 5 * g0.stats()["edges"] // 9
    g0.close()
    for mode in ("device", "host", "rebuild"):
        g = gtc.Graph(to_gpu(xyz), edges, tile_bytes=tb, csr_mode=mode)
        assert g.stats()["windows"] > 1
        np.testing.assert_array_equal(edge_set_from_gpu(g), want)
        g.close()


def test_tiled_c2_full_out_of_core(gpu_available):
    cfg = workloads.get("C2")
    xyz, w = cfg.generate()
    c0, w0, st0 = hip_3pcf(xyz, cfg.edges_sq(), w)
    say("C2 resident", st0["kernel_ms"])
    for mode in ("host", "rebuild"):
        c, ws, st = hip_3pcf(xyz, cfg.edges_sq(), w, tile_bytes=4 * st0["edges"] // 6,
                             csr_mode=mode)
        say("C2 out-of-core", mode, st["windows"], st["tiles"], st["kernel_ms"], st["h2d_ms"])
        assert st["windows"] > 1
        np.testing.assert_array_equal(c, c0)
        np.testing.assert_array_equal(ws, w0)


def test_4pcf_on_tiled_graphs(gpu_available):
    xyz = clustered(44, 15_000, 50, 2000)
    edges = linear_edges_sq(6000, 4)
    e0, o0, st0 = hip_4pcf(xyz, edges)
    e, o, _ = hip_4pcf(xyz, edges, tile_bytes=5 * max(st0["edges"], 1) // 5)
    np.testing.assert_array_equal(e, e0)
    np.testing.assert_array_equal(o, o0)
    for mode in ("host", "rebuild"):
        g = gtc.Graph(to_gpu(xyz), edges, tile_bytes=1 << 16, csr_mode=mode)
        with pytest.raises(gtc.GtcError) as ei:
            g.count_4pcf_parity()
        assert ei.value.status == gtc.GTC_E_UNSUPPORTED
        g.close()

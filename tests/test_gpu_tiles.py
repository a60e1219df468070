"""GPU: the hub-window tile loop gives exactly the resident counts and the oracle's counts, with
the CSR in device memory, in pinned host memory (windows uploaded per tile), or nowhere (windows
emitted again per tile)."""
from __future__ import annotations

import functools

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
        # one launch per hub window with hubs, over all its search windows (resident CSR) or
        # over at most two at a time (out of core)
        assert st["windows"] > 1 and 1 <= st["tiles"]
        if csr_mode == "device":
            assert st["tiles"] <= st["windows"]
        elif frac == 1 / 40:  # hub windows whose spokes reach past the next window: extra launches
            assert st["tiles"] > st["windows"]
        np.testing.assert_array_equal(c, c0)
        if weighted:
            np.testing.assert_array_equal(ws, w0)
            np.testing.assert_array_equal(ws, ow)
        if csr_mode != "device" and st["windows"] > 3:  # (the build leaves three on the device)
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


@functools.lru_cache(maxsize=None)
def oracle_4pcf_tiles_case():
    """The oracle's even counts of the tiled 4pCF case, once per test session."""
    return oracle.Graph(clustered(44, 15_000, 50, 2000), linear_edges_sq(6000, 4)).count_4pcf_parity()[0]


@pytest.mark.parametrize("layout", ["packed", "split"])
@pytest.mark.parametrize("csr_mode", ["device", "host", "rebuild"])
def test_4pcf_on_tiled_graphs(gpu_available, monkeypatch, csr_mode, layout):
    # out of core, the 4-clique count runs over tiles (hub window, search windows c1 <= c2) and
    # gives the resident counts (sorted tuples, S4 configurations, weighted sums) and the oracle's
    if layout == "split":
        monkeypatch.setenv("GTC_CSR_LAYOUT", "split")
    xyz = clustered(44, 15_000, 50, 2000)
    edges = linear_edges_sq(6000, 4)
    w = rng_for(48).uniform(-2.0, 2.0, 15_000)
    wt = torch_f64(w)
    g0 = gtc.Graph(to_gpu(xyz), edges)
    e0, o0, st0 = g0.count_4pcf_parity()
    r0 = g0.count_4pcf_weighted(wt, s4=True)
    csr = 4 * max(g0.stats()["edges"], 1)
    g0.close()
    np.testing.assert_array_equal(e0.cpu().numpy().view(np.uint64), oracle_4pcf_tiles_case())
    # 1/3 and 1/11: every hub window's spokes end in the next window, one launch per hub window
    # on two streams in turn; 1/30: some reach further, a launch per tile (h, c1, c2)
    for frac in (1 / 3, 1 / 11, 1 / 30):
        say("4pcf tiles", csr_mode, layout, frac)
        g = gtc.Graph(to_gpu(xyz), edges, tile_bytes=int(csr * frac), csr_mode=csr_mode)
        e, o, st = g.count_4pcf_parity()
        nw = g.stats()["windows"]
        assert nw > 2
        if csr_mode != "device":
            assert st["tiles"] == nw if frac > 1 / 30 else st["tiles"] > nw
        np.testing.assert_array_equal(e.cpu().numpy(), e0.cpu().numpy())
        np.testing.assert_array_equal(o.cpu().numpy(), o0.cpu().numpy())
        r = g.count_4pcf_weighted(wt, s4=True)
        for x, y in zip(r[:4], r0[:4]):
            np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy())
        g.close()


def torch_f64(w):
    import torch
    return torch.from_numpy(np.asarray(w, np.float64)).cuda()


@pytest.mark.parametrize("drop_coords", [False, True])
def test_build_goes_out_of_core_by_itself(gpu_available, monkeypatch, drop_coords):
    # with no window budget, a CSR beyond 3/4 of the free device memory is kept out of core:
    # re-emitted windows when the coordinates are kept, pinned host memory when they are dropped
    xyz = clustered(45, 30_000, 60, 2500)
    edges = linear_edges_sq(12_000, 9)
    w = 0.5 + rng_for(46).random(30_000)
    c0, w0, st0 = hip_3pcf(xyz, edges, w)
    assert st0["windows"] == 1 and st0["csr_mode"] == gtc.CSR_MODES["device"]
    csr_bytes = 4 * st0["edges"]
    monkeypatch.setenv("GTC_DEVICE_FREE_BYTES", str(csr_bytes))  # 3/4 of it is too little
    say("auto out of core, drop_coords", drop_coords, "csr bytes", csr_bytes)
    c, ws, st = hip_3pcf(xyz, edges, w, drop_coords=drop_coords)
    assert st["windows"] > 2
    assert st["csr_mode"] == gtc.CSR_MODES["host" if drop_coords else "rebuild"]
    np.testing.assert_array_equal(c, c0)
    np.testing.assert_array_equal(ws, w0)
    monkeypatch.setenv("GTC_DEVICE_FREE_BYTES", str(2 * csr_bytes))  # enough: stays resident
    c, _, st = hip_3pcf(xyz, edges)
    assert st["windows"] == 1 and st["csr_mode"] == gtc.CSR_MODES["device"]
    np.testing.assert_array_equal(c, c0)


def test_window_budget_from_the_environment(gpu_available, monkeypatch):
    xyz = uniform(47, 20_000)
    edges = linear_edges_sq(45_000, 6)
    c0, _, st0 = hip_3pcf(xyz, edges)
    monkeypatch.setenv("GTC_TILE_BYTES", str(4 * st0["edges"] // 5))
    c, _, st = hip_3pcf(xyz, edges)
    assert st["windows"] > 1 and st["csr_mode"] == gtc.CSR_MODES["device"]
    np.testing.assert_array_equal(c, c0)
    # an explicit budget wins over the environment
    g = gtc.Graph(to_gpu(xyz), edges, tile_bytes=1 << 40)
    assert g.stats()["windows"] == 1
    g.close()


@pytest.mark.parametrize("csr_mode", ["device", "host"])
def test_torch_allocator_owns_the_graph_memory(gpu_available, csr_mode):
    # with a TorchAllocator every device buffer of the graph (and the pinned CSR) comes from
    # PyTorch's allocators: PyTorch's count rises by at least the CSR while the graph lives and
    # falls back once it is freed; the counts do not change
    import torch
    xyz = clustered(71, 20_000, 40, 2500)
    edges = linear_edges_sq(12_000, 8)
    w = 0.5 + rng_for(72).random(20_000)
    c0, w0, st0 = hip_3pcf(xyz, edges, w)
    xt = to_gpu(xyz)
    wt = torch.from_numpy(w).cuda()
    alloc = gtc.TorchAllocator()
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    kw = {} if csr_mode == "device" else {"tile_bytes": 4 * st0["edges"] // 4, "csr_mode": csr_mode}
    g = gtc.Graph(xt, edges, allocator=alloc, **kw)
    torch.cuda.synchronize()
    if csr_mode == "device":
        assert torch.cuda.memory_allocated() - base >= 4 * st0["edges"]
    else:
        assert alloc._pinned and g.stats()["windows"] > 1
    c, ws, st = g.count_3pcf(wt)
    np.testing.assert_array_equal(c.cpu().numpy().view(np.uint64), c0)
    np.testing.assert_array_equal(ws.cpu().numpy(), w0)
    del c, ws
    g.close()
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == base
    assert not alloc._pinned
    # the estimators take it too
    r = gtc.compute_3pcf(xt[:10_000].contiguous(), None, xt[10_000:].contiguous(), None,
                         edges_sq=edges, allocator=alloc)
    r0 = gtc.compute_3pcf(xt[:10_000].contiguous(), None, xt[10_000:].contiguous(), None,
                          edges_sq=edges)
    np.testing.assert_array_equal(r.zeta, r0.zeta)


def test_hbm_read_probe(gpu_available):
    # the streaming-read probe the bench reports as its measured ceiling: plausible on MI355X
    # (above a quarter of the 8 TB/s peak, not above the peak)
    import torch
    buf = torch.ones(1 << 26, dtype=torch.int32, device="cuda")  # 256 MiB
    rate = gtc.hbm_read_rate(buf, reps=3)
    assert 2000 < rate < 8500, rate


@pytest.mark.parametrize("csr_mode", ["host", "rebuild"])
def test_out_of_core_graph_serves_repeated_calls(gpu_available, csr_mode):
    # one out-of-core graph, used again and again: 3pCF counts (the first starts with the windows
    # the build left on the device, later ones with those the previous count left), a weighted
    # count, the 2pCF, the 4pCF and an export in between, all equal to the resident graph's
    import torch
    xyz = clustered(47, 20_000, 50, 2500)
    edges = linear_edges_sq(9_000, 6)
    w = torch.from_numpy(0.5 + rng_for(48).random(xyz.shape[0])).cuda()
    ref = gtc.Graph(to_gpu(xyz), edges)
    c0 = ref.count_3pcf()[0].cpu().numpy()
    c0w = ref.count_3pcf(w)[1].cpu().numpy()
    p0 = ref.count_2pcf()[0].cpu().numpy()
    e0 = ref.count_4pcf_parity()[0].cpu().numpy()
    x0 = edge_set_from_gpu(ref)
    tb = 4 * ref.stats()["edges"] // 6
    ref.close()
    g = gtc.Graph(to_gpu(xyz), edges, tile_bytes=tb, csr_mode=csr_mode)
    assert g.stats()["windows"] > 2
    for rep in range(2):
        say("ooc repeat", csr_mode, rep)
        np.testing.assert_array_equal(g.count_3pcf()[0].cpu().numpy(), c0)
        np.testing.assert_array_equal(g.count_3pcf(w)[1].cpu().numpy(), c0w)
        np.testing.assert_array_equal(g.count_2pcf()[0].cpu().numpy(), p0)
        np.testing.assert_array_equal(g.count_4pcf_parity()[0].cpu().numpy(), e0)
        np.testing.assert_array_equal(edge_set_from_gpu(g), x0)
    g.close()
    gtc.release_host_cache()


@pytest.mark.parametrize("layout", ["packed", "split"])
def test_device_window_plan_matches_host_planner(gpu_available, monkeypatch, layout):
    """The build plans its hub windows on the device; they are the host planner's windows for the
    graph's own CSR offsets, down to one row per window."""
    import ctypes as C
    if layout == "split":
        monkeypatch.setenv("GTC_CSR_LAYOUT", "split")
    entry = 5 if layout == "split" else 4
    xyz = clustered(45, 6000, 25, 3000)
    edges = linear_edges_sq(9000, 5)
    g0 = gtc.Graph(to_gpu(xyz), edges)
    rp = g0.export()[0]
    b0, o0 = g0.windows()
    g0.close()
    np.testing.assert_array_equal(b0, [0, 6000])
    np.testing.assert_array_equal(o0, [0, rp[-1]])
    max_row = int(np.diff(rp).max())
    for tb in (entry * rp[-1] // 3, entry * rp[-1] // 97, entry * max_row, entry * max_row - 1,
               entry, 1):
        g = gtc.Graph(to_gpu(xyz), edges, tile_bytes=int(tb))
        bounds, offsets = g.windows()
        want = np.empty(len(rp) + 1, np.int64)
        W = gtc.lib().gtc_plan_windows(rp.ctypes.data_as(C.c_void_p), len(rp) - 1, int(tb), entry,
                                       want.ctypes.data_as(C.c_void_p))
        say("window plan", layout, "tile_bytes", tb, "windows", W)
        assert g.stats()["windows"] == W == len(bounds) - 1
        np.testing.assert_array_equal(bounds, want[: W + 1])
        np.testing.assert_array_equal(offsets, rp[bounds])
        g.close()

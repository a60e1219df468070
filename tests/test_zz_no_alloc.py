"""GPU: the allocation-free 3pCF count (gtc_count_3pcf_noalloc, for callers that cannot allocate
device memory) equals gtc_count_3pcf bit for bit, on consecutive calls that share the static
scratch array (a larger input, then a smaller one), unweighted and weighted, and refuses what
the array cannot hold with an error."""
from __future__ import annotations

import numpy as np
import pytest

import graph_triangle_counting_amd as gtc
import oracle
from gpu_common import clustered, to_gpu, uniform
from workloads import linear_edges_sq, rng_for

pytestmark = pytest.mark.gpu


def both_counts(xyz, edges, w):
    import torch
    g = gtc.Graph(to_gpu(xyz), edges)
    wt = None if w is None else torch.from_numpy(w).cuda()
    ref_c, ref_w, _ = g.count_3pcf(wt)
    got_c, got_w = g.count_3pcf_noalloc(wt)
    torch.cuda.synchronize()
    out = (ref_c.cpu().numpy().view(np.uint64), got_c.cpu().numpy().view(np.uint64),
           None if w is None else ref_w.cpu().numpy(), None if w is None else got_w.cpu().numpy())
    g.close()
    return out


@pytest.mark.parametrize("weighted", [False, True])
def test_noalloc_count_matches_the_allocating_count(gpu_available, weighted):
    # two calls in a row on the shared array: a clustered set, then a smaller uniform one whose
    # histogram has fewer configurations (stale contents must not leak into the second call)
    big = clustered(501, 60_000, 40, 2500)
    small = uniform(502, 3_000)
    cases = [(big, linear_edges_sq(11_000, 14)), (small, linear_edges_sq(90_000, 5))]
    for k, (xyz, edges) in enumerate(cases):
        w = 0.5 + rng_for(503 + k).random(xyz.shape[0]) if weighted else None
        ref_c, got_c, ref_w, got_w = both_counts(xyz, edges, w)
        print("call", k, "points", xyz.shape[0], "triangles", int(ref_c.sum()), flush=True)
        assert ref_c.sum() > 0
        np.testing.assert_array_equal(got_c, ref_c)
        if weighted:
            np.testing.assert_array_equal(got_w, ref_w)
        if k == 1:  # the small case against the oracle as well
            oc, ow, _, _ = oracle.Graph(xyz, edges).count_3pcf(w)
            np.testing.assert_array_equal(got_c, oc)
            if weighted:
                np.testing.assert_array_equal(got_w, ow)


def test_noalloc_count_refuses_what_the_array_cannot_hold(gpu_available):
    import torch
    xyz = uniform(504, 4_000)
    edges = linear_edges_sq(60_000, 4)
    # hub windows over a resident CSR are counted, tile by tile
    g = gtc.Graph(to_gpu(xyz), edges, tile_bytes=1 << 14)
    assert g.stats()["windows"] > 1
    a, _, _ = g.count_3pcf()
    b, _ = g.count_3pcf_noalloc()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
    g.close()
    # a CSR out of core needs window buffers: refused
    for mode in ("host", "rebuild"):
        g = gtc.Graph(to_gpu(xyz), edges, tile_bytes=1 << 14, csr_mode=mode)
        with pytest.raises(gtc.GtcError) as ei:
            g.count_3pcf_noalloc()
        assert ei.value.status == gtc.GTC_E_UNSUPPORTED
        g.close()
    # weighted: 8 bytes per point do not fit 32 MiB at 4.5M points (refused before any launch)
    n = 4_500_000
    xyz = uniform(505, n)
    g = gtc.Graph(to_gpu(xyz), linear_edges_sq(2_000, 2))
    w = torch.full((n,), 1.0, dtype=torch.float64, device="cuda")
    with pytest.raises(gtc.GtcError) as ei:
        g.count_3pcf_noalloc(w)
    assert ei.value.status == gtc.GTC_E_UNSUPPORTED and "scratch" in str(ei.value)
    # the unweighted count of the same graph fits, and matches the allocating count
    a, _, _ = g.count_3pcf()
    b, _ = g.count_3pcf_noalloc()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
    g.close()

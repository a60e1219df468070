"""GPU at the full sizes of the two largest workloads (C3: 4M uniform points, 9e9 directed edges;
C5: 16M mixed points), where the oracle cannot count the whole histogram in a test's time:

* sampled hubs: the triangles of ~50 hubs (random labels plus the longest rows), counted by the
  library and by the per-hub oracle from the coordinates in the graph's internal order, bit-exact;
* the whole launch, in the configuration bench.py times, equals the sum of three separately
  launched hub subsets that partition every label (the batching and histogram exchanges of a
  full-size launch against independent schedules).
"""
from __future__ import annotations

import numpy as np
import pytest

import graph_triangle_counting_amd as gtc
import oracle
import workloads
from gpu_common import to_gpu
from workloads import rng_for

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("key", ["C3", "C5"])
def test_full_size_sampled_hubs_and_partition(gpu_available, key):
    cfg = workloads.get(key)
    xyz, _ = cfg.generate()
    n = xyz.shape[0]
    edges = cfg.edges_sq()
    say(key, "points", n)
    g = gtc.Graph(to_gpu(xyz), edges)
    full, _, st = g.count_3pcf()
    full = full.cpu().numpy().view(np.uint64)
    say(key, "full launch", st["triangles"], "kernel ms", st["kernel_ms"], "mode", st["launch_mode"])
    assert st["edges"] > 2**31  # 64-bit row offsets in use

    parts = np.array_split(rng_for(91).permutation(n).astype(np.int32), 3)
    tot = np.zeros_like(full)
    for part in parts:
        c, _, pst = g.count_3pcf_hubs(part)
        tot += c.cpu().numpy().view(np.uint64)
        say(key, "subset", part.size, "kernel ms", pst["kernel_ms"])
    np.testing.assert_array_equal(tot, full)

    perm, rp = g.perm(with_row_ptr=True)
    deg = np.diff(rp)
    sample = np.unique(np.concatenate([rng_for(92).choice(n, 44, replace=False),
                                       np.argsort(deg)[-4:], [0, n - 1]])).astype(np.int32)
    c, _, sst = g.count_3pcf_hubs(sample)
    g.close()
    got = c.cpu().numpy().view(np.uint64)
    say(key, "sampled hubs", sample.size, "max row", int(deg.max()), "triangles", int(got.sum()))
    want, _, _ = oracle.count_3pcf_hubs(xyz[perm], edges, sample)
    np.testing.assert_array_equal(got, want)
    assert got.sum() > 0

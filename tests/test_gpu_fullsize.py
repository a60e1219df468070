"""GPU at the full sizes of the two largest workloads, whole histograms against the oracle.

* BAO-scale 3pCF (4M uniform points, ~9e9 directed edges, 30 bins);
* large mixed 3pCF (16M points, half uniform and half Neyman-Scott, 16 bins).

The expected histograms are ``tests/golden/<key>_counts.npy``, written by
``tests/golden/make_fullsize_golden.py`` from the oracle alone (forward-row graph, the pages'
merge-walk over every hub).  The points are regenerated from the workload's seed and checked
against the recorded SHA-256 first.  Each workload is compared bit for bit in every mode the
library keeps its CSR in: resident, pinned host memory with the windows streamed per tile, and
windows emitted again per tile (GRAMSCI v2 §III.5.3; §IV.8 validates the chunked mode at
production scale the same way).
"""
from __future__ import annotations

import functools
import json
import os

import numpy as np
import pytest

import graph_triangle_counting_amd as gtc
import workloads
from gpu_common import to_gpu

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
GIB = 1 << 30


def say(*a):
    print(*a, flush=True)


def golden(key):
    f = os.path.join(GOLDEN, f"{key}_counts.npy")
    if not os.path.exists(f):
        pytest.skip(f"{f} not written yet (tests/golden/make_fullsize_golden.py {key})")
    with open(os.path.join(GOLDEN, f"{key}_counts.json")) as fh:
        meta = json.load(fh)
    return np.load(f), meta


@functools.lru_cache(maxsize=1)
def points(key):
    xyz, _ = workloads.get(key).generate()
    return xyz


@pytest.mark.parametrize("key,mode,tile", [
    ("C5", "device", 0), ("C5", "host", 2 * GIB), ("C5", "rebuild", 2 * GIB),
    ("C3", "device", 0), ("C3", "host", 4 * GIB), ("C3", "rebuild", 4 * GIB)])
def test_full_size_histogram_matches_the_oracle(gpu_available, key, mode, tile):
    want, meta = golden(key)
    cfg = workloads.get(key)
    xyz = points(key)
    assert workloads.coords_sha256(xyz) == meta["coords_sha256"], "generator changed"
    edges = cfg.edges_sq()
    assert [int(x) for x in edges] == meta["edges_sq"]
    say(key, mode, "tile bytes", tile, "points", xyz.shape[0])
    g = gtc.Graph(to_gpu(xyz), edges, tile_bytes=tile, csr_mode=mode)
    c, _, st = g.count_3pcf()
    got = c.cpu().numpy().view(np.uint64)
    gst = g.stats()
    g.close()
    say(key, mode, "windows", st["windows"], "tiles", st["tiles"], "kernel ms",
        round(st["kernel_ms"], 1), "triangles", st["triangles"])
    assert st["edges"] == meta["undirected_edges"] and st["edges"] > 2**31
    if tile:
        assert st["windows"] > 1 and gst["csr_mode"] == gtc.CSR_MODES[mode]
    np.testing.assert_array_equal(got, want)
    assert int(got.sum()) == meta["triangles"] == st["triangles"]

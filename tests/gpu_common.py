"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI and the oracle on
the same seeded inputs, and compare what is unique."""
from __future__ import annotations

import numpy as np

import graph_triangle_counting_amd as gtc
import oracle
from workloads import GRID, rng_for


def to_gpu(xyz):
    import torch
    return torch.from_numpy(np.ascontiguousarray(xyz, dtype=np.int32)).cuda()


def hip_3pcf(xyz, edges, w=None, **kw):
    import torch
    g = gtc.Graph(to_gpu(xyz), edges, **kw)
    wt = None if w is None else torch.from_numpy(np.asarray(w, np.float64)).cuda()
    c, ws, st = g.count_3pcf(wt)
    torch.cuda.synchronize()
    out = (c.cpu().numpy().view(np.uint64), None if ws is None else ws.cpu().numpy(), st)
    g.close()
    return out


def hip_4pcf(xyz, edges, **kw):
    import torch
    g = gtc.Graph(to_gpu(xyz), edges, **kw)
    e, o, st = g.count_4pcf_parity()
    torch.cuda.synchronize()
    out = (e.cpu().numpy().view(np.uint64), o.cpu().numpy(), st)
    g.close()
    return out


def edge_set_from_gpu(g: gtc.Graph):
    """(min label, max label, bin) of every edge of the HIP graph, in original labels, sorted."""
    rp, col, b, perm = g.export()
    n = rp.size - 1
    src = np.repeat(np.arange(n, dtype=np.int64), np.diff(rp))
    assert np.all(col > src[: col.size]), "rows hold forward neighbours only"
    for i in range(n):
        row = col[rp[i]:rp[i + 1]]
        assert np.all(np.diff(row) > 0), "rows ascending (Eq. 1)"
    a, c = perm[src].astype(np.int64), perm[col].astype(np.int64)
    key = np.stack([np.minimum(a, c), np.maximum(a, c), b.astype(np.int64)], 1)
    return key[np.lexsort(key.T[::-1])]


def edge_set_from_oracle(og: oracle.Graph):
    rp, col, b = og.export()
    src = np.repeat(np.arange(og.n, dtype=np.int64), np.diff(rp))
    keep = col > src
    key = np.stack([src[keep], col[keep].astype(np.int64), b[keep].astype(np.int64)], 1)
    return key[np.lexsort(key.T[::-1])]


def clustered(seed, n, nclust, sigma, box_lo=0, box_hi=GRID):
    rng = rng_for(seed)
    centres = box_lo + rng.random((nclust, 3)) * (box_hi - box_lo)
    xyz = centres[rng.integers(0, nclust, n)] + rng.normal(0.0, sigma, (n, 3))
    return np.clip(np.rint(xyz), 0, GRID - 1).astype(np.int32)


def uniform(seed, n, lo=0, hi=GRID):
    return rng_for(seed).integers(lo, hi, size=(n, 3)).astype(np.int32)


def host_internal_order(xyz, edges, return_keys: bool = False):
    """The internal labels the build's cell list defines, computed here on the host from that
    definition: cubic cells of integer side cs = ceil(r_max) (at most ~2n cells and 512 per axis),
    key (cz g + cy) g + cx, points ordered by key with ties in original order.  Returns
    perm (internal -> original label)."""
    n = xyz.shape[0]
    r2 = int(edges[-1])
    cs = int(np.ceil(np.sqrt(r2)))
    while cs * cs < r2:
        cs += 1
    while cs > 1 and (cs - 1) ** 2 >= r2:
        cs -= 1
    g = -(-GRID // cs)
    cap = 1
    while (cap + 1) ** 3 <= 2 * max(n, 1) and cap < 512:
        cap += 1
    if g > cap:
        g = cap
        cs = -(-GRID // g)
    c = xyz.astype(np.int64) // cs
    key = (c[:, 2] * g + c[:, 1]) * g + c[:, 0]
    perm = np.lexsort((np.arange(n), key)).astype(np.int32)
    return (perm, key) if return_keys else perm


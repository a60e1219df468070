"""ctypes loader for the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; the product package never imports it.  See ``oracle.h`` for
the definitions and the readings of the pages it follows.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle.build import build
            build()
        lib = C.CDLL(LIB_PATH)
        P = C.c_void_p
        i64, i32 = C.c_int64, C.c_int32
        lib.oracle_build_graph.argtypes = [i64, P, i32, P, i32, C.POINTER(P)]
        lib.oracle_build_graph_forward.argtypes = [i64, P, i32, P, i32, C.POINTER(P)]
        lib.oracle_graph_free.argtypes = [P]
        lib.oracle_graph_n.argtypes = [P]
        lib.oracle_graph_n.restype = i64
        lib.oracle_graph_nnz.argtypes = [P]
        lib.oracle_graph_nnz.restype = i64
        lib.oracle_graph_export.argtypes = [P, P, P, P]
        lib.oracle_num_configs.argtypes = [i32, i32]
        lib.oracle_num_configs.restype = i64
        lib.oracle_count_3pcf.argtypes = [P, P, i64, i32, P, P, P, P]
        lib.oracle_count_3pcf_part.argtypes = [P, P, i64, i64, i32, P, P, P, P]
        lib.oracle_count_3pcf_exact.argtypes = [P, P, i64, i32, P, P, P]
        lib.oracle_count_4pcf_parity.argtypes = [P, P, i64, i32, P, P, P]
        lib.oracle_forward_degrees.argtypes = [P, P]
        lib.oracle_count_3pcf_hubs.argtypes = [i64, P, i32, P, P, P, i64, i32, P, P, P]
        lib.oracle_num_configs_s4.argtypes = [i32]
        lib.oracle_num_configs_s4.restype = i64
        lib.oracle_config_bins_s4.argtypes = [i32, P]
        lib.oracle_config_realizable_s4.argtypes = [i32, P, P]
        lib.oracle_count_4pcf_parity_s4.argtypes = [P, P, i64, i32, P, P, P]
        lib.oracle_count_2pcf.argtypes = [P, P, P, P, P]
        lib.oracle_count_4pcf_weighted.argtypes = [P, P, P, i32, i32, P, P, P, P, P]
        lib.oracle_disconnected_4pcf_s4.argtypes = [i32, P, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def num_configs(order: int, nbins: int) -> int:
    return int(_load().oracle_num_configs(order, nbins))


def count_3pcf_hubs(xyz: np.ndarray, edges_sq, hubs, w: np.ndarray | None = None,
                    nthreads: int = 0):
    """Binned triangles whose smallest label is one of `hubs`, by definition from the coordinates
    (no graph).  Returns (counts uint64 [n_cfg], weighted fp64 [n_cfg] or None, scale s)."""
    lib = _load()
    xyz = np.ascontiguousarray(xyz, dtype=np.int32).reshape(-1, 3)
    e = np.ascontiguousarray(np.asarray(edges_sq, dtype=np.int64))
    h = np.ascontiguousarray(np.asarray(hubs, dtype=np.int32))
    nb = e.size - 1
    ncfg = num_configs(3, nb)
    counts = np.zeros(ncfg, np.uint64)
    weighted = None
    if w is not None:
        w = np.ascontiguousarray(w, dtype=np.float64)
        weighted = np.zeros(ncfg, np.float64)
    s = C.c_int32(0)
    rc = lib.oracle_count_3pcf_hubs(xyz.shape[0], _ptr(xyz), nb, _ptr(e), _ptr(w), _ptr(h),
                                    h.size, nthreads, _ptr(counts), _ptr(weighted), C.byref(s))
    if rc:
        raise ValueError(f"oracle_count_3pcf_hubs failed ({rc})")
    return counts, weighted, s.value


def num_configs_s4(nbins: int) -> int:
    """Number of S4 configurations of the 4pCF (six edge bins up to vertex relabelling)."""
    return int(_load().oracle_num_configs_s4(nbins))


def config_bins_s4(nbins: int) -> np.ndarray:
    """Canonical 6-tuples (edge order 01, 02, 03, 12, 13, 23) of the S4 configurations, int32
    [n_cfg, 6], in rank order."""
    out = np.zeros((num_configs_s4(nbins), 6), np.int32)
    if _load().oracle_config_bins_s4(nbins, _ptr(out)):
        raise ValueError("oracle_config_bins_s4 failed")
    return out


def config_realizable_s4(nbins: int, edges_sq) -> np.ndarray:
    """1 where a configuration's bin-centre edge lengths form a tetrahedron (Cayley-Menger)."""
    e = np.ascontiguousarray(np.asarray(edges_sq, dtype=np.int64))
    mask = np.zeros(num_configs_s4(nbins), np.uint8)
    if _load().oracle_config_realizable_s4(nbins, _ptr(e), _ptr(mask)):
        raise ValueError("oracle_config_realizable_s4 failed")
    return mask


def disconnected_4pcf_s4(nbins: int, xi) -> np.ndarray:
    """Eq. (4) per S4 configuration from the binned 2pCF xi [nbins]."""
    x = np.ascontiguousarray(np.asarray(xi, dtype=np.float64))
    out = np.zeros(num_configs_s4(nbins), np.float64)
    if _load().oracle_disconnected_4pcf_s4(nbins, _ptr(x), _ptr(out)):
        raise ValueError("oracle_disconnected_4pcf_s4 failed")
    return out


class Graph:
    """Oracle neighbour graph (caller's labels, rows ascending): full symmetric adjacency, or
    with forward_only=True only the neighbours above each label (half the memory; the counts are
    the same)."""

    def __init__(self, xyz: np.ndarray, edges_sq, nthreads: int = 0, forward_only: bool = False):
        lib = _load()
        self.xyz = np.ascontiguousarray(xyz, dtype=np.int32).reshape(-1, 3)
        self.edges = np.ascontiguousarray(np.asarray(edges_sq, dtype=np.int64))
        self.nbins = int(self.edges.size - 1)
        self.forward_only = bool(forward_only)
        h = C.c_void_p()
        build = lib.oracle_build_graph_forward if forward_only else lib.oracle_build_graph
        rc = build(self.xyz.shape[0], _ptr(self.xyz), self.nbins, _ptr(self.edges), nthreads,
                   C.byref(h))
        if rc:
            raise ValueError(f"oracle_build_graph failed ({rc})")
        self._h = h

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.oracle_graph_free(self._h)
            self._h = None

    @property
    def n(self) -> int:
        return int(_lib.oracle_graph_n(self._h))

    @property
    def nnz(self) -> int:
        return int(_lib.oracle_graph_nnz(self._h))

    def export(self):
        rp = np.empty(self.n + 1, np.int64)
        col = np.empty(max(self.nnz, 1), np.int32)
        b = np.empty(max(self.nnz, 1), np.uint8)
        assert _lib.oracle_graph_export(self._h, _ptr(rp), _ptr(col), _ptr(b)) == 0
        return rp, col[: self.nnz], b[: self.nnz]

    def forward_degrees(self) -> np.ndarray:
        d = np.empty(self.n, np.int32)
        assert _lib.oracle_forward_degrees(self._h, _ptr(d)) == 0
        return d

    def count_3pcf(self, w: np.ndarray | None = None, hub_stride: int = 1, nthreads: int = 0,
                   hub_offset: int = 0):
        """Returns (counts uint64[n_cfg], weighted fp64[n_cfg] or None, scale s, walks) over the
        hubs i with i % hub_stride == hub_offset."""
        ncfg = num_configs(3, self.nbins)
        counts = np.zeros(ncfg, np.uint64)
        weighted = None if w is None else np.zeros(ncfg, np.float64)
        wa = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
        s = C.c_int32(0)
        walks = C.c_uint64(0)
        rc = _lib.oracle_count_3pcf_part(self._h, _ptr(wa), hub_stride, hub_offset, nthreads,
                                         _ptr(counts), _ptr(weighted), C.byref(s),
                                         C.byref(walks))
        if rc:
            raise ValueError(f"oracle_count_3pcf failed ({rc})")
        return counts, weighted, int(s.value), int(walks.value)

    def count_3pcf_exact(self, w: np.ndarray, hub_stride: int = 1, nthreads: int = 0):
        """Returns (counts, exact integer sums of q as Python ints, scale s)."""
        ncfg = num_configs(3, self.nbins)
        counts = np.zeros(ncfg, np.uint64)
        q = np.zeros(2 * ncfg, np.int64)
        wa = np.ascontiguousarray(w, dtype=np.float64)
        s = C.c_int32(0)
        rc = _lib.oracle_count_3pcf_exact(self._h, _ptr(wa), hub_stride, nthreads, _ptr(counts),
                                          _ptr(q), C.byref(s))
        if rc:
            raise ValueError(f"oracle_count_3pcf_exact failed ({rc})")
        u = q.view(np.uint64)
        sums = []
        for c in range(ncfg):
            v = int(u[2 * c]) | (int(u[2 * c + 1]) << 64)
            if v >= 1 << 127:
                v -= 1 << 128
            sums.append(v)
        return counts, sums, int(s.value)

    def count_4pcf_weighted(self, w: np.ndarray, s4: bool = False, nthreads: int = 0):
        """(even uint64, odd int64, even_w fp64, odd_w fp64 [n_cfg], scale s)."""
        ncfg = num_configs_s4(self.nbins) if s4 else num_configs(4, self.nbins)
        even = np.zeros(ncfg, np.uint64)
        odd = np.zeros(ncfg, np.int64)
        ew = np.zeros(ncfg, np.float64)
        ow = np.zeros(ncfg, np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        sc = C.c_int32(0)
        rc = _lib.oracle_count_4pcf_weighted(self._h, _ptr(self.xyz), _ptr(w), int(s4), nthreads,
                                             _ptr(even), _ptr(odd), _ptr(ew), _ptr(ow), C.byref(sc))
        if rc:
            raise ValueError(f"oracle_count_4pcf_weighted failed ({rc})")
        return even, odd, ew, ow, sc.value

    def count_2pcf(self, w: np.ndarray | None = None):
        """Pairs per bin: (counts uint64 [nbins], weighted fp64 [nbins] or None, scale s)."""
        counts = np.zeros(self.nbins, np.uint64)
        weighted = None
        if w is not None:
            w = np.ascontiguousarray(w, dtype=np.float64)
            weighted = np.zeros(self.nbins, np.float64)
        sc = C.c_int32(0)
        rc = _lib.oracle_count_2pcf(self._h, _ptr(w), _ptr(counts), _ptr(weighted), C.byref(sc))
        if rc:
            raise ValueError(f"oracle_count_2pcf failed ({rc})")
        return counts, weighted, sc.value

    def count_4pcf_parity(self, hub_stride: int = 1, nthreads: int = 0, s4: bool = False):
        """Returns (even uint64[n_cfg], odd int64[n_cfg], number of 4-cliques); configurations
        are sorted 6-tuples, or S4 configurations with s4=True."""
        ncfg = num_configs_s4(self.nbins) if s4 else num_configs(4, self.nbins)
        even = np.zeros(ncfg, np.uint64)
        odd = np.zeros(ncfg, np.int64)
        cl = C.c_uint64(0)
        fn = _lib.oracle_count_4pcf_parity_s4 if s4 else _lib.oracle_count_4pcf_parity
        rc = fn(self._h, _ptr(self.xyz), hub_stride, nthreads, _ptr(even), _ptr(odd),
                C.byref(cl))
        if rc:
            raise ValueError(f"oracle_count_4pcf_parity failed ({rc})")
        return even, odd, int(cl.value)

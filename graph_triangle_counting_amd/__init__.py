"""Python binding of libgtc, the MI355X graph 3pCF / 4pCF counter (GRAMSCI v2 method).

Argument marshalling only: every step of the counting runs in the HIP kernels of libgtc.so,
called through its C ABI (include/gtc.h).  PyTorch supplies device memory and the current
stream.  Importing succeeds without the library (so CPU-only tooling can inspect the package),
but every call raises if libgtc.so is absent: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgtc.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "gtc.h")

GTC_OK, GTC_E_INVALID, GTC_E_OOM, GTC_E_HIP, GTC_E_OVERFLOW, GTC_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5
# where the CSR is kept (gtc_options.csr_mode)
CSR_MODES = {"device": 0, "host": 1, "rebuild": 2}


class GtcError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status


_ALLOC = C.CFUNCTYPE(C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p)
_FREE = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p, C.c_void_p)
_HOST_ALLOC = C.CFUNCTYPE(C.c_void_p, C.c_size_t, C.c_void_p)
_HOST_FREE = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p)


class Allocator(C.Structure):
    """gtc_allocator: memory routines the library calls instead of the HIP runtime's."""
    _fields_ = [("alloc", _ALLOC), ("free", _FREE), ("host_alloc", _HOST_ALLOC),
                ("host_free", _HOST_FREE), ("ctx", C.c_void_p)]


class Options(C.Structure):
    _fields_ = [("tile_bytes", C.c_int64), ("csr_mode", C.c_int32), ("drop_coords", C.c_int32),
                ("allocator", C.POINTER(Allocator))]


class TorchAllocator:
    """Routes the library's device memory through PyTorch's caching allocator (stream-ordered
    on the stream the library passes) and its pinned host memory through pinned torch tensors, so
    that PyTorch accounts for every buffer.  Keep the object alive as long as any graph built with
    it (Graph holds a reference)."""

    def __init__(self):
        import torch
        self._pinned = {}

        def alloc(nbytes, stream, ctx):
            try:
                return torch.cuda.caching_allocator_alloc(int(nbytes), stream=int(stream or 0))
            except Exception:
                return None

        def free(ptr, stream, ctx):
            if ptr:
                torch.cuda.caching_allocator_delete(ptr)

        def host_alloc(nbytes, ctx):
            try:
                t = torch.empty(int(nbytes), dtype=torch.uint8, pin_memory=True)
            except Exception:
                return None
            self._pinned[t.data_ptr()] = t
            return t.data_ptr()

        def host_free(ptr, ctx):
            self._pinned.pop(ptr, None)

        self._cbs = (_ALLOC(alloc), _FREE(free), _HOST_ALLOC(host_alloc), _HOST_FREE(host_free))
        self.struct = Allocator(*self._cbs, None)


class Stats(C.Structure):
    _fields_ = [("n", C.c_int64), ("edges", C.c_int64), ("max_out_degree", C.c_int64),
                ("merge_walks", C.c_int64), ("spoke_elements", C.c_int64), ("tiles", C.c_int64),
                ("windows", C.c_int64), ("triangles", C.c_uint64), ("cliques4", C.c_uint64),
                ("q_alg_bytes", C.c_double), ("weight_scale", C.c_int32),
                ("launch_waves", C.c_int32), ("launch_blocks", C.c_int32),
                ("launch_lds_bytes", C.c_int32), ("launch_mode", C.c_int32),
                ("csr_mode", C.c_int32), ("build_ms", C.c_double), ("kernel_ms", C.c_double),
                ("count_ms", C.c_double), ("h2d_ms", C.c_double)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None


def lib() -> C.CDLL:
    """Load libgtc.so (built in-tree by graph_triangle_counting_amd/_build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python graph_triangle_counting_amd/_build.py`")
        L = C.CDLL(LIB_PATH)
        P, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.gtc_build_graph.argtypes = [P, i64, P, i32, C.POINTER(Options), P, C.POINTER(P)]
        L.gtc_count_3pcf.argtypes = [P, P, P, P, C.POINTER(Stats), P]
        L.gtc_count_3pcf_hubs.argtypes = [P, P, i64, P, P, P, C.POINTER(Stats), P]
        L.gtc_count_3pcf_noalloc.argtypes = [P, P, P, P, P]
        L.gtc_release_host_cache.argtypes = []
        L.gtc_release_host_cache.restype = None
        L.gtc_count_4pcf_parity_s4.argtypes = [P, P, P, C.POINTER(Stats), P]
        L.gtc_num_configs_s4.argtypes = [i32]
        L.gtc_num_configs_s4.restype = i64
        L.gtc_config_bins_s4.argtypes = [i32, P]
        L.gtc_config_realizable_s4.argtypes = [i32, P, P]
        L.gtc_count_2pcf.argtypes = [P, P, P, P, C.POINTER(Stats), P]
        L.gtc_disconnected_4pcf_s4.argtypes = [i32, P, P]
        L.gtc_connected_4pcf_s4.argtypes = [i32, P, P, P]
        L.gtc_count_4pcf_parity.argtypes = [P, P, P, C.POINTER(Stats), P]
        L.gtc_count_4pcf_weighted.argtypes = [P, P, i32, P, P, P, P, C.POINTER(Stats), P]
        L.gtc_linear_edges_sq.argtypes = [i64, i64, i32, P]
        L.gtc_equilateral_configs.argtypes = [i32, i32, i32, P]
        L.gtc_hbm_read_rate.argtypes = [P, i64, i32, P, P]
        L.gtc_compute_3pcf.argtypes = [P, i64, P, P, i64, P, P, i32, C.POINTER(Options), P, P, P,
                                       C.POINTER(Stats), P]
        L.gtc_compute_4pcf.argtypes = [P, i64, P, P, i64, P, P, i32, C.POINTER(Options), P, P, P,
                                       P, C.POINTER(Stats), P]
        L.gtc_num_configs.argtypes = [i32, i32]
        L.gtc_num_configs.restype = i64
        L.gtc_config_bins.argtypes = [i32, i32, P]
        L.gtc_graph_export.argtypes = [P, P, P, P, P]
        L.gtc_graph_stats.argtypes = [P, C.POINTER(Stats)]
        L.gtc_plan_windows.argtypes = [P, i64, i64, i32, P]
        L.gtc_plan_windows.restype = i64
        L.gtc_graph_windows.argtypes = [P, P, P, i64]
        L.gtc_graph_windows.restype = i64
        L.gtc_graph_free.argtypes = [P]
        L.gtc_graph_free.restype = None
        L.gtc_status_string.argtypes = [C.c_int]
        L.gtc_status_string.restype = C.c_char_p
        L.gtc_last_error.argtypes = []
        L.gtc_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != GTC_OK:
        raise GtcError(rc, lib().gtc_last_error().decode())


def _stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dptr(t):
    return C.c_void_p(t.data_ptr())


def num_configs(order: int, nbins: int) -> int:
    v = lib().gtc_num_configs(order, nbins)
    if v < 0:
        raise ValueError(f"no configurations for order {order}, nbins {nbins}")
    return int(v)


def config_bins(order: int, nbins: int) -> np.ndarray:
    """Bins of every configuration in rank order: int32 [n_cfg, 3 or 6]."""
    k = 3 if order == 3 else 6
    out = np.empty((num_configs(order, nbins), k), np.int32)
    _check(lib().gtc_config_bins(order, nbins, out.ctypes.data_as(C.c_void_p)))
    return out


def num_configs_s4(nbins: int) -> int:
    """Number of S4 configurations of the 4pCF (six edge bins up to vertex relabelling)."""
    v = lib().gtc_num_configs_s4(nbins)
    if v < 0:
        raise ValueError(f"no S4 configurations for nbins {nbins}")
    return int(v)


def config_bins_s4(nbins: int) -> np.ndarray:
    """Canonical tuples of the S4 configurations (edge order 01, 02, 03, 12, 13, 23): int32
    [n_cfg, 6] in rank order."""
    out = np.empty((num_configs_s4(nbins), 6), np.int32)
    _check(lib().gtc_config_bins_s4(nbins, out.ctypes.data_as(C.c_void_p)))
    return out


def config_realizable_s4(nbins: int, edges_sq) -> np.ndarray:
    """uint8 [n_cfg]: 1 where the configuration's bin centres form a tetrahedron."""
    e = np.ascontiguousarray(np.asarray(edges_sq, dtype=np.int64))
    mask = np.empty(num_configs_s4(nbins), np.uint8)
    _check(lib().gtc_config_realizable_s4(nbins, e.ctypes.data_as(C.c_void_p),
                                          mask.ctypes.data_as(C.c_void_p)))
    return mask


def disconnected_4pcf_s4(nbins: int, xi) -> np.ndarray:
    """Eq. (4) per S4 configuration from the binned 2pCF xi [nbins] (host)."""
    x = np.ascontiguousarray(np.asarray(xi, dtype=np.float64))
    out = np.empty(num_configs_s4(nbins), np.float64)
    _check(lib().gtc_disconnected_4pcf_s4(nbins, x.ctypes.data_as(C.c_void_p),
                                          out.ctypes.data_as(C.c_void_p)))
    return out


def connected_4pcf_s4(nbins: int, zeta, xi) -> np.ndarray:
    """Eq. (5): zeta minus the disconnected part, per S4 configuration (host)."""
    x = np.ascontiguousarray(np.asarray(xi, dtype=np.float64))
    z = np.ascontiguousarray(np.asarray(zeta, dtype=np.float64))
    out = np.empty(num_configs_s4(nbins), np.float64)
    _check(lib().gtc_connected_4pcf_s4(nbins, z.ctypes.data_as(C.c_void_p),
                                       x.ctypes.data_as(C.c_void_p),
                                       out.ctypes.data_as(C.c_void_p)))
    return out


class Graph:
    """Neighbour graph on the current GPU (owned by libgtc; freed by close() or on deletion)."""

    def __init__(self, xyz, edges_sq, tile_bytes: int = 0, host_csr: bool = False,
                 drop_coords: bool = False, stream=None, csr_mode: str | None = None,
                 allocator: TorchAllocator | None = None):
        """csr_mode: "device" (default), "host" (pinned host CSR; host_csr=True is the same) or
        "rebuild" (no stored CSR, windows emitted again per tile); the last two need tile_bytes.
        allocator: a TorchAllocator to take every buffer from PyTorch's allocators."""
        import torch
        if not (isinstance(xyz, torch.Tensor) and xyz.is_cuda and xyz.dtype == torch.int32
                and xyz.dim() == 2 and xyz.shape[1] == 3):
            raise TypeError("xyz must be a CUDA int32 tensor of shape [n, 3]")
        self._xyz = xyz.contiguous()
        e = np.ascontiguousarray(np.asarray(edges_sq, dtype=np.int64))
        self.nbins = int(e.size - 1)
        self.edges = e
        self.n = int(xyz.shape[0])
        mode = CSR_MODES[csr_mode] if csr_mode is not None else (1 if host_csr else 0)
        self._allocator = allocator  # the routines must outlive the graph
        opt = Options(int(tile_bytes), mode, int(bool(drop_coords)),
                      C.pointer(allocator.struct) if allocator is not None else None)
        h = C.c_void_p()
        self._stream = stream
        _check(lib().gtc_build_graph(_dptr(self._xyz) if self.n else None, self.n,
                                     e.ctypes.data_as(C.c_void_p), self.nbins, C.byref(opt),
                                     _stream_ptr(stream), C.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().gtc_graph_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def stats(self) -> dict:
        st = Stats()
        _check(lib().gtc_graph_stats(self._h, C.byref(st)))
        return st.as_dict()

    def count_3pcf(self, w=None, out=None, out_weighted=None):
        """Binned triangle counts.  Returns (counts int64 [n_cfg] on the GPU, holding the uint64
        bit pattern; weighted fp64 [n_cfg] or None; stats dict)."""
        import torch
        ncfg = num_configs(3, self.nbins)
        dev = self._xyz.device
        counts = out if out is not None else torch.empty(ncfg, dtype=torch.int64, device=dev)
        weighted = None
        if w is not None:
            if not (w.is_cuda and w.dtype == torch.float64 and w.numel() == self.n):
                raise TypeError("w must be a CUDA float64 tensor of length n")
            w = w.contiguous()
            weighted = out_weighted if out_weighted is not None else \
                torch.empty(ncfg, dtype=torch.float64, device=dev)
        st = Stats()
        _check(lib().gtc_count_3pcf(self._h, _dptr(w) if w is not None else None, _dptr(counts),
                                    _dptr(weighted) if weighted is not None else None,
                                    C.byref(st), _stream_ptr(self._stream)))
        return counts, weighted, st.as_dict()

    def count_3pcf_noalloc(self, w=None, out=None, out_weighted=None):
        """count_3pcf through gtc_count_3pcf_noalloc: no device allocation in the library (its
        scratch is a static device array), no statistics.  The output tensors may be passed in
        (out, out_weighted), so that the call allocates nothing at all.  Returns (counts,
        weighted or None)."""
        import torch
        ncfg = num_configs(3, self.nbins)
        dev = self._xyz.device
        counts = out if out is not None else torch.empty(ncfg, dtype=torch.int64, device=dev)
        weighted = None
        if w is not None:
            if not (w.is_cuda and w.dtype == torch.float64 and w.numel() == self.n):
                raise TypeError("w must be a CUDA float64 tensor of length n")
            w = w.contiguous()
            weighted = out_weighted if out_weighted is not None else \
                torch.empty(ncfg, dtype=torch.float64, device=dev)
        _check(lib().gtc_count_3pcf_noalloc(self._h, _dptr(w) if w is not None else None,
                                            _dptr(counts),
                                            _dptr(weighted) if weighted is not None else None,
                                            _stream_ptr(self._stream)))
        return counts, weighted

    def count_2pcf(self, w=None):
        """Pairs per bin: (counts int64 [nbins] holding uint64 bits, weighted fp64 [nbins] or None,
        stats)."""
        import torch
        dev = self._xyz.device
        counts = torch.empty(self.nbins, dtype=torch.int64, device=dev)
        weighted = None
        if w is not None:
            if not (w.is_cuda and w.dtype == torch.float64 and w.numel() == self.n):
                raise TypeError("w must be a CUDA float64 tensor of length n")
            w = w.contiguous()
            weighted = torch.empty(self.nbins, dtype=torch.float64, device=dev)
        st = Stats()
        _check(lib().gtc_count_2pcf(self._h, _dptr(w) if w is not None else None, _dptr(counts),
                                    _dptr(weighted) if weighted is not None else None,
                                    C.byref(st), _stream_ptr(self._stream)))
        return counts, weighted, st.as_dict()

    def count_3pcf_hubs(self, hubs, w=None):
        """Binned triangles whose first vertex in the internal order is one of `hubs` (distinct
        internal labels; see perm()).  Returns (counts, weighted or None, stats) as count_3pcf."""
        import torch
        h = np.ascontiguousarray(np.asarray(hubs, dtype=np.int32))
        ncfg = num_configs(3, self.nbins)
        dev = self._xyz.device
        counts = torch.empty(ncfg, dtype=torch.int64, device=dev)
        weighted = None
        if w is not None:
            if not (w.is_cuda and w.dtype == torch.float64 and w.numel() == self.n):
                raise TypeError("w must be a CUDA float64 tensor of length n")
            w = w.contiguous()
            weighted = torch.empty(ncfg, dtype=torch.float64, device=dev)
        st = Stats()
        _check(lib().gtc_count_3pcf_hubs(self._h, h.ctypes.data_as(C.c_void_p), h.size,
                                         _dptr(w) if w is not None else None, _dptr(counts),
                                         _dptr(weighted) if weighted is not None else None,
                                         C.byref(st), _stream_ptr(self._stream)))
        return counts, weighted, st.as_dict()

    def perm(self, with_row_ptr: bool = False):
        """Internal label -> point index (host int32 [n]); with_row_ptr also returns the forward
        CSR offsets (host int64 [n+1]) without copying the rows out."""
        perm = np.empty(max(self.n, 1), np.int32)
        rp = np.empty(self.n + 1, np.int64) if with_row_ptr else None
        p = lambda a: None if a is None else a.ctypes.data_as(C.c_void_p)
        _check(lib().gtc_graph_export(self._h, p(rp), None, None, p(perm)))
        return (perm[: self.n], rp) if with_row_ptr else perm[: self.n]

    def count_4pcf_parity(self, s4: bool = False):
        """Binned 4-clique counts: (even int64 [n_cfg] holding uint64 bits, odd int64, stats);
        configurations are sorted 6-tuples, or S4 configurations with s4=True."""
        import torch
        ncfg = num_configs_s4(self.nbins) if s4 else num_configs(4, self.nbins)
        dev = self._xyz.device
        even = torch.empty(ncfg, dtype=torch.int64, device=dev)
        odd = torch.empty(ncfg, dtype=torch.int64, device=dev)
        st = Stats()
        fn = lib().gtc_count_4pcf_parity_s4 if s4 else lib().gtc_count_4pcf_parity
        _check(fn(self._h, _dptr(even), _dptr(odd), C.byref(st), _stream_ptr(self._stream)))
        return even, odd, st.as_dict()

    def count_4pcf_weighted(self, w, s4: bool = False):
        """Weighted parity 4pCF: (even, odd as count_4pcf_parity; even_w, odd_w fp64 [n_cfg] on
        the GPU, the exact sums of the four-weight products and of their signed-volume signs;
        stats, weight_scale = s)."""
        import torch
        if not (isinstance(w, torch.Tensor) and w.is_cuda and w.dtype == torch.float64
                and w.numel() == self.n):
            raise TypeError("w must be a CUDA float64 tensor of length n")
        w = w.contiguous()
        ncfg = num_configs_s4(self.nbins) if s4 else num_configs(4, self.nbins)
        dev = self._xyz.device
        even = torch.empty(ncfg, dtype=torch.int64, device=dev)
        odd = torch.empty(ncfg, dtype=torch.int64, device=dev)
        ew = torch.empty(ncfg, dtype=torch.float64, device=dev)
        ow = torch.empty(ncfg, dtype=torch.float64, device=dev)
        st = Stats()
        _check(lib().gtc_count_4pcf_weighted(self._h, _dptr(w), int(bool(s4)), _dptr(even),
                                             _dptr(odd), _dptr(ew), _dptr(ow), C.byref(st),
                                             _stream_ptr(self._stream)))
        return even, odd, ew, ow, st.as_dict()

    def windows(self):
        """Hub windows: (label bounds int64 [W+1], their CSR offsets int64 [W+1]) on the host."""
        W = lib().gtc_graph_windows(self._h, None, None, 0)
        _check(int(W) if W < 0 else 0)
        bounds = np.empty(W + 1, np.int64)
        offsets = np.empty(W + 1, np.int64)
        p = lambda a: a.ctypes.data_as(C.c_void_p)
        _check(min(0, int(lib().gtc_graph_windows(self._h, p(bounds), p(offsets), W + 1))))
        return bounds, offsets

    def export(self):
        """Forward CSR in internal labels plus the internal -> original permutation (host)."""
        st = self.stats()
        e = int(st["edges"])
        rp = np.empty(self.n + 1, np.int64)
        col = np.empty(max(e, 1), np.int32)
        b = np.empty(max(e, 1), np.uint8)
        perm = np.empty(max(self.n, 1), np.int32)
        p = lambda a: a.ctypes.data_as(C.c_void_p)
        _check(lib().gtc_graph_export(self._h, p(rp), p(col), p(b), p(perm)))
        return rp, col[:e], b[:e], perm[: self.n]


def build_graph(xyz, edges_sq, **kw) -> Graph:
    return Graph(xyz, edges_sq, **kw)


def release_host_cache() -> None:
    """Free the pinned host block kept for reuse by out-of-core builds."""
    lib().gtc_release_host_cache()


def linear_edges_sq(r_min: int, r_max: int, nbins: int) -> np.ndarray:
    """Integer squared edges of nbins equal bins in r from r_min to r_max (grid units)."""
    e = np.empty(int(nbins) + 1, np.int64)
    _check(lib().gtc_linear_edges_sq(int(r_min), int(r_max), int(nbins),
                                     e.ctypes.data_as(C.c_void_p)))
    return e


def hbm_read_rate(buf, reps: int = 5, stream=None) -> float:
    """GB/s that a plain streaming-read kernel reaches over the CUDA tensor buf."""
    g = C.c_double(0.0)
    _check(lib().gtc_hbm_read_rate(_dptr(buf), buf.numel() * buf.element_size(), int(reps),
                                   C.byref(g), _stream_ptr(stream)))
    return g.value


def equilateral_configs(order: int, nbins: int, s4: bool = False) -> np.ndarray:
    """int64 [nbins]: the rank of the configuration with every edge in bin b (the equilateral
    3pCF's configurations; order 4: the regular tetrahedra, sorted 6-tuples or S4)."""
    out = np.empty(int(nbins), np.int64)
    _check(lib().gtc_equilateral_configs(int(order), int(bool(s4)), int(nbins),
                                         out.ctypes.data_as(C.c_void_p)))
    return out


class Result3pcf:
    """compute_3pcf's result: zeta, NNN, RRR per configuration (fp64 host arrays); bins
    [n_cfg][3] the nondecreasing bin triple of each configuration; r1, r2, r3 its bin centres
    (midpoints in r, grid units); edges_sq the squared edges; stats.  equilateral() gives the
    equilateral 3pCF, one value per bin."""

    def equilateral(self) -> dict:
        """The configurations with all three sides in one bin: r (bin centres), zeta, NNN, RRR."""
        k = equilateral_configs(3, self.edges_sq.size - 1)
        return {"r": self.r1[k], "zeta": self.zeta[k], "NNN": self.NNN[k], "RRR": self.RRR[k]}


class Result4pcf:
    """compute_4pcf's result: zeta_even, zeta_odd, zeta_conn per S4 configuration, xi per bin
    (fp64 host arrays); bins [n_cfg][6] the canonical edge-bin tuple (edge order 01, 02, 03, 12,
    13, 23); r1..r6 their bin centres; realizable the Cayley-Menger mask of the bin centres;
    edges_sq; stats."""


def _catalogue(xyz, w, name):
    import torch
    if not (isinstance(xyz, torch.Tensor) and xyz.is_cuda and xyz.dtype == torch.int32
            and xyz.dim() == 2 and xyz.shape[1] == 3):
        raise TypeError(f"{name} positions must be a CUDA int32 tensor of shape [n, 3]")
    xyz = xyz.contiguous()
    if w is not None:
        if not (isinstance(w, torch.Tensor) and w.is_cuda and w.dtype == torch.float64
                and w.numel() == xyz.shape[0]):
            raise TypeError(f"{name} weights must be a CUDA float64 tensor of length n")
        w = w.contiguous()
    return xyz, w


def _estimator_args(pos_data, w_data, pos_rand, w_rand, rmin, rmax, nbins, edges_sq,
                    tile_bytes, csr_mode, allocator=None):
    xd, wd = _catalogue(pos_data, w_data, "data")
    xr, wr = _catalogue(pos_rand, w_rand, "random")
    if edges_sq is None:
        edges_sq = linear_edges_sq(rmin, rmax, nbins)
    e = np.ascontiguousarray(np.asarray(edges_sq, dtype=np.int64))
    opt = Options(int(tile_bytes), CSR_MODES[csr_mode or "device"], 0,
                  C.pointer(allocator.struct) if allocator is not None else None)
    return xd, wd, xr, wr, e, opt


def _centres(e: np.ndarray) -> np.ndarray:
    r = np.sqrt(e.astype(np.float64))
    return 0.5 * (r[:-1] + r[1:])


def compute_3pcf(pos_data, w_data, pos_rand, w_rand, rmin=None, rmax=None, nbins=None,
                 edges_sq=None, tile_bytes: int = 0, csr_mode: str | None = None,
                 stream=None, allocator: TorchAllocator | None = None) -> Result3pcf:
    """The 3pCF estimator zeta = NNN / RRR over one graph of data and randoms.  Positions are
    CUDA int32 [n, 3] grid coordinates, weights CUDA float64 [n] or None (unit); the bins are
    equal in r from rmin to rmax (grid units), or given as integer squared edges."""
    xd, wd, xr, wr, e, opt = _estimator_args(pos_data, w_data, pos_rand, w_rand, rmin, rmax,
                                             nbins, edges_sq, tile_bytes, csr_mode, allocator)
    nb = e.size - 1
    ncfg = num_configs(3, nb)
    zeta, nnn, rrr = (np.empty(ncfg, np.float64) for _ in range(3))
    st = Stats()
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    _check(lib().gtc_compute_3pcf(_dptr(xd) if xd.shape[0] else None, xd.shape[0],
                                  _dptr(wd) if wd is not None else None, _dptr(xr), xr.shape[0],
                                  _dptr(wr) if wr is not None else None, p(e), nb, C.byref(opt),
                                  p(zeta), p(nnn), p(rrr), C.byref(st), _stream_ptr(stream)))
    r = Result3pcf()
    r.zeta, r.NNN, r.RRR, r.edges_sq, r.stats = zeta, nnn, rrr, e, st.as_dict()
    r.bins = config_bins(3, nb)
    c = _centres(e)
    r.r1, r.r2, r.r3 = (c[r.bins[:, k]] for k in range(3))
    return r


def compute_4pcf(pos_data, w_data, pos_rand, w_rand, rmin=None, rmax=None, nbins=None,
                 edges_sq=None, parity: bool = True, tile_bytes: int = 0,
                 csr_mode: str | None = None, stream=None,
                 allocator: TorchAllocator | None = None) -> Result4pcf:
    """The 4pCF estimator per S4 configuration: zeta_even = NNNN_even / RRRR, zeta_odd =
    NNNN_odd / RRRR, the internal xi = NN / RR and the connected zeta_conn = zeta_even -
    disc(xi).  Arguments as compute_3pcf; nbins <= 16.  Both channels come from one enumeration,
    so parity=False only drops zeta_odd from the result."""
    xd, wd, xr, wr, e, opt = _estimator_args(pos_data, w_data, pos_rand, w_rand, rmin, rmax,
                                             nbins, edges_sq, tile_bytes, csr_mode, allocator)
    nb = e.size - 1
    ncfg = num_configs_s4(nb)
    ze, zo, zc = (np.empty(ncfg, np.float64) for _ in range(3))
    xi = np.empty(nb, np.float64)
    st = Stats()
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    _check(lib().gtc_compute_4pcf(_dptr(xd) if xd.shape[0] else None, xd.shape[0],
                                  _dptr(wd) if wd is not None else None, _dptr(xr), xr.shape[0],
                                  _dptr(wr) if wr is not None else None, p(e), nb, C.byref(opt),
                                  p(ze), p(zo), p(zc), p(xi), C.byref(st), _stream_ptr(stream)))
    r = Result4pcf()
    r.zeta_even, r.zeta_odd, r.zeta_conn, r.xi = ze, (zo if parity else None), zc, xi
    r.edges_sq, r.stats = e, st.as_dict()
    r.bins = config_bins_s4(nb)
    c = _centres(e)
    r.r1, r.r2, r.r3, r.r4, r.r5, r.r6 = (c[r.bins[:, k]] for k in range(6))
    r.realizable = config_realizable_s4(nb, e).astype(bool)
    return r


def header_functions() -> list[str]:
    """Names of the functions include/gtc.h declares."""
    import re
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(gtc_\w+)\s*\(", src, flags=re.M)))

// api.hip - the extern "C" boundary of libgtc: argument checks, handle lifetime, dispatch.
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "gtc_internal.h"

namespace gtc {
const char *last_error();
int build_graph_device(gtc_graph_s *G, const int32_t *d_xyz, hipStream_t s);
int count_3pcf_device(gtc_graph_s *G, const double *d_w, uint64_t *d_counts, double *d_weighted,
                      gtc_stats *st, hipStream_t s, const HubSubset *sub = nullptr,
                      const ExternalScratch *ext = nullptr);
int count_4pcf_device(gtc_graph_s *G, uint64_t *d_even, int64_t *d_odd, gtc_stats *st,
                      hipStream_t s, bool s4, const double *d_w = nullptr,
                      double *d_even_w = nullptr, double *d_odd_w = nullptr);
void config_realizable_s4(int nb, const int64_t *edges, uint8_t *mask);
int count_2pcf_device(gtc_graph_s *G, const double *d_w, uint64_t *d_counts, double *d_weighted,
                      gtc_stats *st, hipStream_t s);
void free_graph_buffers(gtc_graph_s *G);

static int64_t binom(int64_t n, int64_t k) {
    if (k < 0 || n < k) return 0;
    int64_t r = 1;
    for (int64_t t = 1; t <= k; ++t) r = r * (n - k + t) / t;
    return r;
}

void free_graph_buffers(gtc_graph_s *G) {
    hipStream_t s = G->stream;
    if (G->xfer) {  // transfers into the pinned CSR and window buffers have finished
        (void)hipStreamSynchronize(G->xfer);
        (void)hipStreamDestroy(G->xfer);
        G->xfer = nullptr;
    }
    if (G->upl) {
        (void)hipStreamSynchronize(G->upl);
        (void)hipStreamDestroy(G->upl);
        G->upl = nullptr;
    }
    for (hipEvent_t &e : G->win_dl)
        if (e) (void)hipEventDestroy(e);
    G->win_dl.clear();
    if (G->downloaded) (void)hipEventDestroy(G->downloaded);
    if (G->staged) (void)hipEventDestroy(G->staged);
    G->downloaded = G->staged = nullptr;
    dev_free(G->slot_block, s);
    G->slot_block = nullptr;
    for (int k = 0; k < 3; ++k) {
        G->slot_col[k] = nullptr;
        G->slot_bin[k] = nullptr;
        G->slot_win[k] = -1;
    }
    dev_free(G->xyz_s, s);
    dev_free(G->arena_pts, s);
    dev_free(G->arena_csr, s);
    G->arena_pts = G->arena_csr = nullptr;
    G->xyz_s = nullptr;
    G->key_s = nullptr;
    G->perm = G->cell_start = G->col = G->deg = G->hubs = nullptr;
    G->row_ptr = G->work = G->d_edges = nullptr;
    G->slot_off = nullptr;
    G->bin = nullptr;
    if (G->h_col || G->h_bin) {
        (void)hipStreamSynchronize(s);  // copies into the pinned CSR have finished
        host_free_pinned(G->h_col);
        host_free_pinned(G->h_bin);
        G->h_col = nullptr;
        G->h_bin = nullptr;
    }
}

// Restores the caller's current device on scope exit.
struct DeviceGuard {
    int prev = -1;
    int rc = GTC_OK;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) {
            rc = GTC_E_HIP;
            set_error("hipGetDevice failed (no usable GPU?)");
            prev = -1;
            return;
        }
        if (dev >= 0 && dev != prev && hipSetDevice(dev) != hipSuccess) {
            rc = GTC_E_HIP;
            set_error("hipSetDevice(%d) failed", dev);
        }
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

static void fill_graph_stats(const gtc_graph_s *G, gtc_stats *st) {
    st->n = G->n;
    st->edges = G->E;
    st->max_out_degree = G->max_deg;
    st->windows = G->win.empty() ? 1 : (int64_t)G->win.size() - 1;
    st->csr_mode = G->rebuild ? GTC_CSR_REBUILD : (G->host_csr ? GTC_CSR_HOST : GTC_CSR_DEVICE);
    st->spoke_elements = G->spoke_elements;
    st->build_ms = G->build_ms;
}

}  // namespace gtc

// Scratch of the allocation-free count: one array per GPU, held until the process ends.  Host
// code never uses the array's name as an address (in host code it names a host-side stand-in);
// its device address comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[GTC_NOALLOC_SCRATCH_BYTES];

namespace gtc {
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static unsigned char *g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (dev must be current).
static int noalloc_scratch(int dev, unsigned char **out) {
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("device %d: the allocation-free count supports devices 0..%d", dev,
                  kMaxDevices - 1);
        return GTC_E_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)", __FILE__, __LINE__);
        g_scratch_ptr[dev] = static_cast<unsigned char *>(p);
    }
    *out = g_scratch_ptr[dev];
    return GTC_OK;
}
}  // namespace gtc

using namespace gtc;

extern "C" {

int64_t gtc_num_configs(int32_t order, int32_t nbins) {
    if (order == 3 && nbins >= 1 && nbins <= GTC_MAX_BINS) return binom(nbins + 2, 3);
    if (order == 4 && nbins >= 1 && nbins <= GTC_MAX_BINS_4PCF) return binom(nbins + 5, 6);
    return -1;
}

int gtc_config_bins(int32_t order, int32_t nbins, int32_t *h_bins) {
    const int64_t ncfg = gtc_num_configs(order, nbins);
    if (ncfg < 0 || !h_bins) {
        set_error("gtc_config_bins: order must be 3 or 4 with nbins in range, h_bins non-NULL");
        return GTC_E_INVALID;
    }
    const int k = order == 3 ? 3 : 6;
    int v[6] = {0, 0, 0, 0, 0, 0};
    for (int64_t c = 0; c < ncfg; ++c) {
        for (int t = 0; t < k; ++t) h_bins[c * k + t] = v[t];
        // next nondecreasing tuple in lexicographic order
        int t = k - 1;
        while (t >= 0 && v[t] == nbins - 1) --t;
        if (t < 0) break;
        ++v[t];
        for (int u = t + 1; u < k; ++u) v[u] = v[t];
    }
    return GTC_OK;
}

int gtc_build_graph(const int32_t *d_xyz, int64_t n, const int64_t *h_edges_sq, int32_t nbins,
                    const gtc_options *opt, void *hip_stream, gtc_graph *out) {
    if (!out) {
        set_error("gtc_build_graph: out is NULL");
        return GTC_E_INVALID;
    }
    *out = nullptr;
    if (n < 0 || n >= ((int64_t)1 << 31)) {
        set_error("gtc_build_graph: n = %lld outside [0, 2^31)", (long long)n);
        return GTC_E_INVALID;
    }
    if (n > 0 && !d_xyz) {
        set_error("gtc_build_graph: d_xyz is NULL");
        return GTC_E_INVALID;
    }
    if (!h_edges_sq || nbins < 1 || nbins > GTC_MAX_BINS) {
        set_error("gtc_build_graph: need h_edges_sq and nbins in [1, %d]", GTC_MAX_BINS);
        return GTC_E_INVALID;
    }
    if (h_edges_sq[0] < 0) {
        set_error("gtc_build_graph: e_0 must be >= 0");
        return GTC_E_INVALID;
    }
    for (int b = 0; b < nbins; ++b)
        if (h_edges_sq[b + 1] <= h_edges_sq[b]) {
            set_error("gtc_build_graph: bin edges must increase strictly (e_%d >= e_%d)", b, b + 1);
            return GTC_E_INVALID;
        }
    const int64_t dmax = 3 * (int64_t)kGridSide * kGridSide + 1;
    if (h_edges_sq[nbins] > dmax) {
        set_error("gtc_build_graph: e_nbins beyond the largest squared distance on the grid");
        return GTC_E_INVALID;
    }
    gtc_options o{};
    if (opt) o = *opt;
    // GTC_TILE_BYTES=n sets the window budget of a build that gives none (§III.5.3)
    if (o.tile_bytes == 0)
        if (const char *env = std::getenv("GTC_TILE_BYTES")) {
            const long long v = std::atoll(env);
            if (v > 0) o.tile_bytes = v;
        }
    if (o.csr_mode < GTC_CSR_DEVICE || o.csr_mode > GTC_CSR_REBUILD) {
        set_error("gtc_build_graph: csr_mode %d is not one of 0 (device), 1 (host), 2 (rebuild)",
                  o.csr_mode);
        return GTC_E_INVALID;
    }
    if (o.tile_bytes < 0 || (o.csr_mode != GTC_CSR_DEVICE && o.tile_bytes <= 0)) {
        set_error("gtc_build_graph: tile_bytes must be >= 0, and > 0 for an out-of-core csr_mode");
        return GTC_E_INVALID;
    }
    if (o.csr_mode == GTC_CSR_REBUILD && o.drop_coords) {
        set_error("gtc_build_graph: csr_mode GTC_CSR_REBUILD re-emits windows from the coordinates, "
                  "which drop_coords would drop");
        return GTC_E_INVALID;
    }
    DeviceGuard dg(-1);
    if (dg.rc) return dg.rc;
    {
        // keep freed stream-ordered allocations cached in the pool instead of returning them to
        // the driver at every synchronisation (builds and counts allocate per call)
        int dev = 0;
        hipMemPool_t pool;
        if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
            uint64_t thr = UINT64_MAX;
            (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
        }
        (void)hipGetLastError();
    }

    auto t0 = std::chrono::steady_clock::now();
    gtc_graph_s *G = new (std::nothrow) gtc_graph_s();
    if (!G) {
        set_error("gtc_build_graph: host allocation failed");
        return GTC_E_OOM;
    }
    (void)hipGetDevice(&G->device);
    G->stream = reinterpret_cast<hipStream_t>(hip_stream);
    G->n = n;
    G->nb = nbins;
    if (o.allocator) {
        G->alloc = *o.allocator;
        G->has_alloc = true;
    }
    AllocScope alloc_scope(graph_allocator(G));
    G->tile_bytes = o.tile_bytes;
    G->auto_tiles = o.tile_bytes == 0;
    G->keep_coords_requested = !o.drop_coords;
    G->host_csr = o.csr_mode == GTC_CSR_HOST;
    G->rebuild = o.csr_mode == GTC_CSR_REBUILD;
    for (int b = 0; b <= nbins; ++b) G->edges[b] = h_edges_sq[b];
    int rc = build_graph_device(G, d_xyz, G->stream);
    if (rc == GTC_OK && o.drop_coords) {
        dev_free(G->xyz_s, G->stream);
        G->xyz_s = nullptr;
        G->coords_kept = false;
    }
    if (rc == GTC_OK) {
        hipError_t e = hipStreamSynchronize(G->stream);
        if (e != hipSuccess) rc = hip_fail(e, "hipStreamSynchronize", __FILE__, __LINE__);
    }
    if (rc != GTC_OK) {
        free_graph_buffers(G);
        (void)hipStreamSynchronize(G->stream);
        delete G;
        return rc;
    }
    G->build_ms =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    *out = G;
    return GTC_OK;
}

int gtc_count_3pcf(gtc_graph g, const double *d_w, uint64_t *d_counts, double *d_weighted,
                   gtc_stats *st, void *hip_stream) {
    if (!g || !d_counts || (d_w && !d_weighted)) {
        set_error("gtc_count_3pcf: need a graph, d_counts, and d_weighted when d_w is given");
        return GTC_E_INVALID;
    }
    DeviceGuard dg(g->device);
    AllocScope alloc_scope(graph_allocator(g));
    if (dg.rc) return dg.rc;
    auto t0 = std::chrono::steady_clock::now();
    gtc_stats local{};
    fill_graph_stats(g, &local);
    int rc = count_3pcf_device(g, d_w, d_counts, d_weighted, &local,
                               reinterpret_cast<hipStream_t>(hip_stream));
    local.count_ms =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    if (rc == GTC_OK && st) *st = local;
    return rc;
}

void gtc_release_host_cache(void) { release_pinned_cache(); }

int gtc_count_3pcf_noalloc(gtc_graph g, const double *d_w, uint64_t *d_counts,
                           double *d_weighted, void *hip_stream) {
    if (!g || !d_counts || (d_w && !d_weighted)) {
        set_error("gtc_count_3pcf_noalloc: need a graph, d_counts, and d_weighted when d_w is "
                  "given");
        return GTC_E_INVALID;
    }
    DeviceGuard dg(g->device);
    if (dg.rc) return dg.rc;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GTC_E_HIP;
    unsigned char *base = nullptr;
    GTC_TRY(noalloc_scratch(dev, &base));
    ExternalScratch ext;
    ext.base = base;
    ext.bytes = GTC_NOALLOC_SCRATCH_BYTES;
    return count_3pcf_device(g, d_w, d_counts, d_weighted, nullptr,
                             reinterpret_cast<hipStream_t>(hip_stream), nullptr, &ext);
}

int gtc_count_3pcf_hubs(gtc_graph g, const int32_t *h_hubs, int64_t n_hubs, const double *d_w,
                        uint64_t *d_counts, double *d_weighted, gtc_stats *st, void *hip_stream) {
    if (!g || !d_counts || (d_w && !d_weighted) || n_hubs < 0 || (n_hubs > 0 && !h_hubs)) {
        set_error("gtc_count_3pcf_hubs: need a graph, d_counts, h_hubs (n_hubs >= 0), and "
                  "d_weighted when d_w is given");
        return GTC_E_INVALID;
    }
    {
        std::vector<uint8_t> seen((size_t)std::max<int64_t>(g->n, 1), 0);
        for (int64_t t = 0; t < n_hubs; ++t) {
            const int32_t h = h_hubs[t];
            if (h < 0 || h >= g->n || seen[(size_t)h]) {
                set_error("gtc_count_3pcf_hubs: hub %lld (label %d) is out of range or repeated",
                          (long long)t, h);
                return GTC_E_INVALID;
            }
            seen[(size_t)h] = 1;
        }
    }
    if (g->win.size() != 2 || g->windowed()) {
        set_error("gtc_count_3pcf_hubs: needs a graph of one window (tile_bytes 0)");
        return GTC_E_UNSUPPORTED;
    }
    DeviceGuard dg(g->device);
    AllocScope alloc_scope(graph_allocator(g));
    if (dg.rc) return dg.rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
    auto t0 = std::chrono::steady_clock::now();
    int32_t *d_in = nullptr, *d_out = nullptr;
    unsigned long long *d_sums = nullptr;
    void *blk = nullptr;
    GTC_TRY(carve_alloc(&blk, s, [&](Carver &c) {
        c.take(&d_in, n_hubs);
        c.take(&d_out, n_hubs);
        c.take(&d_sums, 3);
    }));
    int rc = GTC_OK;
    if (n_hubs > 0) {
        hipError_t e = hipMemcpyAsync(d_in, h_hubs, sizeof(int32_t) * n_hubs,
                                      hipMemcpyHostToDevice, s);
        if (e != hipSuccess) rc = hip_fail(e, "hub list upload", __FILE__, __LINE__);
    }
    HubSubset sub;
    if (rc == GTC_OK) rc = filter_hubs(g, d_in, n_hubs, d_out, d_sums, &sub, s);
    gtc_stats local{};
    fill_graph_stats(g, &local);
    if (rc == GTC_OK) rc = count_3pcf_device(g, d_w, d_counts, d_weighted, &local, s, &sub);
    dev_free(blk, s);
    local.count_ms =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    if (rc == GTC_OK && st) *st = local;
    return rc;
}

static int count_4pcf(gtc_graph g, uint64_t *d_even, int64_t *d_odd, gtc_stats *st,
                      void *hip_stream, bool s4, const double *d_w = nullptr,
                      double *d_even_w = nullptr, double *d_odd_w = nullptr) {
    const char *fn = d_w ? "gtc_count_4pcf_weighted"
                         : (s4 ? "gtc_count_4pcf_parity_s4" : "gtc_count_4pcf_parity");
    if (!g || !d_even || !d_odd || (d_w && (!d_even_w || !d_odd_w))) {
        set_error("%s: need a graph, d_even and d_odd (and d_even_w, d_odd_w with weights)", fn);
        return GTC_E_INVALID;
    }
    if (g->nb > GTC_MAX_BINS_4PCF) {
        set_error("%s: nbins %d > %d", fn, g->nb, GTC_MAX_BINS_4PCF);
        return GTC_E_INVALID;
    }
    if (!g->coords_kept) {
        set_error("%s: the graph was built with drop_coords", fn);
        return GTC_E_INVALID;
    }
    DeviceGuard dg(g->device);
    AllocScope alloc_scope(graph_allocator(g));
    if (dg.rc) return dg.rc;
    auto t0 = std::chrono::steady_clock::now();
    gtc_stats local{};
    fill_graph_stats(g, &local);
    int rc = count_4pcf_device(g, d_even, d_odd, &local, reinterpret_cast<hipStream_t>(hip_stream),
                               s4, d_w, d_even_w, d_odd_w);
    local.count_ms =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    if (rc == GTC_OK && st) *st = local;
    return rc;
}

int gtc_count_4pcf_parity(gtc_graph g, uint64_t *d_even, int64_t *d_odd, gtc_stats *st,
                          void *hip_stream) {
    return count_4pcf(g, d_even, d_odd, st, hip_stream, false);
}

int gtc_count_4pcf_parity_s4(gtc_graph g, uint64_t *d_even, int64_t *d_odd, gtc_stats *st,
                             void *hip_stream) {
    return count_4pcf(g, d_even, d_odd, st, hip_stream, true);
}

int gtc_count_2pcf(gtc_graph g, const double *d_w, uint64_t *d_counts, double *d_weighted,
                   gtc_stats *st, void *hip_stream) {
    if (!g || !d_counts || (d_w && !d_weighted)) {
        set_error("gtc_count_2pcf: need a graph, d_counts, and d_weighted when d_w is given");
        return GTC_E_INVALID;
    }
    if (g->rebuild && !g->coords_kept) {
        set_error("gtc_count_2pcf: the graph's windows need the coordinates");
        return GTC_E_INVALID;
    }
    DeviceGuard dg(g->device);
    AllocScope alloc_scope(graph_allocator(g));
    if (dg.rc) return dg.rc;
    auto t0 = std::chrono::steady_clock::now();
    gtc_stats local{};
    fill_graph_stats(g, &local);
    int rc = count_2pcf_device(g, d_w, d_counts, d_weighted, &local,
                               reinterpret_cast<hipStream_t>(hip_stream));
    local.count_ms =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    if (rc == GTC_OK && st) *st = local;
    return rc;
}

int gtc_disconnected_4pcf_s4(int32_t nbins, const double *h_xi, double *h_disc) {
    if (nbins < 1 || nbins > GTC_MAX_BINS_4PCF || !h_xi || !h_disc) {
        set_error("gtc_disconnected_4pcf_s4: nbins in [1, %d], h_xi and h_disc non-NULL",
                  GTC_MAX_BINS_4PCF);
        return GTC_E_INVALID;
    }
    disconnected_4pcf_s4(nbins, h_xi, h_disc);
    return GTC_OK;
}

int gtc_connected_4pcf_s4(int32_t nbins, const double *h_zeta, const double *h_xi,
                          double *h_conn) {
    if (!h_zeta) {
        set_error("gtc_connected_4pcf_s4: h_zeta is NULL");
        return GTC_E_INVALID;
    }
    GTC_TRY(gtc_disconnected_4pcf_s4(nbins, h_xi, h_conn));
    for (int64_t c = 0; c < num_configs_s4(nbins); ++c) h_conn[c] = h_zeta[c] - h_conn[c];
    return GTC_OK;
}

int gtc_count_4pcf_weighted(gtc_graph g, const double *d_w, int32_t s4, uint64_t *d_even,
                            int64_t *d_odd, double *d_even_w, double *d_odd_w, gtc_stats *st,
                            void *hip_stream) {
    if (!d_w) {
        set_error("gtc_count_4pcf_weighted: d_w is NULL");
        return GTC_E_INVALID;
    }
    return count_4pcf(g, d_even, d_odd, st, hip_stream, s4 != 0, d_w, d_even_w, d_odd_w);
}

int64_t gtc_num_configs_s4(int32_t nbins) {
    if (nbins < 1 || nbins > GTC_MAX_BINS_4PCF) return -1;
    return num_configs_s4(nbins);
}

int gtc_config_bins_s4(int32_t nbins, int32_t *h_bins) {
    if (nbins < 1 || nbins > GTC_MAX_BINS_4PCF || !h_bins) {
        set_error("gtc_config_bins_s4: nbins in [1, %d] and h_bins non-NULL", GTC_MAX_BINS_4PCF);
        return GTC_E_INVALID;
    }
    config_bins_s4(nbins, h_bins);
    return GTC_OK;
}

int gtc_equilateral_configs(int32_t order, int32_t s4, int32_t nbins, int64_t *h_ranks) {
    const bool ok3 = order == 3 && !s4 && nbins >= 1 && nbins <= GTC_MAX_BINS;
    const bool ok4 = order == 4 && nbins >= 1 && nbins <= GTC_MAX_BINS_4PCF;
    if (!(ok3 || ok4) || !h_ranks) {
        set_error("gtc_equilateral_configs: order 3 (nbins <= %d, s4 = 0) or 4 (nbins <= %d), "
                  "h_ranks non-NULL", GTC_MAX_BINS, GTC_MAX_BINS_4PCF);
        return GTC_E_INVALID;
    }
    if (order == 4 && s4) {  // (b, b, b, b, b, b) is its own canonical tuple; find its rank
        std::vector<int32_t> t(6 * (size_t)num_configs_s4(nbins));
        config_bins_s4(nbins, t.data());
        const int64_t n = (int64_t)t.size() / 6;
        for (int b = 0, c = 0; b < nbins; ++b) {
            while (c < n && !(t[6 * c] == b && t[6 * c + 5] == b)) ++c;
            h_ranks[b] = c;
        }
        return GTC_OK;
    }
    // nondecreasing k-tuples lexicographically below (b, ..., b): those whose first element
    // x < b, multichoose(nbins - x, k - 1) = C(nbins - x + k - 2, k - 1) of them for each x
    const int k = order == 3 ? 3 : 6;
    auto binom = [](int64_t n, int r) {
        int64_t c = 1;
        for (int u = 1; u <= r; ++u) c = c * (n - r + u) / u;
        return c;
    };
    int64_t rank = 0;
    for (int b = 0; b < nbins; ++b) {
        h_ranks[b] = rank;
        rank += binom(nbins - b + k - 2, k - 1);
    }
    return GTC_OK;
}

int gtc_config_realizable_s4(int32_t nbins, const int64_t *h_edges_sq, uint8_t *h_mask) {
    if (nbins < 1 || nbins > GTC_MAX_BINS_4PCF || !h_edges_sq || !h_mask) {
        set_error("gtc_config_realizable_s4: nbins in [1, %d], h_edges_sq and h_mask non-NULL",
                  GTC_MAX_BINS_4PCF);
        return GTC_E_INVALID;
    }
    for (int b = 0; b < nbins; ++b)
        if (h_edges_sq[0] < 0 || h_edges_sq[b + 1] <= h_edges_sq[b]) {
            set_error("gtc_config_realizable_s4: bin edges must be >= 0 and increase strictly");
            return GTC_E_INVALID;
        }
    config_realizable_s4(nbins, h_edges_sq, h_mask);
    return GTC_OK;
}

int gtc_graph_export(gtc_graph g, int64_t *h_row_ptr, int32_t *h_col, uint8_t *h_bin,
                     int32_t *h_perm) {
    if (!g) {
        set_error("gtc_graph_export: graph is NULL");
        return GTC_E_INVALID;
    }
    DeviceGuard dg(g->device);
    AllocScope alloc_scope(graph_allocator(g));
    if (dg.rc) return dg.rc;
    hipStream_t s = g->stream;
    if (h_row_ptr)
        GTC_HIP_CHECK(hipMemcpyAsync(h_row_ptr, g->row_ptr, sizeof(int64_t) * (g->n + 1),
                                     hipMemcpyDeviceToHost, s));
    // packed entries come out through the label array (or a host buffer) and are split below
    std::vector<int32_t> words;
    int32_t *w_dst = h_col;
    if (g->packed && h_bin && !h_col && g->E) {
        words.resize(g->E);
        w_dst = words.data();
    }
    if (g->host_csr) {  // out-of-core graph: the CSR is already in host memory
        if (g->downloaded) GTC_HIP_CHECK(hipEventSynchronize(g->downloaded));
        if (w_dst && g->E) std::memcpy(w_dst, g->h_col, sizeof(int32_t) * g->E);
        if (!g->packed && h_bin && g->E) std::memcpy(h_bin, g->h_bin, g->E);
    } else if (g->rebuild) {  // no stored CSR: emit each window again and copy it out
        if ((w_dst || (!g->packed && h_bin)) && g->E) {
            int32_t *wc = nullptr;
            uint8_t *wb = nullptr;
            void *blk = nullptr;
            GTC_TRY(carve_alloc(&blk, s, [&](Carver &c) {
                c.take(&wc, g->max_window_edges);
                if (!g->packed) c.take(&wb, g->max_window_edges);
            }));
            int rc = GTC_OK;
            for (int64_t w = 0; w + 1 < (int64_t)g->win.size() && rc == GTC_OK; ++w) {
                const int64_t e0 = g->win_e[w];
                const int64_t ne = g->win_e[w + 1] - e0;
                if (ne <= 0) continue;
                rc = emit_window(g, w, wc, wb, s);
                hipError_t e = hipSuccess;
                if (rc == GTC_OK && w_dst)
                    e = hipMemcpyAsync(w_dst + e0, wc, sizeof(int32_t) * ne, hipMemcpyDeviceToHost, s);
                if (rc == GTC_OK && e == hipSuccess && !g->packed && h_bin)
                    e = hipMemcpyAsync(h_bin + e0, wb, ne, hipMemcpyDeviceToHost, s);
                if (rc == GTC_OK && e == hipSuccess) e = hipStreamSynchronize(s);
                if (e != hipSuccess) rc = hip_fail(e, "window export", __FILE__, __LINE__);
            }
            dev_free(blk, s);
            if (rc) return rc;
        }
    } else {
        if (w_dst && g->E)
            GTC_HIP_CHECK(hipMemcpyAsync(w_dst, g->col, sizeof(int32_t) * g->E, hipMemcpyDeviceToHost, s));
        if (!g->packed && h_bin && g->E)
            GTC_HIP_CHECK(hipMemcpyAsync(h_bin, g->bin, g->E, hipMemcpyDeviceToHost, s));
    }
    if (h_perm && g->n)
        GTC_HIP_CHECK(hipMemcpyAsync(h_perm, g->perm, sizeof(int32_t) * g->n, hipMemcpyDeviceToHost, s));
    GTC_HIP_CHECK(hipStreamSynchronize(s));
    if (g->packed && w_dst)
        for (int64_t e = 0; e < g->E; ++e) {
            const uint32_t w = (uint32_t)w_dst[e];
            if (h_bin) h_bin[e] = (uint8_t)(w >> 24);
            if (h_col) h_col[e] = (int32_t)(w & kLabelMask);
        }
    return GTC_OK;
}

int gtc_graph_stats(gtc_graph g, gtc_stats *st) {
    if (!g || !st) {
        set_error("gtc_graph_stats: need a graph and st");
        return GTC_E_INVALID;
    }
    *st = gtc_stats{};
    fill_graph_stats(g, st);
    return GTC_OK;
}

void gtc_graph_free(gtc_graph g) {
    if (!g) return;
    DeviceGuard dg(g->device);
    AllocScope alloc_scope(graph_allocator(g));
    free_graph_buffers(g);
    (void)hipStreamSynchronize(g->stream);
    delete g;
}

int64_t gtc_plan_windows(const int64_t *h_row_ptr, int64_t n, int64_t tile_bytes,
                         int32_t entry_bytes, int64_t *h_bounds) {
    if (!h_row_ptr || !h_bounds || n < 0 || tile_bytes <= 0 || entry_bytes <= 0) {
        set_error("gtc_plan_windows: need row offsets, a bounds array, n >= 0, tile_bytes > 0 "
                  "and entry_bytes > 0");
        return GTC_E_INVALID;
    }
    for (int64_t i = 0; i < n; ++i)
        if (h_row_ptr[i + 1] < h_row_ptr[i]) {
            set_error("gtc_plan_windows: row offsets decrease at row %lld", (long long)i);
            return GTC_E_INVALID;
        }
    return plan_windows(h_row_ptr, n, tile_bytes, entry_bytes, h_bounds);
}

int64_t gtc_graph_windows(gtc_graph g, int64_t *h_bounds, int64_t *h_offsets, int64_t capacity) {
    if (!g) {
        set_error("gtc_graph_windows: null graph");
        return GTC_E_INVALID;
    }
    const int64_t W = (int64_t)g->win.size() - 1;
    if (capacity < 0 || (capacity > 0 && !h_bounds && !h_offsets)) {
        set_error("gtc_graph_windows: need capacity >= 0 and an output array when it is > 0");
        return GTC_E_INVALID;
    }
    if (capacity >= W + 1) {
        for (int64_t k = 0; k <= W; ++k) {
            if (h_bounds) h_bounds[k] = g->win[k];
            if (h_offsets) h_offsets[k] = g->win_e[k];
        }
    }
    return W;
}

const char *gtc_status_string(int status) {
    switch (status) {
        case GTC_OK: return "ok";
        case GTC_E_INVALID: return "invalid argument";
        case GTC_E_OOM: return "out of memory";
        case GTC_E_HIP: return "HIP runtime error";
        case GTC_E_OVERFLOW: return "count overflow";
        case GTC_E_UNSUPPORTED: return "unsupported";
        default: return "unknown status";
    }
}

const char *gtc_last_error(void) { return gtc::last_error(); }

}  // extern "C"

// gtc_internal.h - declarations shared by the libgtc translation units (host and device).
//
// Data layout in device memory (internal labels = cell-sorted order):
//   xyz_s      int4 [n]      (x, y, z, cell key) of each point, cell-sorted
//   key_s      int32 [n]     cell key of each point
//   perm       int32 [n]     internal -> original label
//   cell_start int32 [ncell+1] first internal label of each cell (cells in key order)
//   row_ptr    int64 [n+1]   forward CSR offsets (64-bit: edge counts pass 2^31, §III.5.1)
//   col        int32 [E]     forward neighbours j > i, ascending per row (Eq.(1)); in a packed
//                            graph (n <= 2^24) each word also holds the edge's bin in its top byte
//   bin        uint8 [E]     radial bin of each edge (§II.1); absent (null) in a packed graph
//   deg        int32 [n]     forward degree d+(i)
//   work       int64 [n]     sum of d+(j) over the row of i (spoke elements of hub i)
//   slot_off   u32 [n][16]   where each of the 14 forward cell slots of row i starts (own cell,
//                            then the 13 forward cells in key order); [14] is the row length
//   hubs       int32 [n_hubs] hubs with at least one possible triangle, heaviest first
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <vector>

#include "gtc.h"

namespace gtc {

constexpr int kGridSide = 1 << GTC_GRID_BITS;
constexpr int kWave = 64;

// ------------------------------------------------------------------ errors (host)
void set_error(const char *fmt, ...);
int hip_fail(hipError_t e, const char *what, const char *file, int line);

#define GTC_HIP_CHECK(call)                                                     \
    do {                                                                        \
        hipError_t gtc_e_ = (call);                                             \
        if (gtc_e_ != hipSuccess) return gtc::hip_fail(gtc_e_, #call, __FILE__, __LINE__); \
    } while (0)

#define GTC_TRY(expr)                   \
    do {                                \
        int gtc_rc_ = (expr);           \
        if (gtc_rc_ != GTC_OK) return gtc_rc_; \
    } while (0)

// ------------------------------------------------------------------ device memory (host)
// Stream-ordered allocations: from the caller's gtc_allocator of the current API call (see
// AllocScope), else from the device's default pool (kept cached between calls).
int dev_alloc(void **p, size_t bytes, hipStream_t s);
void dev_free(void *p, hipStream_t s);
// pinned host memory, through the same routines
int host_alloc_pinned(void **p, size_t bytes);
void host_free_pinned(void *p);
// free the pinned block kept for reuse (runtime route), if any
void release_pinned_cache();
// The allocator of the API call running on this thread (null: the HIP runtime's).  Every entry
// point that allocates opens a scope with the allocator its graph or options carry.
const gtc_allocator *current_allocator();
struct AllocScope {
    const gtc_allocator *prev;
    explicit AllocScope(const gtc_allocator *a);
    ~AllocScope();
};
template <class T>
int dev_alloc_n(T **p, size_t count, hipStream_t s) {
    return dev_alloc(reinterpret_cast<void **>(p), sizeof(T) * (count ? count : 1), s);
}
// Several arrays in one device allocation.  A pass with no base only sizes the block; a pass over
// the allocated base hands the arrays out, each 256-byte aligned.  One allocation and one free
// per group of arrays: the stream-ordered pool's per-call cost (up to ~2 ms for some frees) is
// paid once per group instead of once per array.
struct Carver {
    unsigned char *base = nullptr;
    size_t off = 0;
    template <class T>
    void take(T **p, size_t count) {
        if (base) *p = reinterpret_cast<T *>(base + off);
        off += (sizeof(T) * (count ? count : 1) + 255) & ~(size_t)255;
    }
};

// Allocate the arrays that layout(Carver &) takes, as one block (*block, freed with dev_free).
template <class F>
int carve_alloc(void **block, hipStream_t s, F &&layout) {
    Carver size_pass;
    layout(size_pass);
    GTC_TRY(dev_alloc(block, size_pass.off, s));
    Carver give;
    give.base = static_cast<unsigned char *>(*block);
    layout(give);
    return GTC_OK;
}

int fill_u64(uint64_t *p, int64_t count, uint64_t value, hipStream_t s);
int fill_u32(uint32_t *p, int64_t count, uint32_t value, hipStream_t s);

// Exact fixed-point sums to doubles, on the device: for c < n, out[c] = 2^-s (sum of the q of
// configuration c), where every added q was split as q = (hi - 2^29) 2^28 + lo, the lo and hi
// limbs summed as 128-bit words [lo128, hi128] at limbs[4c .. 4c+3] of each of `copies` copies
// (copy_stride words apart), and counts[c] terms were added.  One rounding per sum.
int finalize_limbs(const unsigned long long *limbs, int64_t n, int copies, int64_t copy_stride,
                   const unsigned long long *counts, int s, double *out, hipStream_t st);
// The parity 4pCF's sums by handedness class: [n][3] two's complement 128-bit words (low, high)
// A+, A-, A0 per copy; even[c] = 2^-s (A+ + A- + A0), odd[c] = 2^-s (A+ - A-), one rounding each.
int finalize_class_sums(const unsigned long long *w, int64_t n, int copies, int64_t copy_stride,
                        int s, double *even, double *odd, hipStream_t st);

// Scale exponent of the exact weighted sums of products of `factors` weights: s = 57 - e with
// M = fl(...fl(fl(a*a)*a)...*a) (`factors` copies of a = max |w|) = f 2^e, f in [0.5, 1), so that
// |p 2^s| < 2^57 for every product p (s = 0 when M == 0).  GTC_E_UNSUPPORTED when M overflows
// (the products have no finite scale) or 2^s is beyond the largest double (max |w| so small that
// the products' scale would exceed 2^1023); *scale is left 0 then.
int weight_scale(double maxabs, int factors, int *scale);

// hub windows: bounds[0..W] of consecutive rows whose CSR (entry_bytes per edge) fits tile_bytes
int64_t plan_windows(const int64_t *row_ptr, int64_t n, int64_t tile_bytes, int64_t entry_bytes,
                     int64_t *bounds);

// exclusive scan of n int32 values: out[0..n], out[n] = total.  ws: scan_workspace_bytes(n) bytes
// of device scratch (partial sums of the tiles).
size_t scan_workspace_bytes(int64_t n);
int exclusive_scan_i32_to_i64(const int32_t *in, int64_t *out, int64_t n, void *ws, hipStream_t s);
int exclusive_scan_i32_to_i32(const int32_t *in, int32_t *out, int64_t n, void *ws, hipStream_t s);

// ------------------------------------------------------------------ CSR entries
// A packed CSR keeps each entry in one 32-bit word: the neighbour label in the low 24 bits, the
// bin in the high 8.  It needs labels below 2^24 and moves 4 bytes per entry where a label array
// plus a bin array move 5.
constexpr int64_t kPackedMaxN = (int64_t)1 << 24;
constexpr uint32_t kLabelMask = 0xffffffu;

__host__ __device__ inline uint32_t pack_entry(int32_t j, int32_t b) {
    return (uint32_t)j | ((uint32_t)b << 24);
}

// entry e of a CSR (col, bin): its neighbour label and bin
template <bool PK>
__device__ __forceinline__ void csr_entry(const int32_t *col, const uint8_t *bin, int64_t e,
                                          int32_t &k, int32_t &b) {
    const int32_t w = col[e];
    if (PK) {
        k = (int32_t)((uint32_t)w & kLabelMask);
        b = (int32_t)((uint32_t)w >> 24);
    } else {
        k = w;
        b = bin[e];
    }
}

// ------------------------------------------------------------------ cell grid
struct Grid {
    int32_t g;       // cells per axis
    int32_t cs;      // integer cell side (>= r_max)
    int64_t ncell;   // g^3
};

// The hub-map domain of hub i: the id ranges of the key runs that hold its forward stencil.
// Cell keys are (cz*g + cy)*g + cx, so the 13 forward neighbour cells of cell c lie in five key
// runs: [c, c+2), [c+g-1, c+g+2), [c+g^2-g-1, c+g^2-g+2), [c+g^2-1, c+g^2+2),
// [c+g^2+g-1, c+g^2+g+2).  Their points form five label ranges; the first starts at i+1.
struct HubDomain {
    int32_t lo[5];
    int32_t hi[5];
    int32_t delta[5];  // map offset of label k in run t: k + delta[t]
    int32_t size;      // total labels covered
};

__device__ __forceinline__ void hub_domain(int32_t i, int32_t c, const Grid &gr,
                                           const int32_t *__restrict__ cell_start, HubDomain &d) {
    const int64_t g = gr.g, gg = g * g, nc = gr.ncell;
    int64_t klo[5], khi[5];
    if (g >= 3) {
        const int64_t off_lo[5] = {0, g - 1, gg - g - 1, gg - 1, gg + g - 1};
        for (int t = 0; t < 5; ++t) {
            klo[t] = c + off_lo[t];
            khi[t] = klo[t] + (t == 0 ? 2 : 3);
        }
    } else {
        klo[0] = c;
        khi[0] = c + gg + g + 2;
        for (int t = 1; t < 5; ++t) klo[t] = khi[t] = khi[0];
    }
    int32_t base = 0;
    for (int t = 0; t < 5; ++t) {
        const int64_t a = klo[t] < nc ? klo[t] : nc, b = khi[t] < nc ? khi[t] : nc;
        int32_t lo = cell_start[a], hi = cell_start[b];
        if (t == 0) lo = i + 1;
        if (hi < lo) hi = lo;
        d.lo[t] = lo;
        d.hi[t] = hi;
        d.delta[t] = base - lo;
        base += hi - lo;
    }
    d.size = base;
}

// ------------------------------------------------------------------ hub queue
// Hub lists are ordered heaviest first by class: class c holds the hubs whose spoke-element work w
// has floor(log2 w) = 63 - c.  Enumeration waves take hubs from one counter per class, in class
// order, a batch at a time: one hub per take in the classes of 2^15 elements and more, up to 64
// hubs per take in the light classes.  A single shared counter taken once per hub serialises in
// the L2 atomic unit at about one take per 10 ns, which alone costs ~10 ms per million hubs.
constexpr int kHubClasses = 64;
constexpr int kQueueStride = 64;  // u32 words between class counters (a 256-byte line each)
// Each class's hub range is split into kQueueParts parts, one per XCD: workgroup b takes hubs from
// part b % kQueueParts first (its XCD's L2 then serves one neighbourhood of the cell order), and
// from the other parts once its own is drained.
constexpr int kQueueParts = 8;
constexpr int64_t kQueueWords = (int64_t)kHubClasses * kQueueParts * kQueueStride;
constexpr int kBatchWorkLog2 = 15;

__device__ __forceinline__ int hub_class(int64_t m, int64_t w) {
    if (m < 2 || w <= 0) return -1;
    return kHubClasses - 1 - (63 - __clzll((unsigned long long)w));
}

__host__ __device__ inline uint32_t class_batch(int c, uint32_t cap) {
    const int e = 63 - c;  // the class's work is at least 2^e
    if (e >= kBatchWorkLog2) return 1u;
    const int b = kBatchWorkLog2 - e;
    const uint32_t v = 1u << (b < 6 ? b : 6);
    return v < cap ? v : cap;
}

// Largest batch that still leaves every wave of the launch about 16 takes: a power of two in
// [1, 64], so that the last batches do not leave a few waves working long after the rest.
inline uint32_t batch_cap(int64_t n_hubs, int64_t total_waves) {
    const int64_t per = total_waves > 0 ? n_hubs / (total_waves * 16) : 1;
    uint32_t cap = 1;
    while (cap < 64 && (int64_t)(cap * 2) <= per) cap *= 2;
    return cap;
}

// counts[c] = hubs of class c in hubs[0, n_hubs) (counts zeroed here)
int hub_class_counts(const int32_t *hubs, int64_t n_hubs, const int64_t *row_ptr,
                     const int64_t *work, uint32_t *counts, hipStream_t s);

// Per-wave view of the class queue.  Every lane holds the hub-list range of class `lane`.
struct HubQueue {
    uint32_t cbeg, cend;  // lane c: queue entries [cbeg, cend) of class c
    uint32_t hbeg;        // lane c: hub-list position of class c's first hub
    uint32_t pos, end;    // current batch (wave-uniform)
    int cls;              // current class (wave-uniform)
    int tried;            // parts of the current class drained so far (wave-uniform)
    int home;             // first part to take from
    uint32_t cap;         // batch cap of this launch

    // (mult: queue entries per hub of class `lane`)
    __device__ __forceinline__ void init(const uint32_t *counts, uint32_t batch_cap, int lane,
                                         int home_part, uint32_t mult = 1) {
        const uint32_t h = counts[lane], c = h * mult;
        uint32_t incl = c, hincl = h;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const uint32_t o = __shfl_up(incl, d, kWave), ho = __shfl_up(hincl, d, kWave);
            if (lane >= d) {
                incl += o;
                hincl += ho;
            }
        }
        cbeg = incl - c;
        cend = incl;
        hbeg = hincl - h;
        pos = end = 0;
        cls = 0;
        tried = 0;
        home = home_part;
        cap = batch_cap;
    }

    // Next hub-list position for this wave; false once every class is drained.
    __device__ __forceinline__ bool next(uint32_t *counters, int lane, uint32_t &hq) {
        while (pos >= end) {
            if (cls >= kHubClasses) return false;
            const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)cbeg, cls);
            const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)cend, cls);
            if (b < e && tried < kQueueParts) {
                const int p = (home + tried) % kQueueParts;
                const uint64_t len = e - b;
                const uint32_t pb = b + (uint32_t)(len * p / kQueueParts);
                const uint32_t pe = b + (uint32_t)(len * (p + 1) / kQueueParts);
                if (pb < pe) {
                    const uint32_t batch = class_batch(cls, cap);
                    uint32_t t = 0;
                    if (lane == 0) t = atomicAdd(&counters[(cls * kQueueParts + p) * kQueueStride], batch);
                    t = (uint32_t)__builtin_amdgcn_readfirstlane((int)__shfl(t, 0, kWave));
                    if (t < pe - pb) {
                        pos = pb + t;
                        end = pe - pos < batch ? pe : pos + batch;
                        break;
                    }
                }
                ++tried;
                continue;
            }
            ++cls;
            tried = 0;
        }
        hq = pos++;
        return true;
    }

    // Hub-list position of entry hq of the current class, one entry per hub (init's mult 1).
    __device__ __forceinline__ uint32_t hub_pos(uint32_t hq) const {
        const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)cbeg, cls);
        return (uint32_t)__builtin_amdgcn_readlane((int)hbeg, cls) + (hq - b);
    }

    // Entry hq of the current class when each of its hubs has `parts` entries (init's mult for
    // the class), taken group by group: the entries of a group of g hubs are its hubs' part 0,
    // then their part 1, and so on.  The hub's hub-list position and the part (wave-uniform).
    __device__ __forceinline__ void split(uint32_t hq, uint32_t parts, uint32_t g, uint32_t &hpos,
                                          uint32_t &part) const {
        const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)cbeg, cls);
        const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)cend, cls);
        const uint32_t hb = (uint32_t)__builtin_amdgcn_readlane((int)hbeg, cls);
        const uint32_t nh = (e - b) / parts, t = hq - b;
        const uint32_t grp = t / (parts * g), r = t - grp * parts * g;
        const uint32_t gsz = nh - grp * g < g ? nh - grp * g : g;
        part = r / gsz;
        hpos = hb + grp * g + (r - part * gsz);
    }
};

// ------------------------------------------------------------------ configuration ranks
// Rank of a nondecreasing triple (x <= y <= z) among all nondecreasing triples over [0, nb) in
// lexicographic order:  rank = F(x) + P(y) - P(x) + (z - y), where F(x) = sum_{t<x} C(nb-t+1, 2)
// counts the triples whose first element is below x and P(y) = sum_{u<y} (nb - u) counts, for a
// fixed first element, the pairs whose middle element is below y.  With A[x] = F(x) - P(x) and
// B[y] = P(y) - y the rank is A[x] + B[y] + z.
__host__ __device__ inline void rank3_tables(int nb, int32_t *A, int32_t *B) {
    int32_t first = 0;  // triples whose first element is < x
    int32_t pairs_before = 0;  // sum_{u<x} (nb - u)
    for (int x = 0; x < nb; ++x) {
        A[x] = first - pairs_before;  // rank = first + (pairs_before(y) - pairs_before(x)) + z - y
        first += (nb - x) * (nb - x + 1) / 2;
        pairs_before += nb - x;
    }
    int32_t pb = 0;
    for (int y = 0; y < nb; ++y) {
        B[y] = pb - y;
        pb += nb - y;
    }
}

}  // namespace gtc

// The graph handle.
struct gtc_graph_s {
    int device = 0;
    hipStream_t stream = nullptr;  // stream of the build (frees are ordered on it)
    int64_t n = 0;
    int32_t nb = 0;
    int64_t edges[GTC_MAX_BINS + 1] = {};
    gtc::Grid grid{};
    // device arrays: xyz_s in a block of its own (dropped on request after the build), the other
    // per-point arrays in arena_pts, the CSR (col, bin) in arena_csr
    void *arena_pts = nullptr;
    void *arena_csr = nullptr;
    int4 *xyz_s = nullptr;     // (x, y, z, cell key)
    int32_t *key_s = nullptr;  // cell key of each point (kept)
    int32_t *perm = nullptr;
    int32_t *cell_start = nullptr;
    int64_t *row_ptr = nullptr;
    bool packed = false;       // col holds packed entries and bin is null (labels below 2^24)
    int32_t *col = nullptr;
    uint8_t *bin = nullptr;
    int32_t *deg = nullptr;
    int64_t *work = nullptr;
    uint32_t *slot_off = nullptr;  // [n][16]: start of each forward cell slot in the row, [14] = end
    int32_t *hubs = nullptr;
    int64_t *d_edges = nullptr;  // device copy of the bin edges
    // scalars
    int64_t E = 0;
    int64_t n_hubs = 0;
    int64_t max_deg = 0;
    int64_t max_domain = 0;
    int64_t max_band = 0;        // longest label range of one key run of a hub domain
    int64_t spoke_elements = 0;  // sum of work over all hubs
    int64_t walks = 0;           // sum of d+(i) over hubs in the hub list
    bool coords_kept = true;
    double build_ms = 0.0;
    // hub windows (§III.5.3): label bounds win[0..W], one window [0, n) unless tiled
    int64_t tile_bytes = 0;
    bool auto_tiles = false;  // no budget given: go out of core if the CSR exceeds free memory
    bool keep_coords_requested = true;
    std::vector<int64_t> win;       // W+1 label bounds
    std::vector<int64_t> win_hubs;  // W+1 offsets into hubs: window k's hubs, heaviest first
    std::vector<int32_t> win_smax;  // last window holding a spoke of window k's hubs
    std::vector<int64_t> win_e;     // W+1 CSR offsets of the bounds: row_ptr[win[k]]
    int64_t max_window_edges = 0;
    // out-of-core: the CSR in pinned host memory, only windows go to the device
    bool host_csr = false;   // the CSR in pinned host memory (h_col, h_bin)
    bool rebuild = false;    // no stored CSR: windows are emitted again when a tile needs them
    bool windowed() const { return host_csr || rebuild; }
    // the caller's memory routines (gtc_options.allocator), if any: every buffer of the graph, and
    // the scratch of every call on it, comes from them
    gtc_allocator alloc{};
    bool has_alloc = false;
    int32_t *h_col = nullptr;
    uint8_t *h_bin = nullptr;
    // Out-of-core transfers and window buffers.  The build downloads the windows of a pinned CSR
    // on `xfer` and returns without waiting; `downloaded` follows the last download, and every
    // reader of h_col / h_bin waits for it (wait_host_csr).  The three window buffers serve the
    // build as staging and the 3pCF count as its tile windows; slot_win[k] is the window buffer k
    // holds (-1: none), valid once `staged` (on the build stream) has completed, so a count
    // starts with the windows the build left on the device.
    hipStream_t xfer = nullptr;
    hipEvent_t downloaded = nullptr;
    // A count's window uploads run on `upl`, each after its window's download and after the
    // download out of the buffer it overwrites (win_dl[w], recorded on xfer), not behind every
    // download of the build.
    hipStream_t upl = nullptr;
    std::vector<hipEvent_t> win_dl;
    hipEvent_t staged = nullptr;
    void *slot_block = nullptr;
    int32_t *slot_col[3] = {nullptr, nullptr, nullptr};
    uint8_t *slot_bin[3] = {nullptr, nullptr, nullptr};
    int64_t slot_win[3] = {-1, -1, -1};
};

namespace gtc {
inline const gtc_allocator *graph_allocator(const gtc_graph_s *G) {
    return G->has_alloc ? &G->alloc : nullptr;
}

// Make stream s wait for the build's downloads into the pinned host CSR (no-op without one).
inline int wait_host_csr(const gtc_graph_s *G, hipStream_t s) {
    if (G->downloaded) GTC_HIP_CHECK(hipStreamWaitEvent(s, G->downloaded, 0));
    return GTC_OK;
}

// Emit the CSR rows of hub window w (labels win[w]..win[w+1]) into col/bin (bin null for packed
// entries), entry e of the graph at col[e - win_e[w]]: the pair search of the build,
// run again.  Needs the sorted coordinates.
int emit_window(const gtc_graph_s *G, int64_t w, int32_t *col, uint8_t *bin, hipStream_t s);

// S4 configurations of the 4pCF (clique4.hip): count, canonical tuples [n][6] in rank order
int64_t num_configs_s4(int nb);
void config_bins_s4(int nb, int32_t *bins);
// Eq. (4) per S4 configuration from the binned 2pCF (twopoint.hip)
void disconnected_4pcf_s4(int nb, const double *xi, double *disc);

// A hub list to count instead of the graph's own (one-window graphs), with its totals.
struct HubSubset {
    const int32_t *hubs = nullptr;  // device, internal labels, each able to close a triangle
    int64_t n_hubs = 0;
    int64_t walks = 0;           // sum of forward degrees
    int64_t spoke_elements = 0;  // sum of work
};

// Device scratch a caller hands over (the allocation-free count): the count carves its arrays
// from [base, base + bytes) instead of allocating, and runs without timing events or a final
// synchronisation.
struct ExternalScratch {
    unsigned char *base = nullptr;
    size_t bytes = 0;
};

// Keep the hubs of in[0..n_in) (device) that can close a triangle, into out (device, n_in
// entries); d_sums: 3 device words of scratch.
int filter_hubs(const gtc_graph_s *G, const int32_t *in, int64_t n_in, int32_t *out,
                unsigned long long *d_sums, HubSubset *res, hipStream_t s);
}  // namespace gtc

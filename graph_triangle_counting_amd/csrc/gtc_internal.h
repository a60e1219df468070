// gtc_internal.h - declarations shared by the libgtc translation units (host and device).
//
// Data layout in device memory (internal labels = cell-sorted order):
//   xyz_s      int4 [n]      (x, y, z, cell key) of each point, cell-sorted
//   key_s      int32 [n]     cell key of each point
//   perm       int32 [n]     internal -> original label
//   cell_start int32 [ncell+1] first internal label of each cell (cells in key order)
//   row_ptr    int64 [n+1]   forward CSR offsets (64-bit: edge counts pass 2^31, §III.5.1)
//   col        int32 [E]     forward neighbours j > i, ascending per row (Eq.(1))
//   bin        uint8 [E]     radial bin of each edge (§II.1)
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
// Stream-ordered allocations from the device's default pool (kept cached between calls).
int dev_alloc(void **p, size_t bytes, hipStream_t s);
void dev_free(void *p, hipStream_t s);
template <class T>
int dev_alloc_n(T **p, size_t count, hipStream_t s) {
    return dev_alloc(reinterpret_cast<void **>(p), sizeof(T) * (count ? count : 1), s);
}
int fill_u64(uint64_t *p, int64_t count, uint64_t value, hipStream_t s);
int fill_u32(uint32_t *p, int64_t count, uint32_t value, hipStream_t s);

// hub windows: bounds[0..W] of consecutive rows whose CSR (5 bytes per edge) fits tile_bytes
int64_t plan_windows(const int64_t *row_ptr, int64_t n, int64_t tile_bytes, int64_t *bounds);

// exclusive scan of n int32 values: out[0..n], out[n] = total
int exclusive_scan_i32_to_i64(const int32_t *in, int64_t *out, int64_t n, hipStream_t s);
int exclusive_scan_i32_to_i32(const int32_t *in, int32_t *out, int64_t n, hipStream_t s);

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
    // device arrays
    int4 *xyz_s = nullptr;     // (x, y, z, cell key); dropped on request after the build
    int32_t *key_s = nullptr;  // cell key of each point (kept)
    int32_t *perm = nullptr;
    int32_t *cell_start = nullptr;
    int64_t *row_ptr = nullptr;
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
    std::vector<int64_t> win;       // W+1 label bounds
    std::vector<int64_t> win_hubs;  // W+1 offsets into hubs: window k's hubs, heaviest first
    std::vector<int32_t> win_smax;  // last window holding a spoke of window k's hubs
    std::vector<int64_t> h_row_ptr; // host copy of row_ptr (tiled graphs)
    int64_t max_window_edges = 0;
    // out-of-core: the CSR in pinned host memory, only windows go to the device
    bool host_csr = false;
    int32_t *h_col = nullptr;
    uint8_t *h_bin = nullptr;
};

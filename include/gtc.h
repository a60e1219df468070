/* gtc.h - C ABI of libgtc, the MI355X (gfx950) graph 3-point / 4-point correlation counter.
 *
 * The method is GRAMSCI v2, "Fast Graph-based Higher-Order Clustering Statistics on the GPU"
 * (arXiv 2607.06604): a fixed-radius neighbour graph stored as sorted adjacency rows with a
 * radial-bin byte per edge (§II.1, Eq.(1); CSR layout §III.5.1), hub-and-spoke triangle and
 * tetrahedron enumeration by sorted-list intersection (§II.2, §III.1, §III.1.1), counts binned by
 * side-length configuration (§V.1) and a parity split of the tetrahedra by the sign of the signed
 * volume (§III.2, Eq.(3)); graphs larger than a tile are processed in hub windows (§III.5.3).
 *
 * Conventions for every function:
 *   - Return value: GTC_OK (0) or a negative gtc_status.  No exception or abort crosses the ABI.
 *     gtc_last_error() gives a human-readable detail of the last failure on the calling thread.
 *   - Pointers named d_* are device pointers on the current HIP device; h_* are host pointers.
 *     The caller owns every buffer it passes; outputs are overwritten, never accumulated.
 *   - hip_stream is a hipStream_t (NULL = the null stream).  Work is ordered on it.  The count
 *     functions return after their outputs are complete (they synchronise the stream);
 *     gtc_build_graph synchronises once to size the edge arrays.
 *   - Argument checks that need no device data (null pointers, sizes, bin edges) fail with
 *     GTC_E_INVALID before any HIP call is made.
 *
 * Definitions (exact integer arithmetic throughout):
 *   - points: n integer triples in [0, 2^20)^3; d2(i,j) = sum of squared coordinate differences.
 *   - edges_sq: nbins+1 integers e_0 < e_1 < ... < e_nbins, e_0 >= 0.  i and j (i != j) are
 *     neighbours iff e_0 <= d2 < e_nbins, and the edge is in bin b iff e_b <= d2 < e_{b+1}.
 *   - each triangle (4-clique) is counted once.  Its configuration is the nondecreasing triple
 *     (6-tuple) of its edge bins; configurations are ranked from 0 in lexicographic order, which is
 *     the nested-loop order b1 = 0..nb-1, b2 = b1..nb-1, ... (the Fig. 8 configuration key).
 *   - weighted 3pCF: per triangle p = fl(fl(w1*w2)*w3) with its three weights in ascending
 *     order (fp64, separately rounded products).  weighted[c] is the exact sum over the
 *     configuration's triangles of q = rint(p * 2^s), rounded once to fp64, times 2^-s.
 *     s = 57 - e where a = max |w| over all n weights, M = fl(fl(a*a)*a) = f * 2^e with
 *     f in [0.5, 1) (s = 0 when M = 0).  q is exact whenever p's last significant bit is at least
 *     2^-s, e.g. for all weights in [0.5, 1.5).
 *   - parity: the four vertices of a tetrahedron are ordered by key(v) = sum of d2 to the other
 *     three, ascending; V = det[x1 - x0; x2 - x0; x3 - x0] (rows), i.e. (r01 x r02) . r03 of
 *     Eq.(3).  even[c] counts every tetrahedron; odd[c] adds +1 for V > 0, -1 for V < 0 and 0 if
 *     V == 0 or two keys are equal (no label-free handedness, the §III.2 degenerate rule).
 */
#ifndef GTC_H
#define GTC_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GTC_OK = 0,
    GTC_E_INVALID = -1,     /* bad argument or input value */
    GTC_E_OOM = -2,         /* device or pinned-host allocation failed */
    GTC_E_HIP = -3,         /* a HIP runtime call failed (detail in gtc_last_error) */
    GTC_E_OVERFLOW = -4,    /* a count does not fit the library's fixed-width types */
    GTC_E_UNSUPPORTED = -5  /* valid input outside what this build handles (detail given) */
} gtc_status;

#define GTC_MAX_BINS 255       /* 3pCF: nbins in [1, 255] */
#define GTC_MAX_BINS_4PCF 16   /* parity 4pCF: nbins in [1, 16] */
#define GTC_GRID_BITS 20       /* coordinates in [0, 2^20) */
#define GTC_NOALLOC_SCRATCH_BYTES (32u << 20) /* static device scratch of gtc_count_3pcf_noalloc,
                                                 per GPU */

/* gtc_options.csr_mode */
#define GTC_CSR_DEVICE 0
#define GTC_CSR_HOST 1
#define GTC_CSR_REBUILD 2

/* Opaque neighbour graph, owned by the library (device CSR in internal labels, see
 * gtc_graph_export).  Free with gtc_graph_free. */
typedef struct gtc_graph_s *gtc_graph;

/* Optional memory routines, so that a caller (e.g. PyTorch's caching allocator) owns every buffer
 * the library allocates.  alloc returns device memory usable on hip_stream in stream order (NULL on
 * failure, reported as GTC_E_OOM); free releases it in stream order.  host_alloc / host_free give
 * pinned host memory (the out-of-core CSR); NULL members fall back to hipMallocAsync /
 * hipFreeAsync / hipHostMalloc / hipHostFree.  The routines and ctx must stay valid while any
 * graph built with them lives: counts, exports and gtc_graph_free use the graph's routines. */
typedef struct {
    void *(*alloc)(size_t bytes, void *hip_stream, void *ctx);
    void (*free)(void *ptr, void *hip_stream, void *ctx);
    void *(*host_alloc)(size_t bytes, void *ctx);
    void (*host_free)(void *ptr, void *ctx);
    void *ctx;
} gtc_allocator;

/* Build options.  A zero-initialised struct (or NULL) means: resident CSR, coordinates kept,
 * memory from the HIP runtime. */
typedef struct {
    /* > 0: rows are split into hub windows whose CSR is at most tile_bytes (a single longer row
     * gets a window of its own), and counting runs as a loop over (hub window, search windows)
     * tiles (§III.5.3): a 3pCF tile takes every search window of its hub window when the CSR is
     * on the device, at most two otherwise.  The CSR takes 4 bytes per edge when n <= 2^24 (label and bin packed in
     * one word) and 5 bytes per edge otherwise.
     * 0: the environment variable GTC_TILE_BYTES, if set, gives the budget; otherwise one resident
     * window, unless the CSR would take more than 3/4 of the free device memory: then the build
     * goes out of core by itself, windows of 1/8 of the free memory, csr_mode GTC_CSR_REBUILD
     * (GTC_CSR_HOST if drop_coords is set).  gtc_graph_stats reports the outcome (windows,
     * csr_mode). */
    int64_t tile_bytes;
    /* Where the CSR is kept (§III.5.3):
     *   GTC_CSR_DEVICE  (0): in device memory.
     *   GTC_CSR_HOST    (1): in pinned host memory; a tile's windows are copied to the device
     *                        (on a copy stream, overlapped with the previous tile's counting).
     *   GTC_CSR_REBUILD (2): nowhere; a tile's windows are emitted again on the device from the
     *                        sorted coordinates (a window's pair search costs less than its copy
     *                        over the host link).  Needs the coordinates (not dropped).
     * Modes 1 and 2 need tile_bytes > 0.  The graph then holds three window buffers on the
     * device for its lifetime: the build stages its windows through them, and a 3pCF count
     * starts with the windows they hold.  In mode 1 the build returns while its last windows are
     * still being copied to host memory; every reader of the host CSR waits for those copies. */
    int32_t csr_mode;
    /* nonzero: drop the sorted coordinates after the build (gtc_count_4pcf_parity then fails
     * with GTC_E_INVALID).  Zero keeps them. */
    int32_t drop_coords;
    /* NULL: the HIP runtime's allocators.  Copied into the graph (the pointer need not outlive
     * the call, the routines and ctx must). */
    const gtc_allocator *allocator;
} gtc_options;

/* Run statistics.  Counts refer to one call; byte figures are algorithmic (see the
 * description of q_alg_bytes), times are HIP-event times on the call's stream. */
typedef struct {
    int64_t n;                 /* points */
    int64_t edges;             /* undirected edges E (= forward edges, stored once) */
    int64_t max_out_degree;    /* max forward degree d+(i) = |{j in N(i): j > i}| */
    int64_t merge_walks;       /* hub-spoke intersections performed (forward edges walked) */
    int64_t spoke_elements;    /* sum over walks of d+(j): spoke-row elements available to walk */
    int64_t tiles;             /* kernel launches of the enumeration (1 when resident) */
    int64_t windows;           /* hub windows */
    uint64_t triangles;        /* triangles counted (3pCF) */
    uint64_t cliques4;         /* 4-cliques counted (4pCF) */
    double q_alg_bytes;        /* 3pCF algorithmic bytes: 5E + 4*sum d+(j) over walks + triangles */
    int32_t weight_scale;      /* s of the weighted sums (0 when unweighted) */
    int32_t launch_waves;      /* enumeration kernel: waves per workgroup */
    int32_t launch_blocks;     /* enumeration kernel: persistent workgroups */
    int32_t launch_lds_bytes;  /* enumeration kernel: LDS per workgroup */
    int32_t launch_mode;       /* 3pCF: bit 0 banded walk (else one map over the hub domain),
                                  bit 1 histogram over the unsorted bin triple, bit 2 twice the
                                  spoke-row loads in flight per lane */
    int32_t csr_mode;          /* where the graph's CSR is kept: GTC_CSR_* (the build may go out
                                  of core by itself, see gtc_options.tile_bytes) */
    double build_ms;           /* gtc_build_graph: whole call */
    double kernel_ms;          /* enumeration kernels only (sum over tiles; 4pCF tiles that
                                * overlap on two streams: first start to last end) */
    double count_ms;           /* count call: whole call */
    double h2d_ms;             /* out-of-core: window copies (GTC_CSR_HOST) or window emits
                                  (GTC_CSR_REBUILD), summed; they overlap the counting */
} gtc_stats;

/* Free the pinned host block the library keeps for reuse.  Out-of-core builds with the CSR in
 * pinned host memory (GTC_CSR_HOST, no caller allocator) keep the largest freed pinned block and
 * give it to the next build whose CSR fits it (between the request and twice it), since pinning
 * costs about 10 ms per GB.  Call this to return that memory; graphs alive keep theirs. */
void gtc_release_host_cache(void);

/* Build the neighbour graph of n points (§II.1, Eq.(1)).
 *   d_xyz     device int32 [n][3], coordinates in [0, 2^20) (checked on the device:
 *             GTC_E_INVALID if any is outside).  Not retained: the graph keeps its own copy.
 *   n         0 <= n < 2^31.
 *   h_edges_sq host int64 [nbins+1], strictly increasing, e_0 >= 0, e_nbins <= 3*2^40 + 1.
 *   nbins     1..GTC_MAX_BINS.
 *   opt       may be NULL.
 *   out       receives the handle (NULL on failure).
 * Internal labels are the cell-sorted order (cells of side >= r_max); rows hold the forward
 * neighbours (j > i) ascending, with a bin byte per edge. */
int gtc_build_graph(const int32_t *d_xyz, int64_t n, const int64_t *h_edges_sq, int32_t nbins,
                    const gtc_options *opt, void *hip_stream, gtc_graph *out);

/* Binned triangle counts, the 3pCF numerator (§II.2, merge intersection §III.1).
 *   d_w        device fp64 [n] weights in the caller's (original) labels, or NULL.  Must be
 *              finite (GTC_E_INVALID otherwise).
 *   d_counts   device uint64 [gtc_num_configs(3, nbins)].
 *   d_weighted device fp64 [same], required iff d_w != NULL.
 *   st         may be NULL. */
int gtc_count_3pcf(gtc_graph g, const double *d_w, uint64_t *d_counts, double *d_weighted,
                   gtc_stats *st, void *hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): gtc_count_3pcf on a graph built beforehand, with every
 * per-call device buffer (hub-queue counters; weighted: the weights in internal order, the exact
 * sum limbs) carved from one static device array of GTC_NOALLOC_SCRATCH_BYTES on each GPU, which
 * that GPU holds until the process ends.  No hipMalloc, hipFree or other allocation, no timing
 * events; the call is asynchronous on hip_stream except that a weighted count synchronises once
 * to read max |w| (the scale of the exact sums).  Results equal gtc_count_3pcf's bit for bit.
 *   g, d_w, d_counts, d_weighted, hip_stream: as gtc_count_3pcf (no statistics).
 * Errors: GTC_E_INVALID as gtc_count_3pcf; GTC_E_UNSUPPORTED for a graph whose CSR is out of
 * core (GTC_CSR_HOST or GTC_CSR_REBUILD: its window buffers are per-call allocations; hub
 * windows over a resident CSR are counted) or when the call's scratch exceeds the array
 * (unweighted: a few KB; weighted: 8 bytes per point plus 32 per configuration, so about 4M
 * points); GTC_E_HIP if the array's device address cannot be obtained.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on different
 * streams or threads) race and give wrong results; calls ordered on one stream are safe.  The
 * array keeps the last call's contents; each call clears what it needs zeroed. */
int gtc_count_3pcf_noalloc(gtc_graph g, const double *d_w, uint64_t *d_counts,
                           double *d_weighted, void *hip_stream);

/* The 3pCF of a subset of hubs: the binned triangles whose first vertex in the graph's internal
 * order (gtc_graph_export's h_perm maps internal labels to point indices) is one of the listed
 * hubs.  Disjoint hub sets give counts that add up to gtc_count_3pcf's, which makes this the
 * per-shard primitive of a split hub range, and lets full-size runs be checked hub by hub.
 *   h_hubs  host int32 [n_hubs]: distinct internal labels in [0, n) (hubs that can close no
 *           triangle are allowed and contribute nothing).
 *   d_w, d_counts, d_weighted, st, hip_stream: as gtc_count_3pcf.  The weighted scale s comes
 *           from max |w| over all points, as in gtc_count_3pcf.  st describes the subset
 *           (merge_walks, spoke_elements and q_alg_bytes of the listed hubs).
 * GTC_E_INVALID for a repeated or out-of-range label; GTC_E_UNSUPPORTED for a graph of more than
 * one hub window. */
int gtc_count_3pcf_hubs(gtc_graph g, const int32_t *h_hubs, int64_t n_hubs, const double *d_w,
                        uint64_t *d_counts, double *d_weighted, gtc_stats *st, void *hip_stream);

/* Binned 4-clique counts split by parity (§II.2, §III.1.1, §III.2).  Needs nbins <=
 * GTC_MAX_BINS_4PCF and the coordinates (not dropped).  Out-of-core graphs (csr_mode 1 or 2) run
 * as tiles (hub window h, search windows c1 <= c2) (§III.5.3): the tetrahedra i < a < b < c
 * whose hub i, spoke a and spoke b lie in windows h, c1 and c2, so that three windows are
 * resident at a time; st->tiles reports the launches.
 *   d_even     device uint64 [gtc_num_configs(4, nbins)]: every tetrahedron.
 *   d_odd      device int64  [same]: signed handedness sum. */
int gtc_count_4pcf_parity(gtc_graph g, uint64_t *d_even, int64_t *d_odd, gtc_stats *st,
                          void *hip_stream);

/* S4 configurations of the 4pCF (§III.3): a tetrahedron's six edge bins, in the edge order
 * (01, 02, 03, 12, 13, 23) of its vertices 0..3, up to the 24 relabellings of the vertices -- the
 * configuration on which Eq. (4) is evaluated.  A configuration's canonical tuple is its
 * lexicographically smallest relabelling; configurations are numbered by canonical tuple in
 * lexicographic order.  There are (k^6 + 9 k^4 + 14 k^2) / 24 of them for k bins (276 at 4 bins,
 * 12,496 at 8).  nbins <= GTC_MAX_BINS_4PCF.
 *   gtc_count_4pcf_parity_s4: as gtc_count_4pcf_parity, with even / odd of
 *     [gtc_num_configs_s4(nbins)] indexed by S4 configuration.
 *   gtc_num_configs_s4: the number of configurations, or -1 for nbins out of range.
 *   gtc_config_bins_s4: h_bins host int32 [n_cfg][6], the canonical tuples in rank order.
 *   gtc_config_realizable_s4: h_mask host uint8 [n_cfg]: 1 where the bin centres (midpoint in r of
 *     [sqrt(e_b), sqrt(e_{b+1}))) are the edge lengths of a tetrahedron of positive volume -- a
 *     positive Cayley-Menger determinant, every face a proper triangle (§V.2: 178 of 276 at
 *     4 bins); h_edges_sq as gtc_build_graph.  Host only. */
int gtc_count_4pcf_parity_s4(gtc_graph g, uint64_t *d_even, int64_t *d_odd, gtc_stats *st,
                             void *hip_stream);

/* The 2pCF on the graph's pairs (§II.1; the internal 2pCF of §III.3): every pair (each edge once)
 * counted in its bin, and with weights the exact sums of w_i w_j.  Each product p = fl(w_i * w_j)
 * is scaled to the integer q = rint(p * 2^s), s = 57 - e for M = fl(a * a) = f * 2^e, f in
 * [0.5, 1), a = max |w| (s = 0 if M == 0); the q are summed exactly and each bin is rounded once.
 * With data weights summing to +1 and random weights to -1, the sums are the Landy-Szalay
 * numerator DD - 2DR + RR, so xi = sum / RR.
 *   d_w        device double [n] in original labels, or NULL.
 *   d_counts   device uint64 [nbins] (overwritten); d_weighted device double [nbins] or NULL.
 *   st         stats: kernel_ms summed over windows, weight_scale = s, q_alg_bytes.
 * Works on every csr_mode (out-of-core windows are uploaded or emitted again one at a time).
 * GTC_E_INVALID for a non-finite weight. */
int gtc_count_2pcf(gtc_graph g, const double *d_w, uint64_t *d_counts, double *d_weighted,
                   gtc_stats *st, void *hip_stream);

/* The disconnected 4pCF, Eq. (4), per S4 configuration from the binned 2pCF (host only):
 * h_disc[c] = xi(b01) xi(b23) + xi(b02) xi(b13) + xi(b03) xi(b12) for configuration c's canonical
 * tuple, the sum over the three splits of the four vertices into two pairs.
 *   h_xi host double [nbins]; h_disc host double [gtc_num_configs_s4(nbins)].
 * gtc_connected_4pcf_s4 returns Eq. (5), h_conn = h_zeta - disc, for a full 4pCF h_zeta of the
 * same shape (the parity-even channel; the odd channel is connected as it is). */
int gtc_disconnected_4pcf_s4(int32_t nbins, const double *h_xi, double *h_disc);
int gtc_connected_4pcf_s4(int32_t nbins, const double *h_zeta, const double *h_xi,
                          double *h_conn);
/* Weighted parity 4pCF (the numerator NNNN of the 4pCF estimator, §II.1, §III.2): the counts of
 * gtc_count_4pcf_parity (s4 == 0) or gtc_count_4pcf_parity_s4 (s4 != 0), and the sums over the
 * tetrahedra of p = fl(fl(fl(w1*w2)*w3)*w4), the four weights ascending, without fused
 * multiply-add (even channel, d_even_w) and of sign(V) * p (odd channel, d_odd_w).  Each p is
 * scaled to the integer q = rint(p * 2^s), s = 57 - e for M = fl(fl(fl(a*a)*a)*a) = f * 2^e,
 * a = max |w|; the q are summed exactly and each configuration's sums are rounded once.
 *   d_w device double [n], original labels; d_even_w, d_odd_w device double [n_cfg].
 *   st->weight_scale receives s. */
int gtc_count_4pcf_weighted(gtc_graph g, const double *d_w, int32_t s4, uint64_t *d_even,
                            int64_t *d_odd, double *d_even_w, double *d_odd_w, gtc_stats *st,
                            void *hip_stream);
int64_t gtc_num_configs_s4(int32_t nbins);
int gtc_config_bins_s4(int32_t nbins, int32_t *h_bins);
int gtc_config_realizable_s4(int32_t nbins, const int64_t *h_edges_sq, uint8_t *h_mask);

/* The equilateral configurations (§III.5's equilateral 3pCF query; its 4pCF analogue, the regular
 * tetrahedron): h_ranks[b] = the rank of the configuration whose edges all lie in bin b, for b <
 * nbins, among gtc_config_bins(3 or 4, nbins) (s4 == 0) or gtc_config_bins_s4(nbins) (order 4,
 * s4 != 0).  The equilateral 3pCF of bin b is a 3pCF output at h_ranks[b].  Host only.
 *   h_ranks host int64 [nbins].  GTC_E_INVALID for order not 3 or 4, s4 with order 3, nbins out
 *   of range or h_ranks NULL. */
int gtc_equilateral_configs(int32_t order, int32_t s4, int32_t nbins, int64_t *h_ranks);

/* Number of configurations: C(nbins+2, 3) for order 3, C(nbins+5, 6) for order 4; -1 if the
 * order or nbins is out of range. */
int64_t gtc_num_configs(int32_t order, int32_t nbins);

/* The bins of every configuration in rank order: h_bins int32 [n_cfg][order == 3 ? 3 : 6]
 * (host), each row nondecreasing. */
int gtc_config_bins(int32_t order, int32_t nbins, int32_t *h_bins);

/* Copy the graph out to host memory (for tests and inspection).
 *   h_row_ptr int64 [n+1], h_col int32 [E], h_bin uint8 [E]: forward CSR in internal labels
 *   (unpacked: labels and bins come out separately whatever the device layout);
 *   h_perm    int32 [n]: h_perm[internal] = original label.  Any pointer may be NULL. */
int gtc_graph_export(gtc_graph g, int64_t *h_row_ptr, int32_t *h_col, uint8_t *h_bin,
                     int32_t *h_perm);

/* Hub windows of the tile loop (§III.5.3), for inspection and tests; host only, needs no GPU.
 *   h_row_ptr host int64 [n+1] forward CSR offsets (nondecreasing).
 *   tile_bytes > 0: budget per window in CSR bytes; a row longer than the budget gets a window
 *              of its own.
 *   entry_bytes > 0: CSR bytes per edge (gtc_build_graph: 4 when n <= 2^24, else 5).
 *   h_bounds  host int64 [n+1] (at least 2): receives the label bounds 0 = b_0 < ... < b_W = n of
 *              consecutive rows (b_1 = 0 when n = 0).
 * Returns W >= 1, or GTC_E_INVALID.  gtc_build_graph uses the same windows; tile (h, s) then
 * walks the spokes of hub window h that lie in window s, for s from h to the window of the
 * largest spoke label of window h, so every forward edge is walked in exactly one tile. */
int64_t gtc_plan_windows(const int64_t *h_row_ptr, int64_t n, int64_t tile_bytes,
                         int32_t entry_bytes, int64_t *h_bounds);

/* Hub windows of a built graph (§III.5.3), for inspection and tests; host only, no GPU work.
 *   h_bounds  host int64 [W+1] or NULL: label bounds b_0 = 0 < ... < b_W = n of the windows, as
 *             gtc_plan_windows gives them for the graph's CSR offsets and budget (the build plans
 *             them on the device; one window [0, n) when the graph is not tiled).
 *   h_offsets host int64 [W+1] or NULL: CSR offsets of the bounds, row_ptr[b_k].
 *   capacity  entries each non-NULL array holds; the arrays are written only when capacity >=
 *             W + 1 (call with capacity 0 to learn W).
 * Returns W >= 1, or GTC_E_INVALID for a null graph, capacity < 0, or capacity > 0 with both
 * arrays NULL. */
int64_t gtc_graph_windows(gtc_graph g, int64_t *h_bounds, int64_t *h_offsets, int64_t capacity);

/* Squared edges of nbins equal radial bins from r_min to r_max (§IV: bins equally spaced in r
 * from r_min to r_max), as integers: h_edges_sq[b] = ceil(r_b^2), r_b = r_min + b (r_max - r_min)
 * / nbins, so that an integer squared distance d^2 falls in bin b exactly when r_b <= d < r_{b+1}.
 * Pairs closer than r_min are outside every bin.
 *   r_min, r_max grid units, 0 <= r_min < r_max <= 2^21; h_edges_sq host int64 [nbins + 1].
 * GTC_E_INVALID for a range out of bounds or two bins whose integer edges coincide.  Host only. */
int gtc_linear_edges_sq(int64_t r_min, int64_t r_max, int32_t nbins, int64_t *h_edges_sq);

/* The 3pCF and 4pCF estimators on a data catalogue D and a random catalogue R (§II.1, §III.3;
 * the compute_3pcf / compute_4pcf interface of §II.2).  One neighbour graph is built over D then
 * R (D's points take labels 0..n_data-1, R's the rest).  The numerators take the signed,
 * normalised weights w / sum_D w on D and -w / sum_R w on R (the sums rounded correctly); the
 * denominators take w / sum_R w on R and 0 on D, which only all-random cliques feed, so they are
 * counted on a second graph over R alone (same cliques, bins and exact sums, fewer cliques):
 *   3pCF: zeta = NNN / RRR per configuration of gtc_count_3pcf.
 *   4pCF: zeta_even = NNNN_even / RRRR and zeta_odd = NNNN_odd / RRRR per S4 configuration of
 *         gtc_count_4pcf_parity_s4; xi = NN / RR per bin from the graph's pairs; zeta_conn =
 *         zeta_even - disc(xi), Eq. (4) and (5).
 * A configuration with no random triangle (tetrahedron) gives 0/0 or x/0 (NaN or infinity).
 *   d_xyz_data device int32 [n_data][3], d_xyz_rand device int32 [n_rand][3]: grid coordinates as
 *              gtc_build_graph; n_data >= 0, n_rand >= 1, n_data + n_rand < 2^31.
 *   d_w_data, d_w_rand device double [n_data], [n_rand], finite, or NULL for unit weights; each
 *              catalogue's weights must not sum to zero.
 *   h_edges_sq, nbins, opt: as gtc_build_graph (gtc_compute_4pcf: nbins <= GTC_MAX_BINS_4PCF and
 *              coordinates kept).
 *   h_zeta     host double [gtc_num_configs(3, nbins)]; h_nnn, h_rrr the same or NULL.
 *   h_zeta_even, h_zeta_odd host double [gtc_num_configs_s4(nbins)]; h_zeta_conn the same or
 *              NULL; h_xi host double [nbins] or NULL.
 *   st         may be NULL: the first count's statistics, kernel_ms and count_ms summed over
 *              every count of the call.
 * The call builds and frees its own graph and synchronises the stream before it returns. */
int gtc_compute_3pcf(const int32_t *d_xyz_data, int64_t n_data, const double *d_w_data,
                     const int32_t *d_xyz_rand, int64_t n_rand, const double *d_w_rand,
                     const int64_t *h_edges_sq, int32_t nbins, const gtc_options *opt,
                     double *h_zeta, double *h_nnn, double *h_rrr, gtc_stats *st,
                     void *hip_stream);
int gtc_compute_4pcf(const int32_t *d_xyz_data, int64_t n_data, const double *d_w_data,
                     const int32_t *d_xyz_rand, int64_t n_rand, const double *d_w_rand,
                     const int64_t *h_edges_sq, int32_t nbins, const gtc_options *opt,
                     double *h_zeta_even, double *h_zeta_odd, double *h_zeta_conn, double *h_xi,
                     gtc_stats *st, void *hip_stream);

/* Measurement: the HBM read rate of a plain streaming kernel (16-byte loads over d_buf, grid-
 * stride, best of reps timed launches after one untimed), in GB/s of bytes read: the measured
 * ceiling of a read-dominated kernel beside the vendor peak.
 *   d_buf device, 16-byte aligned, bytes >= 16 (read, not written); reps >= 1.
 * Synchronises the stream.  GTC_E_INVALID for bad arguments. */
int gtc_hbm_read_rate(const void *d_buf, int64_t bytes, int32_t reps, double *h_gbs,
                      void *hip_stream);

/* Graph-level statistics (n, edges, max_out_degree, windows, spoke_elements, build_ms). */
int gtc_graph_stats(gtc_graph g, gtc_stats *st);

/* Free a graph (NULL is a no-op).  Device memory is released in order on the build stream. */
void gtc_graph_free(gtc_graph g);

/* Static description of a status code, and the detail of the last failure on this thread. */
const char *gtc_status_string(int status);
const char *gtc_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GTC_H */

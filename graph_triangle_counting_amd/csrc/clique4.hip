// clique4.hip - binned 4-clique (tetrahedron) counts split by parity (GRAMSCI v2 §II.2,
// §III.1.1, §III.2, per-hub local connectivity matrix §III.5.2).
//
// One wavefront per hub i.  With N+(i) = {j_0 < ... < j_{m-1}} the wave builds the hub's local
// connectivity among its forward neighbours: bit b of row a is set iff j_a ~ j_b (a < b).  Row a
// comes from one walk of N+(j_a) against the hub, exactly the triangle walk of the 3pCF kernel,
// with the LDS hub map holding row positions.  This replaces the pages' three-pointer walk per
// (i, j1, j2) by one walk per (i, j1) plus bitset intersections: every tetrahedron i < j_a < j_b
// < j_c is a set bit c of row_a AND row_b.  The pages keep this matrix in a global scratch slot
// per gang; it lives in LDS here.
//
// The hub's tetrahedra are dealt out evenly over the lanes: a wave-wide prefix sum numbers the
// edges (a, b) of a batch of bitset words, a second one numbers the tetrahedra of 64 such edges,
// and each lane walks an equal share of them in order.
//
// Per tetrahedron: the six edge bins, sorted and ranked (lexicographic rank of the nondecreasing
// 6-tuple, one table entry per position), and the parity sign: vertices ordered by the sum of
// their squared edge lengths, and the sign of the signed volume (r01 x r02) . r03 (Eq.(3)) in that
// order, zero for a tie or zero volume.  Lengths and keys are exact in fp64 (hub-relative integer
// coordinates below 2^20); the volume's sign comes from fp64 behind an error-bound filter, or
// exactly from int64 when the filter cannot decide.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <cmath>
#include <thread>
#include <mutex>
#include <map>
#include <vector>

#include "gtc_internal.h"

namespace gtc {

struct CliqueArgs {
    const int64_t *row_ptr;
    // The rows a launch reads (§III.5.3, 4pCF tiles): hub rows from window h, spoke rows from
    // windows c1 <= c2 with label ranges [w1_lo, w1_hi) and [w2_lo, w2_hi).  Entry e of the graph
    // sits at col_x[e - base_x] (bin_x likewise; null: packed entries, the bin in the top byte).
    // A tile counts the tetrahedra (i, a, b, c), i < a < b < c, with a in c1 and b in c2: the
    // edges among the spokes come from the rows of a and b.  A resident graph is one tile with
    // all three windows the whole CSR.
    // A launch over a hub window and the next one together takes both as c1 = c2, their rows
    // in two buffers of one allocation: spoke rows at or after CSR offset e_split then sit at
    // col_1[e - base_1b].
    const int32_t *col_h, *col_1, *col_2;
    const uint8_t *bin_h, *bin_1, *bin_2;
    int64_t base_h, base_1, base_2;
    int64_t e_split, base_1b;
    int32_t w1_lo, w1_hi, w2_lo, w2_hi;
    int32_t tiled;         // 0: one resident tile (every spoke in both ranges)
    uint32_t label_mask;   // label bits of a col word
    const uint32_t *s4rank;  // null: sorted 6-tuple ranks; else the S4 configuration of every
                             // base-nb key of the six bins in edge order (01,02,03,12,13,23)
    const int32_t *hubs;
    int32_t n_hubs;
    int32_t nb, ncfg;
    int32_t map_bytes;     // per-wave position map (uint16 per domain label), multiple of 16
    int32_t max_m;         // longest forward row
    int32_t words;         // 32-bit words per bitset row = ceil(max_m / 32)
    const int4 *xyz_s;
    const int32_t *cell_start;
    Grid gr;
    unsigned int *queue;         // class counters, kQueueStride words apart
    const unsigned int *qcount;  // [kHubClasses] hubs per class in the hub list
    unsigned int batch_cap;      // largest batch of hubs per take
    unsigned long long *even;  // [ncfg]
    unsigned long long *odd;   // [ncfg], two's complement int64
    unsigned int flush_at;
    // weighted: weights in internal order, 2^s, and the sums of q by handedness class (sign(V) =
    // +1, -1, 0) as [ncfg][3] two's complement 128-bit words (low, high), replicated over wcopies
    // copies wstride words apart (workgroup b adds to copy b % wcopies)
    const double *w_s;
    double two_s;
    unsigned long long *wsum;
    int wcopies;
    long long wstride;
    // LDS configuration cache (weighted, WM 3): cache_k configurations have an LDS slot:
    // cache_slot[rank] is the slot or -1, cache_rank[slot] the configuration
    int32_t cache_k;
    int32_t slot_in_rank;  // S4 with a cache: s4rank entries carry slot + 1 in bits 20-31
    const int16_t *cache_slot;
    const int32_t *cache_rank;
};

__device__ __forceinline__ void wave_lds_sync4() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) / 16 * 16; }

// rank of a nondecreasing 6-tuple b_0 <= ... <= b_5 of [0, nb) in lexicographic order, as a sum
// of one table entry per position: rank = sum_q G[q][b_q].  With N = nb + 5 and c_q = b_q + q the
// combinatorial number system gives rank = C(N, 6) + sum_{q<5} C(N - c_q - 1, 5 - q) -
// sum_q C(N - c_q, 6 - q); G[q][b] collects the terms of position q (C(N, 6) goes to q = 0).
constexpr int kRankTab = 6 * GTC_MAX_BINS_4PCF;
// S4 rank table entries: the rank in the low 20 bits (num_configs_s4(16) = 723,776 < 2^20) and,
// with a configuration cache, the rank's slot + 1 above them (0: not cached)
constexpr uint32_t kRankMask = (1u << 20) - 1;
constexpr int kSlotShift = 20;
constexpr int kMaxTableSlots = (1 << (32 - kSlotShift)) - 2;

// fixed part: even / odd count bins (unless global), the rank table G[6][16], (LDS class sums)
// [ncfg][3][2] words.  With an LDS configuration cache of k > 0 slots: even / odd bins and class
// sums per slot, the slot of every configuration (int16) and the configuration of every slot.
__host__ __device__ inline size_t clique_lds_fixed(int ncfg, bool gh, bool wl = false, int k = 0,
                                                   bool slot_table = true) {
    if (k > 0)
        return align16(4 * (size_t)k) * 2 + 4 * kRankTab + 32 * (size_t)k +
               (slot_table ? align16(2 * (size_t)ncfg) : 0) + align16(4 * (size_t)k);
    return (gh ? 0 : align16(4 * (size_t)ncfg) * 2) + 4 * kRankTab + (wl ? 48 * (size_t)ncfg : 0);
}
// per-wave enumeration scratch: bitset words and their edge offsets, edges and their
// tetrahedron offsets, 64 entries each
constexpr size_t kEnumScratch = 4 * 64 * 4;
constexpr int kConnLoads = 4;  // row loads in flight per lane while building the connectivity
constexpr int kCacheStride = 64;  // configuration cache: every 64th hub of the hub list is sampled
constexpr int kCacheMin = 256;    // fewest LDS slots worth a cache
// per-wave part: position map, row coordinates (hub-relative), hub-edge bins, bitset rows,
// (weighted) row weights, enumeration scratch
__host__ __device__ inline size_t clique_lds_wave(int map_bytes, int max_m, int words,
                                                  bool weighted = false) {
    return (size_t)map_bytes + align16(16 * (size_t)max_m) + align16((size_t)max_m) +
           align16(4 * (size_t)max_m * words) + (weighted ? align16(8 * (size_t)max_m) : 0) +
           kEnumScratch;
}

// Add a signed 64-bit v to the two's complement 128-bit word p[0] (low) | p[1] (high): the low
// word takes v, the high word its sign extension plus the carry, which cancel (and skip the second
// atomic) unless v >= 0 carries or v < 0 borrows -- rare for |v| << 2^64.  Concurrent adds commute.
__device__ __forceinline__ void add_i128(unsigned long long *p, long long v) {
    const unsigned long long u = (unsigned long long)v;
    const unsigned long long old = atomicAdd(p, u);
    const long long dh = (v < 0 ? -1ll : 0ll) + (old + u < old ? 1ll : 0ll);
    if (dh) atomicAdd(p + 1, (unsigned long long)dh);
}

// add the 128-bit word (lo, hi) to p[0] | p[1]
__device__ __forceinline__ void add_u128_pair(unsigned long long *p, unsigned long long lo,
                                              unsigned long long hi) {
    const unsigned long long old = atomicAdd(p, lo);
    hi += (old + lo < old) ? 1ull : 0ull;
    if (hi) atomicAdd(p + 1, hi);
}

template <class T>
__device__ __forceinline__ void cswap(T &a, T &b) {
    const T lo = a < b ? a : b, hi = a < b ? b : a;
    a = lo;
    b = hi;
}

// Sign of C . X for X = A x B (A, B, C integer vectors with |components| < 2^20, so X's
// components are exact doubles below 2^41): the fp64 value decides when it exceeds a bound on its
// rounding error (three roundings of terms at most S = sum |C_k X_k|, well inside 8 u S); else the
// exact int64 value (|C . X| < 3 2^61).
__device__ __forceinline__ int orient_sign(double4 C, double X0, double X1, double X2) {
    const double d = fma(C.z, X2, fma(C.y, X1, C.x * X0));
    const double S = fabs(C.x * X0) + fabs(C.y * X1) + fabs(C.z * X2);
    if (fabs(d) > 0x1p-50 * S) return d > 0.0 ? 1 : -1;
    const int64_t v = (int64_t)C.x * (int64_t)X0 + (int64_t)C.y * (int64_t)X1 +
                      (int64_t)C.z * (int64_t)X2;
    return (v > 0) - (v < 0);
}

// inclusive prefix sum of v over the 64 lanes of the wave
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(v, d, kWave);
        if (lane >= d) v += u;
    }
    return v;
}

// largest L in [0, 64) with off[L] <= x, for nondecreasing off[0..63] with off[0] <= x
__device__ __forceinline__ int last_le(const int32_t *off, int x) {
    int L = 0;
#pragma unroll
    for (int s = 32; s > 0; s >>= 1)
        if (off[L + s] <= x) L += s;
    return L;
}

// position of the set bit of x with r set bits below it (0 <= r < popcount(x))
__device__ __forceinline__ int select_bit(uint32_t x, int r) {
    int pos = 0;
#pragma unroll
    for (int h = 16; h > 0; h >>= 1) {
        const int c = __popc(x & ((1u << h) - 1u));
        const bool up = r >= c;
        r = up ? r - c : r;
        x = up ? x >> h : x;
        pos = up ? pos + h : pos;
    }
    return pos;
}

// bin of an exact squared distance d2 < e_nb (a double below 2^53): se holds the edges as doubles,
// padded with +inf up to a power of two P >= nb, and the search takes log2(P) steps of a size the
// whole wave shares (h = P/2, P/4, ..., 1)
__device__ __forceinline__ int edge_bin_d(double d2, const double *se, int half) {
    int l = 0;
    for (int h = half; h > 0; h >>= 1)
        if (d2 >= se[l + h]) l += h;
    return l;
}

__device__ __forceinline__ double sq3(double x, double y, double z) { return fma(z, z, fma(y, y, x * x)); }

// an integer vector (|components| < 2^20) as doubles, with its squared length: all exact
__device__ __forceinline__ double4 rel4(int4 q) {
    const double x = q.x, y = q.y, z = q.z;
    return make_double4(x, y, z, sq3(x, y, z));
}


// GH: bins go straight to global memory (configuration counts too large for LDS).  WM: 0
// unweighted; 1 weighted, class sums in global memory; 2 weighted, class sums in LDS, added to
// global memory when the workgroup ends; 3 weighted, counts and class sums of the cache_k cached
// configurations in LDS, of the others in global memory.
template <bool GH, int WM>
__global__ void __launch_bounds__(1024) k_clique4(CliqueArgs a, const int64_t *edges) {
    constexpr bool WT = WM != 0;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ double se[GTC_MAX_BINS_4PCF + 1];  // squared edges (integers below 2^53), +inf pad
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int nslot = WM == 3 ? a.cache_k : a.ncfg;  // LDS count bins (and class sums)
    const size_t hist_bytes = GH ? 0 : align16(4 * (size_t)nslot);
    uint32_t *ev = reinterpret_cast<uint32_t *>(smem);
    int32_t *od = reinterpret_cast<int32_t *>(smem + hist_bytes);
    int32_t *rtab = reinterpret_cast<int32_t *>(smem + 2 * hist_bytes);  // G[q][b] at q * 16 + b
    unsigned long long *wl = reinterpret_cast<unsigned long long *>(smem + 2 * hist_bytes + 4 * kRankTab);
    // class sums in LDS: [nslot][3] 128-bit words (A+, A-, A0) in WM 2; in WM 3 [nslot][2], the
    // even sum E = A+ + A- + A0 and the odd sum O = A+ - A- (32 bytes a slot, so more slots fit)
    constexpr int kSlotWords = WM == 3 ? 4 : 6;
    int16_t *slot16 = reinterpret_cast<int16_t *>(smem + 2 * hist_bytes + 4 * kRankTab +
                                                  8 * kSlotWords * (size_t)nslot);
    // (S4: the slots come with the configuration's rank from the rank table, no LDS slot index)
    const bool sir = WM == 3 && a.slot_in_rank;
    int32_t *rank_of = reinterpret_cast<int32_t *>(reinterpret_cast<unsigned char *>(slot16) +
                                                   (sir ? 0 : align16(2 * (size_t)a.ncfg)));
    unsigned char *wbase = smem + clique_lds_fixed(a.ncfg, GH, WM == 2, WM == 3 ? a.cache_k : 0, !sir) +
                           (size_t)wid * clique_lds_wave(a.map_bytes, a.max_m, a.words, WT);
    uint16_t *pmap = reinterpret_cast<uint16_t *>(wbase);
    int4 *rc = reinterpret_cast<int4 *>(wbase + a.map_bytes);
    uint8_t *rbin = wbase + a.map_bytes + align16(16 * (size_t)a.max_m);
    uint32_t *adj = reinterpret_cast<uint32_t *>(wbase + a.map_bytes + align16(16 * (size_t)a.max_m) +
                                                 align16((size_t)a.max_m));
    double *rw = reinterpret_cast<double *>(reinterpret_cast<unsigned char *>(adj) +
                                            align16(4 * (size_t)a.max_m * a.words));
    // enumeration scratch: after the weights (weighted) or the bitset rows
    int32_t *sw_off = reinterpret_cast<int32_t *>(reinterpret_cast<unsigned char *>(rw) +
                                                  (WT ? align16(8 * (size_t)a.max_m) : 0));
    uint32_t *sw_bits = reinterpret_cast<uint32_t *>(sw_off + kWave);
    int32_t *eb_off = reinterpret_cast<int32_t *>(sw_bits + kWave);
    uint32_t *eb_ab = reinterpret_cast<uint32_t *>(eb_off + kWave);
    const int N = a.nb + 5;  // 6-combinations of [0, N) <-> nondecreasing 6-tuples of [0, nb)
    unsigned long long *wg = nullptr;  // this workgroup's copy of the global class sums
    if (WT) wg = a.wsum + (long long)(blockIdx.x % (unsigned)a.wcopies) * a.wstride;
    if (WM >= 2)
        for (int t = threadIdx.x; t < kSlotWords * nslot; t += blockDim.x) wl[t] = 0ull;
    if (WM == 3) {
        if (!sir)
            for (int t = threadIdx.x; t < a.ncfg; t += blockDim.x) slot16[t] = a.cache_slot[t];
        for (int t = threadIdx.x; t < nslot; t += blockDim.x) rank_of[t] = a.cache_rank[t];
    }

    if (!GH)
        for (int t = threadIdx.x; t < nslot; t += blockDim.x) {
            ev[t] = 0;
            od[t] = 0;
        }
    int bin_half = 1;  // P / 2 for the smallest power of two P >= nb (0 for nb = 1)
    while (2 * bin_half < a.nb) bin_half *= 2;
    if (a.nb == 1) bin_half = 0;
    for (int t = threadIdx.x; t <= GTC_MAX_BINS_4PCF; t += blockDim.x)
        se[t] = t <= a.nb ? (double)edges[t] : __longlong_as_double(0x7ff0000000000000ll);
    for (int t = threadIdx.x; t < kRankTab; t += blockDim.x) {
        const int q = t / GTC_MAX_BINS_4PCF, b = t % GTC_MAX_BINS_4PCF, c = b + q;
        auto C = [](int x, int r) -> int64_t {  // C(x, r), exact at each step; 0 outside
            if (r < 0 || x < r) return 0;
            int64_t v = 1;
            for (int u = 1; u <= r; ++u) v = v * (x - r + u) / u;
            return v;
        };
        const int64_t g = (q <= 4 ? C(N - c - 1, 5 - q) : 0) - C(N - c, 6 - q) + (q == 0 ? C(N, 6) : 0);
        rtab[t] = b < a.nb ? (int32_t)g : 0;
    }
    __syncthreads();

    unsigned int wave_cl = 0;
    // weighted, global class sums: the lane's pending class sum (index 3 rank + class, 128-bit
    // value), added out when a tetrahedron of another configuration or class comes, and at the
    // end (global atomics are bound by throughput; a run of one configuration takes one)
    int pend = -1;
    unsigned long long plo = 0ull, phi = 0ull;
    HubQueue hub_queue;
    hub_queue.init(a.qcount, a.batch_cap, lane, (int)(blockIdx.x % kQueueParts));
    for (;;) {
        uint32_t hq;
        if (!hub_queue.next(a.queue, lane, hq)) break;
        const int32_t i = __builtin_amdgcn_readfirstlane(a.hubs[hq]);
        const int64_t rb = a.row_ptr[i];
        const int32_t m = (int32_t)(a.row_ptr[i + 1] - rb);
        if (m < 3) continue;
        const int32_t *hrow = a.col_h + (rb - a.base_h);
        const uint8_t *hbin = a.bin_h ? a.bin_h + (rb - a.base_h) : nullptr;
        auto hlab = [&](int p) { return (int32_t)((uint32_t)hrow[p] & a.label_mask); };
        // spoke positions [p1_lo, p1_hi) in window c1 and [p2_lo, p2_hi) in window c2
        auto lower = [&](int32_t lab) {
            int l = 0, h = m;
            while (l < h) { const int md = (l + h) >> 1; if (hlab(md) < lab) l = md + 1; else h = md; }
            return l;
        };
        const int p1_lo = a.tiled ? lower(a.w1_lo) : 0, p1_hi = a.tiled ? lower(a.w1_hi) : m;
        const int p2_lo = a.w2_lo == a.w1_lo ? p1_lo : lower(a.w2_lo);
        const int p2_hi = a.w2_lo == a.w1_lo ? p1_hi : lower(a.w2_hi);
        if (p1_lo >= p1_hi || p2_lo >= p2_hi) continue;  // no spoke pair of this tile
        const int4 pi = a.xyz_s[i];
        HubDomain dom;
        hub_domain(i, pi.w, a.gr, a.cell_start, dom);
        const int W = (m + 31) >> 5;

        uint32_t *pm32 = reinterpret_cast<uint32_t *>(pmap);
        for (int t = lane; t < ((dom.size + 1) >> 1); t += kWave) pm32[t] = 0u;
        for (int t = lane; t < m * W; t += kWave) adj[t] = 0u;
        wave_lds_sync4();
        for (int p = lane; p < m; p += kWave) {
            const uint32_t w = (uint32_t)hrow[p];
            const int32_t k = (int32_t)(w & a.label_mask);
            int32_t d = dom.delta[0];
#pragma unroll
            for (int t = 1; t < 5; ++t)
                if (k >= dom.lo[t]) d = dom.delta[t];
            pmap[k + d] = (uint16_t)(p + 1);
            {  // hub-relative coordinates (|d| < 2^20)
                const int4 q = a.xyz_s[k];
                rc[p] = make_int4(q.x - pi.x, q.y - pi.y, q.z - pi.z, 0);
            }
            rbin[p] = hbin ? hbin[p] : (uint8_t)(w >> 24);
            if (WT) rw[p] = a.w_s[k];
        }
        const double wi = WT ? a.w_s[i] : 0.0;
        wave_lds_sync4();
        const int32_t hub_hi = hlab(m - 1);

        // local connectivity: for every spoke a of the tile's windows, the row N+(j_a) against
        // the hub map (the rows of the other spokes are not needed: no pair of this tile uses
        // them).  64 spokes at a time: a wave scan lays their rows end to end, and the lanes read
        // the flat range with kConnLoads loads in flight each, so a hub waits for one round of
        // row pointers per 64 spokes rather than one per spoke.
        int32_t *fpre = sw_off;  // flat start of each spoke's row
        const int32_t **fptr = reinterpret_cast<const int32_t **>(eb_off);  // row - flat start
        const int sp_end = min(m - 1, max(p1_hi, p2_hi));
        for (int p0 = p1_lo; p0 < sp_end; p0 += kWave) {
            const int sp = p0 + lane;
            int32_t len = 0;
            const int32_t *row = a.col_1;
            if (sp < sp_end) {
                const bool in1 = sp < p1_hi, in2 = sp >= p2_lo && sp < p2_hi;
                if (in1 || in2) {
                    const int32_t j = hlab(sp);
                    const int64_t jb = a.row_ptr[j];
                    len = (int32_t)(a.row_ptr[j + 1] - jb);
                    row = in1 ? a.col_1 + (jb - (jb >= a.e_split ? a.base_1b : a.base_1))
                              : a.col_2 + (jb - a.base_2);
                }
            }
            const int incl = wave_incl_scan(len, lane);
            const int total = __shfl(incl, kWave - 1, kWave);
            if (total == 0) continue;
            fpre[lane] = incl - len;
            fptr[lane] = row - (incl - len);
            wave_lds_sync4();
            for (int t0 = 0; t0 < total; t0 += kWave * kConnLoads) {
                int32_t kk[kConnLoads], qq[kConnLoads];
#pragma unroll
                for (int u = 0; u < kConnLoads; ++u) {
                    const int t = t0 + u * kWave + lane;
                    kk[u] = INT_MAX;
                    qq[u] = 0;
                    if (t < total) {
                        const int q = last_le(fpre, t);  // the spoke whose row holds t
                        qq[u] = q;
                        kk[u] = (int32_t)((uint32_t)fptr[q][t] & a.label_mask);
                    }
                }
#pragma unroll
                for (int u = 0; u < kConnLoads; ++u) {
                    const int32_t k = kk[u];
                    if (k > hub_hi) continue;  // past the hub's last neighbour (or no element)
                    int32_t d = dom.delta[0], lim = dom.hi[0];
#pragma unroll
                    for (int t = 1; t < 5; ++t)
                        if (k >= dom.lo[t]) { d = dom.delta[t]; lim = dom.hi[t]; }
                    if (k < lim) {
                        const int32_t v = pmap[k + d];
                        if (v) {
                            const int b = v - 1;
                            atomicOr(&adj[(p0 + qq[u]) * W + (b >> 5)], 1u << (b & 31));
                        }
                    }
                }
            }
            wave_lds_sync4();
        }
        wave_lds_sync4();

        // tetrahedra: every local edge (a, b), a in window c1 and b in window c2, with every
        // common bit c of rows a and b.  The work is spread evenly over the lanes: lanes take 64
        // bitset words of rows a and a prefix sum over the wave numbers their edges; lanes take
        // 64 of these edges and count their tetrahedra (a second prefix sum); each lane then
        // walks an equal share of those tetrahedra in order.
        unsigned int my_cl = 0;
        for (int t0 = p1_lo * W; t0 < p1_hi * W; t0 += kWave) {
            const int t = t0 + lane;
            uint32_t bits = 0u;
            if (t < p1_hi * W) {
                const int wa = t % W;
                // positions [p2_lo, p2_hi) of word wa
                const int blo = min(max(p2_lo - wa * 32, 0), 32), bhi = min(max(p2_hi - wa * 32, 0), 32);
                const uint32_t range = (bhi >= 32 ? 0xffffffffu : ((1u << bhi) - 1u)) &
                                       ~(blo >= 32 ? 0xffffffffu : ((1u << blo) - 1u));
                bits = adj[t] & range;
            }
            const int ecnt = __popc(bits);
            const int eincl = wave_incl_scan(ecnt, lane);
            const int ne = __shfl(eincl, kWave - 1, kWave);
            if (ne == 0) continue;
            sw_bits[lane] = bits;
            sw_off[lane] = eincl - ecnt;
            wave_lds_sync4();
            for (int e0 = 0; e0 < ne; e0 += kWave) {
                // edge e0 + lane: (a, b) packed as a | b << 16, and its tetrahedron count (an
                // idle lane holds b = 0xffff, no words, no tetrahedra)
                const int e = e0 + lane;
                uint32_t ab = 0xffff0000u;
                int tcnt = 0;
                if (e < ne) {
                    const int L = last_le(sw_off, e);
                    const int tw = t0 + L, ea = tw / W;
                    const int eb = (tw - ea * W) * 32 + select_bit(sw_bits[L], e - sw_off[L]);
                    ab = (uint32_t)ea | ((uint32_t)eb << 16);
                    for (int w2 = (eb + 1) >> 5; w2 < W; ++w2)
                        tcnt += __popc(adj[ea * W + w2] & adj[eb * W + w2]);
                }
                const int tincl = wave_incl_scan(tcnt, lane);
                const int nt = __shfl(tincl, kWave - 1, kWave);
                eb_ab[lane] = ab;
                eb_off[lane] = tincl - tcnt;
                wave_lds_sync4();
                // this lane's share [kbeg, kend) of the nt tetrahedra, from edge j, word w2, bits cm
                const int kbeg = (int)(((int64_t)lane * nt) >> 6);
                const int kend = (int)(((int64_t)(lane + 1) * nt) >> 6);
                int j = 0, ra = 0, rbb = 0, w2 = 0;
                uint32_t cm = 0u;
                if (kbeg < kend) {
                    j = last_le(eb_off, kbeg);
                    ra = (int)(eb_ab[j] & 0xffffu);
                    rbb = (int)(eb_ab[j] >> 16);
                    int r = kbeg - eb_off[j];
                    w2 = (rbb + 1) >> 5;
                    cm = adj[ra * W + w2] & adj[rbb * W + w2];
                    for (int c = __popc(cm); r >= c && w2 + 1 < W; c = __popc(cm)) {
                        r -= c;
                        ++w2;
                        cm = adj[ra * W + w2] & adj[rbb * W + w2];
                    }
                    cm &= 0xffffffffu << select_bit(cm, r);
                }
                // terms of the pair (a, b), computed when the edge changes: hub-relative
                // coordinates A, B (hub at the origin), the bins of (i, a), (i, b), (a, b),
                // |a - b|^2, X = A x B (exact: products below 2^40) and the parts of the vertex
                // keys that c does not change (integer sums, exact)
                int pj = -1, bia = 0, bib = 0, bab = 0;
                double4 A = make_double4(0, 0, 0, 0), B = A;
                double dab = 0, X0 = 0, X1 = 0, X2 = 0, kab = 0, ka = 0, kb = 0;
                for (int k = kbeg; k < kend; ++k) {
                    if (j != pj) {
                        pj = j;
                        A = rel4(rc[ra]);
                        B = rel4(rc[rbb]);
                        bia = rbin[ra];
                        bib = rbin[rbb];
                        dab = sq3(A.x - B.x, A.y - B.y, A.z - B.z);
                        bab = edge_bin_d(dab, se, bin_half);
                        X0 = fma(A.y, B.z, -(A.z * B.y));
                        X1 = fma(A.z, B.x, -(A.x * B.z));
                        X2 = fma(A.x, B.y, -(A.y * B.x));
                        kab = A.w + B.w;
                        ka = A.w + dab;
                        kb = B.w + dab;
                    }
                    const int rcc = w2 * 32 + __builtin_ctz(cm);
                    const double4 Cc = rel4(rc[rcc]);
                    const double dac = sq3(A.x - Cc.x, A.y - Cc.y, A.z - Cc.z);
                    const double dbc = sq3(B.x - Cc.x, B.y - Cc.y, B.z - Cc.z);
                    // the six bins in edge order of the vertices (i, a, b, c)
                    int bb[6] = {bia, bib, rbin[rcc], bab, edge_bin_d(dac, se, bin_half),
                                 edge_bin_d(dbc, se, bin_half)};
                    // the configuration: its rank, with the cache's slot in the S4 table's high
                    // bits (taken apart only below, so the table read overlaps the geometry)
                    uint32_t packed = 0;
                    if (a.s4rank) {  // S4 configuration: one table read
                        int key = 0;
#pragma unroll
                        for (int q = 0; q < 6; ++q) key = key * a.nb + bb[q];
                        packed = a.s4rank[key];
                    } else {  // sorted 6-tuple: sorting network, one rank-table entry per position
                        cswap(bb[1], bb[2]); cswap(bb[4], bb[5]); cswap(bb[0], bb[2]);
                        cswap(bb[3], bb[5]); cswap(bb[0], bb[1]); cswap(bb[3], bb[4]);
                        cswap(bb[1], bb[4]); cswap(bb[0], bb[3]); cswap(bb[2], bb[5]);
                        cswap(bb[1], bb[3]); cswap(bb[2], bb[4]); cswap(bb[2], bb[3]);
                        int r = 0;
#pragma unroll
                        for (int q = 0; q < 6; ++q) r += rtab[q * GTC_MAX_BINS_4PCF + bb[q]];
                        packed = (uint32_t)r;
                    }
                    // vertex keys (sums of the three squared edge lengths, exact) of i, a, b,
                    // c; sorting them ascending permutes the vertices, and the orientation of
                    // the sorted tetrahedron is the parity of that permutation (the parity of its
                    // inversions) times orient(i, a, b, c) = C . (A x B); a tie leaves no
                    // handedness
                    const double k0 = kab + Cc.w, k1 = ka + dac, k2 = kb + dbc, k3 = Cc.w + dac + dbc;
                    const bool tie = k0 == k1 || k0 == k2 || k0 == k3 || k1 == k2 || k1 == k3 ||
                                     k2 == k3;
                    const bool par = (k0 > k1) ^ (k0 > k2) ^ (k0 > k3) ^ (k1 > k2) ^ (k1 > k3) ^
                                     (k2 > k3);
                    int sgn = 0;
                    if (!tie) {
                        const int o = orient_sign(Cc, X0, X1, X2);
                        sgn = par ? -o : o;
                    }
                    double qv = 0.0;
                    if (WT) {  // the four weights ascending, product without fusion
                        double v0 = wi, v1 = rw[ra], v2 = rw[rbb], v3 = rw[rcc], t;
                        t = fmin(v0, v1); v1 = fmax(v0, v1); v0 = t;
                        t = fmin(v2, v3); v3 = fmax(v2, v3); v2 = t;
                        t = fmin(v0, v2); v2 = fmax(v0, v2); v0 = t;
                        t = fmin(v1, v3); v3 = fmax(v1, v3); v1 = t;
                        t = fmin(v1, v2); v2 = fmax(v1, v2); v1 = t;
                        const double pr = __dmul_rn(__dmul_rn(__dmul_rn(v0, v1), v2), v3);
                        qv = rint(__dmul_rn(pr, a.two_s));  // exact, |qv| < 2^57
                    }
                    const int rank = sir ? (int)(packed & kRankMask) : (int)packed;
                    // the configuration's LDS slot (WM 3: -1 when it is not cached)
                    const int sl = WM == 3 ? (sir ? (int)(packed >> kSlotShift) - 1 : (int)slot16[rank])
                                           : rank;
                    if (WT) {
                        const int cls = sgn > 0 ? 0 : (sgn < 0 ? 1 : 2);
                        const int idx = 3 * rank + cls;
                        if (WM == 3 && sl >= 0) {
                            add_i128(wl + 4 * sl, (long long)qv);
                            if (sgn) add_i128(wl + 4 * sl + 2, (long long)(sgn > 0 ? qv : -qv));
                        } else if (WM == 2) {
                            add_i128(wl + 2 * (3 * sl + cls), (long long)qv);
                        } else {
                            if (idx != pend) {
                                if (pend >= 0) add_u128_pair(wg + 2 * pend, plo, phi);
                                pend = idx;
                                plo = 0ull;
                                phi = 0ull;
                            }
                            const unsigned long long u = (unsigned long long)(long long)qv;
                            const unsigned long long n0 = plo + u;
                            phi += (qv < 0.0 ? ~0ull : 0ull) + (n0 < plo ? 1ull : 0ull);
                            plo = n0;
                        }
                    }
                    if (GH || (WM == 3 && sl < 0)) {
                        atomicAdd(&a.even[rank], 1ull);
                        if (sgn) atomicAdd(&a.odd[rank], (unsigned long long)(long long)sgn);
                    } else {
                        atomicAdd(&ev[sl], 1u);
                        if (sgn) atomicAdd(&od[sl], sgn);
                    }
                    ++my_cl;
                    // the next tetrahedron: next bit, word or edge (the counts promise one while
                    // k + 1 < kend; the bound on j only guards the scratch)
                    cm &= cm - 1u;
                    if (k + 1 < kend) {
                        while (!cm) {
                            if (++w2 >= W) {
                                do {
                                    ++j;
                                    ra = (int)(eb_ab[j] & 0xffffu);
                                    rbb = (int)(eb_ab[j] >> 16);
                                    w2 = (rbb + 1) >> 5;
                                } while (w2 >= W && j < kWave - 1);
                                if (w2 >= W) break;
                            }
                            cm = adj[ra * W + w2] & adj[rbb * W + w2];
                        }
                        if (!cm) break;
                    }
                }
                wave_lds_sync4();
            }
        }
        unsigned int tot = my_cl;
#pragma unroll
        for (int dd = kWave / 2; dd > 0; dd >>= 1) tot += __shfl_xor(tot, dd, kWave);
        wave_cl += tot;
        if (!GH && wave_cl >= a.flush_at) {
            for (int t = lane; t < nslot; t += kWave) {
                const int r = WM == 3 ? rank_of[t] : t;
                const uint32_t v = atomicExch(&ev[t], 0u);
                if (v) atomicAdd(&a.even[r], (unsigned long long)v);
                const int32_t o = atomicExch(&od[t], 0);
                if (o) atomicAdd(&a.odd[r], (unsigned long long)(long long)o);
            }
            wave_cl = 0;
        }
        wave_lds_sync4();
    }
    if ((WM == 1 || WM == 3) && pend >= 0) add_u128_pair(wg + 2 * pend, plo, phi);
    if (GH) return;
    __syncthreads();
    for (int t = threadIdx.x; t < nslot; t += blockDim.x) {
        const int r = WM == 3 ? rank_of[t] : t;
        const uint32_t v = ev[t];
        if (v) atomicAdd(&a.even[r], (unsigned long long)v);
        const int32_t o = od[t];
        if (o) atomicAdd(&a.odd[r], (unsigned long long)(long long)o);
    }
    if (WM == 2)
        for (int t = threadIdx.x; t < 3 * nslot; t += blockDim.x) {
            const unsigned long long lo = wl[2 * t], hi = wl[2 * t + 1];
            if (lo | hi) add_u128_pair(wg + 2 * t, lo, hi);
        }
    if (WM == 3)  // (E, O) of a slot goes in as A+ += O, A0 += E - O: the same even and odd sums
        for (int t = threadIdx.x; t < nslot; t += blockDim.x) {
            const unsigned long long e0 = wl[4 * t], e1 = wl[4 * t + 1];
            const unsigned long long o0 = wl[4 * t + 2], o1 = wl[4 * t + 3];
            const unsigned long long d0 = e0 - o0, d1 = e1 - o1 - (e0 < o0 ? 1ull : 0ull);
            const int w = 3 * rank_of[t];
            if (o0 | o1) add_u128_pair(wg + 2 * w, o0, o1);
            if (d0 | d1) add_u128_pair(wg + 2 * (w + 2), d0, d1);
        }
}

// ------------------------------------------------------------------ S4 configurations (§III.3)
// A tetrahedron's six edge bins in the edge order (01, 02, 03, 12, 13, 23) of its vertices, up to
// the 24 relabellings of the vertices; a relabelling p moves the bin of edge (u, v) to edge
// (p(u), p(v)).  The canonical tuple is the smallest relabelling; as base-nb keys with edge 01 most
// significant keep lexicographic order, it is the relabelling with the smallest key.
__host__ __device__ inline int s4_edge(int u, int v) {
    const int lo = u < v ? u : v, hi = u < v ? v : u;
    return lo == 0 ? hi - 1 : lo + hi;  // 01->0 02->1 03->2 12->3 13->4 23->5
}

__host__ __device__ inline uint32_t s4_canonical_key(uint32_t key, int nb) {
    int t[6];
    for (int e = 5; e >= 0; --e) {
        t[e] = (int)(key % (uint32_t)nb);
        key /= (uint32_t)nb;
    }
    constexpr int eu[6] = {0, 0, 0, 1, 1, 2}, ev[6] = {1, 2, 3, 2, 3, 3};
    uint32_t best = 0xffffffffu;
    for (int perm = 0; perm < 24; ++perm) {  // perm -> a permutation of {0,1,2,3} (factorial base)
        int p[4] = {0, 1, 2, 3};
        int code = perm;
        for (int k = 0; k < 3; ++k) {
            const int span = 4 - k, j = k + code % span;
            code /= span;
            const int tmp = p[k];
            p[k] = p[j];
            p[j] = tmp;
        }
        int r[6];
        for (int e = 0; e < 6; ++e) r[s4_edge(p[eu[e]], p[ev[e]])] = t[e];
        uint32_t k2 = 0;
        for (int e = 0; e < 6; ++e) k2 = k2 * (uint32_t)nb + (uint32_t)r[e];
        best = k2 < best ? k2 : best;
    }
    return best;
}

int64_t num_s4_keys(int nb) {
    int64_t k = 1;
    for (int e = 0; e < 6; ++e) k *= nb;
    return k;
}

__global__ void k_s4_canon(uint32_t nkeys, int nb, uint32_t *__restrict__ canon,
                           int32_t *__restrict__ is_canon) {
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nkeys) return;
    const uint32_t c = s4_canonical_key(t, nb);
    canon[t] = c;
    is_canon[t] = c == t;
}

__global__ void k_s4_rank(uint32_t nkeys, const int32_t *__restrict__ canon_rank,
                          uint32_t *__restrict__ canon /* in: canonical key, out: rank */) {
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < nkeys) canon[t] = (uint32_t)canon_rank[canon[t]];
}

// rank[key] for every base-nb 6-tuple key: the number of canonical keys below its canonical key
static int s4_rank_table(int nb, uint32_t *rank, int32_t *flags, int32_t *scan, void *ws,
                         hipStream_t s) {
    const int64_t nk = num_s4_keys(nb);
    const unsigned blocks = (unsigned)((nk + 255) / 256);
    hipLaunchKernelGGL(k_s4_canon, dim3(blocks), dim3(256), 0, s, (uint32_t)nk, nb, rank, flags);
    GTC_HIP_CHECK(hipGetLastError());
    GTC_TRY(exclusive_scan_i32_to_i32(flags, scan, nk, ws, s));
    hipLaunchKernelGGL(k_s4_rank, dim3(blocks), dim3(256), 0, s, (uint32_t)nk, scan, rank);
    GTC_HIP_CHECK(hipGetLastError());
    return GTC_OK;
}

int64_t num_configs_s4(int nb) {
    const int64_t k = nb;
    return (k * k * k * k * k * k + 9 * k * k * k * k + 14 * k * k) / 24;  // Burnside over S4
}

// true when no relabelling of the key's tuple gives a smaller key (the canonical tuple); most
// keys meet a smaller relabelling within the first few, so the loop stops early
static bool s4_is_canonical(uint32_t key, int nb) {
    int t[6];
    uint32_t k = key;
    for (int e = 5; e >= 0; --e) {
        t[e] = (int)(k % (uint32_t)nb);
        k /= (uint32_t)nb;
    }
    constexpr int eu[6] = {0, 0, 0, 1, 1, 2}, ev[6] = {1, 2, 3, 2, 3, 3};
    for (int perm = 1; perm < 24; ++perm) {  // perm 0 is the identity
        int p[4] = {0, 1, 2, 3};
        int code = perm;
        for (int q = 0; q < 3; ++q) {
            const int span = 4 - q, j = q + code % span;
            code /= span;
            const int tmp = p[q];
            p[q] = p[j];
            p[j] = tmp;
        }
        int r[6];
        for (int e = 0; e < 6; ++e) r[s4_edge(p[eu[e]], p[ev[e]])] = t[e];
        uint32_t k2 = 0;
        for (int e = 0; e < 6; ++e) k2 = k2 * (uint32_t)nb + (uint32_t)r[e];
        if (k2 < key) return false;
    }
    return true;
}

// canonical tuples in rank order (host), computed once per bin count and process: the canonical
// test runs on all hardware threads, the tables are kept for later calls
void config_bins_s4(int nb, int32_t *bins) {
    static std::mutex mu;
    static std::map<int, std::vector<int32_t>> done;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = done.find(nb);
        if (it != done.end()) {
            std::copy(it->second.begin(), it->second.end(), bins);
            return;
        }
    }
    const int64_t nk = num_s4_keys(nb);
    std::vector<uint8_t> canon(nk);
    const int nt = std::max(1u, std::min(32u, std::thread::hardware_concurrency()));
    std::vector<std::thread> pool;
    for (int t = 0; t < nt; ++t)
        pool.emplace_back([&, t]() {
            for (int64_t key = t; key < nk; key += nt) canon[key] = s4_is_canonical((uint32_t)key, nb);
        });
    for (auto &th : pool) th.join();
    std::vector<int32_t> table(6 * (size_t)num_configs_s4(nb));
    int64_t r = 0;
    for (int64_t key = 0; key < nk; ++key) {
        if (!canon[key]) continue;
        int64_t k2 = key;
        for (int e = 5; e >= 0; --e) {
            table[6 * r + e] = (int32_t)(k2 % nb);
            k2 /= nb;
        }
        ++r;
    }
    std::copy(table.begin(), table.end(), bins);
    std::lock_guard<std::mutex> lock(mu);
    done.emplace(nb, std::move(table));
}

// Cayley-Menger: 288 V^2 of the tetrahedron with squared edges d (5x5 bordered determinant by
// elimination with partial pivoting), and 16 A^2 of the triangle with squared sides a, b, c
static long double cm_volume(long double d[4][4]) {
    long double m[5][5];
    for (int i = 0; i < 5; ++i)
        for (int j = 0; j < 5; ++j)
            m[i][j] = (i == 0 || j == 0) ? (i == j ? 0.0L : 1.0L) : d[i - 1][j - 1];
    long double det = 1.0L;
    for (int c = 0; c < 5; ++c) {
        int piv = c;
        for (int r = c + 1; r < 5; ++r)
            if (std::fabs(m[r][c]) > std::fabs(m[piv][c])) piv = r;
        if (m[piv][c] == 0.0L) return 0.0L;
        if (piv != c) {
            for (int k = 0; k < 5; ++k) std::swap(m[c][k], m[piv][k]);
            det = -det;
        }
        det *= m[c][c];
        for (int r = c + 1; r < 5; ++r) {
            const long double f = m[r][c] / m[c][c];
            for (int k = c; k < 5; ++k) m[r][k] -= f * m[c][k];
        }
    }
    return det;
}

void config_realizable_s4(int nb, const int64_t *edges, uint8_t *mask) {
    std::vector<int32_t> bins(6 * num_configs_s4(nb));
    config_bins_s4(nb, bins.data());
    constexpr int eu[6] = {0, 0, 0, 1, 1, 2}, ev[6] = {1, 2, 3, 2, 3, 3};
    for (int64_t c = 0; c < num_configs_s4(nb); ++c) {
        long double d[4][4] = {};
        for (int e = 0; e < 6; ++e) {
            const int b = bins[6 * c + e];
            const long double r = 0.5L * (std::sqrt((long double)edges[b]) +
                                          std::sqrt((long double)edges[b + 1]));
            d[eu[e]][ev[e]] = d[ev[e]][eu[e]] = r * r;
        }
        bool ok = cm_volume(d) > 0.0L;
        for (int f = 0; f < 4 && ok; ++f) {  // the face opposite vertex f
            int u[3], k = 0;
            for (int q = 0; q < 4; ++q)
                if (q != f) u[k++] = q;
            const long double x = d[u[0]][u[1]], y = d[u[1]][u[2]], z = d[u[0]][u[2]];
            ok = 2 * x * y + 2 * y * z + 2 * z * x - x * x - y * y - z * z > 0.0L;
        }
        mask[c] = ok ? 1 : 0;
    }
}

int gather_weights(const gtc_graph_s *G, const double *d_w, double *w_s, unsigned long long *d_m,
                   int32_t *d_bad, double *maxabs, hipStream_t s);

// Copies of the global class sums: a few hot configurations take most tetrahedra, and their
// global atomics serialise; workgroup b adds to copy b % copies (a multiple of the 8 XCDs, so each
// copy stays in the L2 of one XCD), within a 256 MiB budget.
// out[t] = hubs[t * stride] for t < ceil(n / stride): a sample that keeps the class order
__global__ void k_every_nth(const int32_t *__restrict__ hubs, int64_t n, int stride,
                            int32_t *__restrict__ out) {
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (t * stride < n) out[t] = hubs[t * stride];
}

// s4rank[key] |= (slot[rank] + 1) << kSlotShift for the cached configurations
__global__ void k_s4_attach_slots(uint32_t *__restrict__ s4rank, int64_t nkeys,
                                  const int16_t *__restrict__ slot) {
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (t >= nkeys) return;
    const uint32_t r = s4rank[t] & kRankMask;
    const int sl = slot[r];
    if (sl >= 0) s4rank[t] = r | ((uint32_t)(sl + 1) << kSlotShift);
}

static int weighted_copies(int64_t ncfg) {
    const int64_t per_copy = 48 * ncfg;  // [ncfg][3] 128-bit words
    int64_t c = std::min<int64_t>(256, std::max<int64_t>(1, ((int64_t)256 << 20) / per_copy));
    if (c >= 8) c &= ~(int64_t)7;
    return (int)c;
}

int count_4pcf_device(gtc_graph_s *G, uint64_t *d_even, int64_t *d_odd, gtc_stats *st,
                      hipStream_t s, bool s4, const double *d_w, double *d_even_w,
                      double *d_odd_w) {
    const bool WT = d_w != nullptr;
    const int64_t ncfg = s4 ? num_configs_s4(G->nb) : gtc_num_configs(4, G->nb);
    GTC_TRY(fill_u64(d_even, ncfg, 0ull, s));
    GTC_TRY(fill_u64(reinterpret_cast<uint64_t *>(d_odd), ncfg, 0ull, s));
    if (G->max_deg >= 65535) {
        set_error("4pCF: a forward row of %lld entries exceeds the 16-bit position map",
                  (long long)G->max_deg);
        return GTC_E_UNSUPPORTED;
    }
    CliqueArgs a{};
    a.row_ptr = G->row_ptr;
    // resident: one tile with every window the whole CSR (out-of-core graphs set these per tile)
    a.col_h = a.col_1 = a.col_2 = G->col;
    a.bin_h = a.bin_1 = a.bin_2 = G->bin;
    a.base_h = a.base_1 = a.base_2 = 0;
    a.e_split = INT64_MAX;
    a.base_1b = 0;
    a.w1_lo = a.w2_lo = 0;
    a.w1_hi = a.w2_hi = (int32_t)G->n;
    a.tiled = 0;
    a.label_mask = G->packed ? kLabelMask : 0xffffffffu;
    a.hubs = G->hubs;
    a.n_hubs = (int32_t)G->n_hubs;
    a.nb = G->nb;
    a.ncfg = (int32_t)ncfg;
    a.map_bytes = (int32_t)align16(2 * (size_t)std::max<int64_t>(G->max_domain, 1));
    a.max_m = (int32_t)std::max<int64_t>(G->max_deg, 1);
    a.words = (a.max_m + 31) / 32;
    a.xyz_s = G->xyz_s;
    a.cell_start = G->cell_start;
    a.gr = G->grid;
    a.even = reinterpret_cast<unsigned long long *>(d_even);
    a.odd = reinterpret_cast<unsigned long long *>(d_odd);

    int dev = 0, cus = 0, ldsmax = 0;
    GTC_HIP_CHECK(hipGetDevice(&dev));
    GTC_HIP_CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    GTC_HIP_CHECK(hipDeviceGetAttribute(&ldsmax, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
    // LDS bins while they leave room for two waves' hub data (global atomics per tetrahedron cost
    // several times the occupancy the histogram takes)
    // (weighted: the class sums too, in LDS on the same terms, else in global memory)
    const size_t static_lds0 = sizeof(int64_t) * (GTC_MAX_BINS_4PCF + 1);
    const size_t per = clique_lds_wave(a.map_bytes, a.max_m, a.words, WT);
    const bool WL = WT && static_lds0 + clique_lds_fixed(a.ncfg, false, true) + 2 * per <= (size_t)ldsmax;
    const bool GH = static_lds0 + clique_lds_fixed(a.ncfg, false) + 2 * per > (size_t)ldsmax;
    // Weighted sums too large for LDS, on a resident graph: an LDS cache for the configurations
    // that an unweighted pass over every kCacheStride-th hub finds most frequent (the rest go to
    // global memory).  The slot count fills the LDS left beside 8 (else 4) waves of hub data.
    const size_t fixed_u = clique_lds_fixed(a.ncfg, false);
    const size_t per_u = clique_lds_wave(a.map_bytes, a.max_m, a.words, false);
    int cache_k = 0, cache_waves = 0;
    bool cache_ok = WT && !WL && !GH && !G->windowed() && G->n_hubs > 0 &&
                    static_lds0 + fixed_u + per_u <= (size_t)ldsmax;
    if (const char *env = std::getenv("GTC_CONFIG_CACHE"))  // "off": global sums only (tests)
        if (std::strcmp(env, "off") == 0) cache_ok = false;
    // GTC_CACHE_WAVES=w: waves per workgroup beside the cache (default 10, else 5; fewer waves
    // leave room for more cached configurations, whose tetrahedra then add in LDS)
    int w_first = 10;
    if (const char *env = std::getenv("GTC_CACHE_WAVES"))
        w_first = std::max(1, std::min(16, std::atoi(env)));
    if (cache_ok)
        for (int w = w_first; w >= std::min(4, w_first) && !cache_k; w >>= 1) {
            const size_t used = static_lds0 + (size_t)w * per + 4 * kRankTab +
                                (s4 ? 0 : align16(2 * (size_t)ncfg));
            if (used >= (size_t)ldsmax) continue;
            int64_t k = std::min<int64_t>({ncfg, (int64_t)(s4 ? kMaxTableSlots : 32767),
                                           (int64_t)((ldsmax - used) / 44)});
            while (k > 0 && static_lds0 + clique_lds_fixed(a.ncfg, false, false, (int)k, !s4) + w * per >
                                (size_t)ldsmax)
                --k;
            if (k >= kCacheMin) {
                cache_k = (int)k;
                cache_waves = w;
            }
        }
    size_t fixed = cache_k ? clique_lds_fixed(a.ncfg, false, false, cache_k, !s4)
                           : clique_lds_fixed(a.ncfg, GH, WL);
    // Workgroups of 4 waves; a large LDS histogram (S4 configurations) allows one workgroup per
    // CU, which then takes as many waves (up to 16) as the LDS beside the histogram holds.
    const size_t static_lds = sizeof(int64_t) * (GTC_MAX_BINS_4PCF + 1);
    int waves = 4;
    if (!GH && fixed > (size_t)ldsmax / 2)
        waves = (int)std::min<size_t>(16, (ldsmax - static_lds - fixed) / std::max<size_t>(per, 1));
    while (waves > 1 && static_lds + fixed + waves * per > (size_t)ldsmax) waves >>= 1;
    if (waves < 1) waves = 1;
    if (cache_k) waves = cache_waves;
    size_t lds = fixed + waves * per;
    if (static_lds + lds > (size_t)ldsmax) {
        set_error("4pCF needs %zu bytes of LDS per workgroup (longest row %d, hub domain %d); the "
                  "device allows %d", lds, a.max_m, a.map_bytes / 2, ldsmax);
        return GTC_E_UNSUPPORTED;
    }
    const unsigned long long mm = (unsigned long long)a.max_m;
    const unsigned long long max_hub = mm * (mm - 1) * (mm - 2) / 6;
    const unsigned long long budget = 0x7fffffffull / (unsigned long long)waves;
    if (!GH && max_hub >= budget / 2) {
        set_error("4pCF: a hub with %d forward neighbours could overflow the 32-bit LDS bins", a.max_m);
        return GTC_E_UNSUPPORTED;
    }
    a.flush_at = GH ? 0u : (unsigned int)(budget - max_hub);
    // GTC_CLIQUE_FLUSH_AT=n drains the LDS count bins at least every n tetrahedra of a
    // wave
    if (const char *env = std::getenv("GTC_CLIQUE_FLUSH_AT")) {
        const long long v = std::atoll(env);
        if (!GH && v > 0 && (unsigned long long)v < a.flush_at) a.flush_at = (unsigned int)v;
    }

    unsigned int *queue = nullptr, *qcount = nullptr;
    uint32_t *s4rank = nullptr;
    int32_t *s4flags = nullptr, *s4scan = nullptr;
    int64_t *s4ws = nullptr;
    double *w_s = nullptr;
    unsigned long long *wsum = nullptr, *d_maxabs = nullptr;
    int32_t *d_bad = nullptr;
    int32_t *cache_hubs = nullptr, *cache_rank = nullptr;
    int16_t *cache_slot = nullptr;
    unsigned long long *cache_even = nullptr, *cache_odd = nullptr;
    const int64_t cache_ns = cache_k ? (G->n_hubs + kCacheStride - 1) / kCacheStride : 0;
    void *scratch = nullptr;
    const int64_t nkeys = s4 ? num_s4_keys(G->nb) : 0;
    const int copies = WT ? weighted_copies(ncfg) : 0;
    // out-of-core graphs (§III.5.3): three window buffers, for the hub window and the two search
    // windows of a tile
    const bool tiled = G->windowed();
    constexpr int kSlots = 3;
    int32_t *wcol[kSlots] = {nullptr, nullptr, nullptr};
    uint8_t *wbin[kSlots] = {nullptr, nullptr, nullptr};
    unsigned int *queue2 = nullptr, *qcount2 = nullptr;  // the second stream's launches (tiles)
    GTC_TRY(carve_alloc(&scratch, s, [&](Carver &c) {
        c.take(&queue, (size_t)kQueueWords);
        c.take(&qcount, kHubClasses);
        if (tiled) {
            c.take(&queue2, (size_t)kQueueWords);
            c.take(&qcount2, kHubClasses);
        }
        if (tiled)
            for (int k = 0; k < kSlots; ++k) {
                c.take(&wcol[k], std::max<int64_t>(G->max_window_edges, 1));
                if (!G->packed) c.take(&wbin[k], std::max<int64_t>(G->max_window_edges, 1));
            }
        if (cache_k) {
            c.take(&cache_hubs, cache_ns);
            c.take(&cache_even, ncfg);
            c.take(&cache_odd, ncfg);
            c.take(&cache_slot, ncfg);
            c.take(&cache_rank, cache_k);
        }
        if (WT) {
            c.take(&w_s, G->n);
            c.take(&wsum, 6 * (size_t)ncfg * copies);
            c.take(&d_maxabs, 1);
            c.take(&d_bad, 1);
        }
        if (s4) {
            c.take(&s4rank, nkeys);
            c.take(&s4flags, nkeys);
            c.take(&s4scan, nkeys + 1);
            c.take(&s4ws, scan_workspace_bytes(nkeys) / sizeof(int64_t));
        }
    }));
    int rc = fill_u32(queue, kQueueWords, 0u, s);
    if (!rc && s4) rc = s4_rank_table(G->nb, s4rank, s4flags, s4scan, s4ws, s);
    int scale = 0;
    if (!rc && WT) {
        double maxabs = 0.0;
        rc = gather_weights(G, d_w, w_s, d_maxabs, d_bad, &maxabs, s);
        if (!rc) rc = weight_scale(maxabs, 4, &scale);
        if (!rc) rc = fill_u64(reinterpret_cast<uint64_t *>(wsum), 6 * ncfg * copies, 0ull, s);
    }
    a.w_s = w_s;
    a.two_s = std::ldexp(1.0, scale);
    a.wsum = wsum;
    a.wcopies = copies;
    a.wstride = 6 * ncfg;
    a.s4rank = s4rank;
    a.queue = queue;
    a.qcount = qcount;
    std::vector<hipEvent_t> kev;  // start / end of every launch
    float kms = 0.f;
    int32_t launched_blocks = 0;
    int64_t tiles_run = 0;
    const void *kfn = nullptr;
    int64_t max_blocks = 1;
    // configuration cache: the unweighted pass over the sampled hubs, then slots for the most
    // frequent configurations it met (at least one slot, so the layout stays the sized one)
    if (!rc && cache_k) {
        CliqueArgs pa = a;
        const int wu = (int)std::max<size_t>(
            1, std::min<size_t>(16, (ldsmax - static_lds - fixed_u) / std::max<size_t>(per_u, 1)));
        const unsigned long long budget_u = 0x7fffffffull / (unsigned long long)wu;
        const size_t lds_u = fixed_u + (size_t)wu * per_u;
        const void *kfu = reinterpret_cast<const void *>(&k_clique4<false, 0>);
        rc = fill_u64(reinterpret_cast<uint64_t *>(cache_even), ncfg, 0ull, s);
        if (!rc) rc = fill_u64(reinterpret_cast<uint64_t *>(cache_odd), ncfg, 0ull, s);
        if (!rc) {
            hipLaunchKernelGGL(k_every_nth, dim3((unsigned)((cache_ns + 255) / 256)), dim3(256), 0, s,
                               G->hubs, (int64_t)G->n_hubs, kCacheStride, cache_hubs);
            rc = hipGetLastError() == hipSuccess ? GTC_OK : GTC_E_HIP;
        }
        if (!rc) rc = hub_class_counts(cache_hubs, cache_ns, G->row_ptr, G->work, qcount, s);
        if (!rc) rc = fill_u32(queue, kQueueWords, 0u, s);
        if (!rc && max_hub < budget_u / 2) {
            pa.even = cache_even;
            pa.odd = cache_odd;
            pa.hubs = cache_hubs;
            pa.n_hubs = (int32_t)cache_ns;
            pa.batch_cap = 1;
            pa.flush_at = (unsigned int)(budget_u - max_hub);
            pa.cache_k = 0;
            if (lds_u > 65536)
                (void)hipFuncSetAttribute(kfu, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_u);
            int pcu = 0;
            (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&pcu, kfu, wu * kWave, lds_u);
            const int64_t blocks_u = std::min<int64_t>((int64_t)cus * std::max(pcu, 1), (cache_ns + wu - 1) / wu);
            const int64_t *edges_dev = G->d_edges;
            void *args[] = {&pa, &edges_dev};
            hipEvent_t e0 = nullptr, e1 = nullptr;  // timed with the count's launches
            hipError_t e = hipEventCreate(&e0);
            if (e == hipSuccess) kev.push_back(e0);
            if (e == hipSuccess) e = hipEventCreate(&e1);
            if (e == hipSuccess) kev.push_back(e1);
            if (e == hipSuccess) e = hipEventRecord(e0, s);
            if (e == hipSuccess)
                e = hipLaunchKernel(kfu, dim3((unsigned)std::max<int64_t>(blocks_u, 1)),
                                    dim3(wu * kWave), args, lds_u, s);
            if (e == hipSuccess) e = hipGetLastError();
            if (e == hipSuccess) e = hipEventRecord(e1, s);
            if (e != hipSuccess) rc = hip_fail(e, "k_clique4 sample launch", __FILE__, __LINE__);
        }
        std::vector<unsigned long long> hc(ncfg, 0ull);
        if (!rc) {
            hipError_t e = hipMemcpyAsync(hc.data(), cache_even, 8 * ncfg, hipMemcpyDeviceToHost, s);
            if (e == hipSuccess) e = hipStreamSynchronize(s);
            if (e != hipSuccess) rc = hip_fail(e, "4pCF sample readback", __FILE__, __LINE__);
        }
        if (!rc) {
            std::vector<int32_t> order(ncfg);
            for (int64_t c = 0; c < ncfg; ++c) order[c] = (int32_t)c;
            const int64_t hot = std::count_if(hc.begin(), hc.end(), [](unsigned long long v) { return v > 0; });
            cache_k = (int)std::max<int64_t>(1, std::min<int64_t>(cache_k, hot));
            std::partial_sort(order.begin(), order.begin() + cache_k, order.end(),
                              [&](int32_t x, int32_t y) { return hc[x] != hc[y] ? hc[x] > hc[y] : x < y; });
            std::vector<int16_t> slot(ncfg, (int16_t)-1);
            for (int k = 0; k < cache_k; ++k) slot[order[k]] = (int16_t)k;
            hipError_t e = hipMemcpyAsync(cache_slot, slot.data(), 2 * ncfg, hipMemcpyHostToDevice, s);
            if (e == hipSuccess)
                e = hipMemcpyAsync(cache_rank, order.data(), 4 * (size_t)cache_k, hipMemcpyHostToDevice, s);
            if (e == hipSuccess && s4) {  // the slots into the rank table
                hipLaunchKernelGGL(k_s4_attach_slots, dim3((unsigned)((nkeys + 255) / 256)), dim3(256),
                                   0, s, s4rank, (int64_t)nkeys, cache_slot);
                e = hipGetLastError();
            }
            if (e == hipSuccess) e = hipStreamSynchronize(s);  // the host vectors go out of scope
            if (e != hipSuccess) rc = hip_fail(e, "4pCF cache tables", __FILE__, __LINE__);
            fixed = clique_lds_fixed(a.ncfg, false, false, cache_k, !s4);
            a.slot_in_rank = s4 ? 1 : 0;
            lds = fixed + waves * per;
            a.cache_k = cache_k;
            a.cache_slot = cache_slot;
            a.cache_rank = cache_rank;
        }
    }
    if (!rc && G->n_hubs > 0) {
#define GTC_K4(G_, W_) reinterpret_cast<const void *>(&k_clique4<G_, W_>)
        kfn = GH ? (WT ? GTC_K4(true, 1) : GTC_K4(true, 0))
                 : (cache_k ? GTC_K4(false, 3)
                            : (WL ? GTC_K4(false, 2) : (WT ? GTC_K4(false, 1) : GTC_K4(false, 0))));
#undef GTC_K4
        if (lds > 65536)
            (void)hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        int per_cu = 0;
        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, waves * kWave, lds);
        if (per_cu < 1) per_cu = 1;
        max_blocks = (int64_t)cus * per_cu;
    }
    // one launch over the hub list hubs[0, nh): one hub per take (a hub's 4-clique work grows like
    // the cube of its row, which the spoke-element classes predict poorly, and the takes, a few
    // thousand per ms, are far below what one counter serves)
    // (on stream st with the queue counters q, qc; by default the counting stream's)
    auto launch = [&](const int32_t *hubs, int64_t nh, hipStream_t st = nullptr,
                      unsigned int *q = nullptr, unsigned int *qc = nullptr) -> int {
        if (nh <= 0) return GTC_OK;
        if (!st) {
            st = s;
            q = queue;
            qc = qcount;
        }
        GTC_TRY(hub_class_counts(hubs, nh, G->row_ptr, G->work, qc, st));
        GTC_TRY(fill_u32(q, kQueueWords, 0u, st));
        a.queue = q;
        a.qcount = qc;
        a.hubs = hubs;
        a.n_hubs = (int32_t)nh;
        a.batch_cap = 1;
        const int64_t blocks = std::min<int64_t>(max_blocks, (nh + waves - 1) / waves);
        const dim3 grid((unsigned)std::max<int64_t>(blocks, 1)), block(waves * kWave);
        launched_blocks = std::max<int32_t>(launched_blocks, (int32_t)grid.x);
        hipEvent_t e0 = nullptr, e1 = nullptr;
        GTC_HIP_CHECK(hipEventCreate(&e0));
        kev.push_back(e0);
        GTC_HIP_CHECK(hipEventCreate(&e1));
        kev.push_back(e1);
        GTC_HIP_CHECK(hipEventRecord(e0, st));
        const int64_t *edges_dev = G->d_edges;
        void *args[] = {&a, &edges_dev};
        hipError_t e = hipLaunchKernel(kfn, grid, block, args, lds, st);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "k_clique4 launch", __FILE__, __LINE__);
        GTC_HIP_CHECK(hipEventRecord(e1, st));
        ++tiles_run;
        return GTC_OK;
    };
    if (!rc && G->n_hubs > 0 && !tiled) rc = launch(G->hubs, G->n_hubs);
    // Out of core, when every hub window's spokes reach no further than the next window: one
    // launch per hub window (windows h and h + 1), on two streams in turn, so that a launch's
    // last hubs overlap the next launch.  Two launches in flight hold at most three windows (h - 1,
    // h, h + 1), the three buffers.  A buffer is refilled (on the stream of the launch that needs
    // it) after every launch that read it, on either stream; a launch waits for its windows.
    bool two_streams = !rc && G->n_hubs > 0 && tiled;
    const int64_t nwin = (int64_t)G->win.size() - 1;
    for (int64_t h = 0; two_streams && h < nwin; ++h)
        if (G->win_hubs[h + 1] > G->win_hubs[h] && G->win_smax[h] > h + 1) two_streams = false;
    if (two_streams) {
        hipStream_t s2 = nullptr;
        hipEvent_t ev_start = nullptr, ev_end2 = nullptr, ready[kSlots] = {}, done[kSlots][2] = {};
        bool done_set[kSlots][2] = {};
        int64_t slot_win[kSlots] = {-1, -1, -1}, slot_used[kSlots] = {0, 0, 0}, clock = 0;
        auto two = [&]() -> int {
            GTC_HIP_CHECK(hipStreamCreateWithFlags(&s2, hipStreamNonBlocking));
            GTC_HIP_CHECK(hipEventCreateWithFlags(&ev_start, hipEventDisableTiming));
            GTC_HIP_CHECK(hipEventCreateWithFlags(&ev_end2, hipEventDisableTiming));
            for (int k = 0; k < kSlots; ++k) {
                GTC_HIP_CHECK(hipEventCreateWithFlags(&ready[k], hipEventDisableTiming));
                for (int q = 0; q < 2; ++q)
                    GTC_HIP_CHECK(hipEventCreateWithFlags(&done[k][q], hipEventDisableTiming));
            }
            GTC_TRY(wait_host_csr(G, s));  // uploads read the pinned CSR after the build's downloads
            GTC_HIP_CHECK(hipEventRecord(ev_start, s));
            GTC_HIP_CHECK(hipStreamWaitEvent(s2, ev_start, 0));
            a.tiled = 1;
            int64_t prev_h = -1, prev_s = -1;  // windows of the launch in flight on the other stream
            int t = 0;
            for (int64_t h = 0; h < nwin; ++h) {
                const int64_t nh = G->win_hubs[h + 1] - G->win_hubs[h];
                if (nh <= 0) continue;
                const int q = t & 1;
                hipStream_t st = q ? s2 : s;
                const int64_t smax = G->win_smax[h];
                int sl[2] = {-1, -1};
                const int64_t need[2] = {h, smax};
                for (int u = 0; u < 2; ++u) {
                    const int64_t w = need[u];
                    for (int k = 0; k < kSlots; ++k)
                        if (slot_win[k] == w) sl[u] = k;
                    if (sl[u] >= 0) continue;
                    int victim = -1;
                    for (int pass = 0; pass < 2 && victim < 0; ++pass) {
                        for (int k = 0; k < kSlots; ++k) {
                            const int64_t x = slot_win[k];
                            if (x == h || x == smax) continue;
                            if (pass == 0 && (x == prev_h || x == prev_s)) continue;
                            if (victim < 0 || slot_used[k] < slot_used[victim]) victim = k;
                        }
                    }
                    if (victim < 0) {
                        set_error("4pCF tiles: no window buffer free for window %lld", (long long)w);
                        return GTC_E_HIP;
                    }
                    for (int r = 0; r < 2; ++r)  // after every launch that read the buffer
                        if (done_set[victim][r]) GTC_HIP_CHECK(hipStreamWaitEvent(st, done[victim][r], 0));
                    const int64_t e0w = G->win_e[w], ne = G->win_e[w + 1] - e0w;
                    if (ne > 0) {
                        if (G->rebuild) {
                            GTC_TRY(emit_window(G, w, wcol[victim], wbin[victim], st));
                        } else {
                            GTC_HIP_CHECK(hipMemcpyAsync(wcol[victim], G->h_col + e0w,
                                                         sizeof(int32_t) * ne, hipMemcpyHostToDevice, st));
                            if (!G->packed)
                                GTC_HIP_CHECK(hipMemcpyAsync(wbin[victim], G->h_bin + e0w, ne,
                                                             hipMemcpyHostToDevice, st));
                        }
                    }
                    GTC_HIP_CHECK(hipEventRecord(ready[victim], st));
                    slot_win[victim] = w;
                    sl[u] = victim;
                }
                for (int u = 0; u < 2; ++u) {
                    GTC_HIP_CHECK(hipStreamWaitEvent(st, ready[sl[u]], 0));
                    slot_used[sl[u]] = ++clock;
                }
                const int sh = sl[0], sn = sl[1];
                a.col_h = a.col_1 = a.col_2 = wcol[sh];
                a.bin_h = a.bin_1 = a.bin_2 = wbin[sh];
                a.base_h = a.base_1 = a.base_2 = G->win_e[h];
                a.w1_lo = a.w2_lo = (int32_t)G->win[h];
                a.w1_hi = a.w2_hi = (int32_t)G->win[smax + 1];
                a.e_split = smax > h ? G->win_e[smax] : INT64_MAX;
                a.base_1b = smax > h ? G->win_e[smax] - ((intptr_t)wcol[sn] - (intptr_t)wcol[sh]) / 4 : 0;
                GTC_TRY(launch(G->hubs + G->win_hubs[h], nh, st, q ? queue2 : queue, q ? qcount2 : qcount));
                for (int u = 0; u < 2; ++u) {
                    GTC_HIP_CHECK(hipEventRecord(done[sl[u]][q], st));
                    done_set[sl[u]][q] = true;
                }
                prev_h = h;
                prev_s = smax;
                ++t;
            }
            a.e_split = INT64_MAX;
            a.base_1b = 0;
            GTC_HIP_CHECK(hipEventRecord(ev_end2, s2));
            GTC_HIP_CHECK(hipStreamWaitEvent(s, ev_end2, 0));
            return GTC_OK;
        };
        rc = two();
        if (s2) {
            (void)hipStreamSynchronize(s2);
            (void)hipStreamDestroy(s2);
        }
        if (ev_start) (void)hipEventDestroy(ev_start);
        if (ev_end2) (void)hipEventDestroy(ev_end2);
        for (int k = 0; k < kSlots; ++k) {
            if (ready[k]) (void)hipEventDestroy(ready[k]);
            for (int q = 0; q < 2; ++q)
                if (done[k][q]) (void)hipEventDestroy(done[k][q]);
        }
    }
    if (!rc && G->n_hubs > 0 && tiled && !two_streams) {
        // Tiles (h, c1, c2), h <= c1 <= c2 <= the last window holding a spoke of window h: the
        // tetrahedra with hub i in window h, spoke a in c1 and spoke b in c2 (i < a < b), each
        // counted in exactly one tile.  When the spokes of window h reach no further than window
        // h + 1, one launch takes all of them (c1 = c2 = windows h and h + 1), so that each hub
        // is set up once.  The windows are made resident (copied from the pinned CSR or emitted
        // again), evicting the least recently used window a tile does not need; all on the
        // counting stream, after the kernels that read the buffer.
        int64_t slot_win[kSlots] = {-1, -1, -1}, slot_used[kSlots] = {0, 0, 0}, clock = 0;
        rc = wait_host_csr(G, s);  // uploads read the pinned CSR after the build's downloads
        auto ensure = [&](int64_t w, int64_t keep1, int64_t keep2, int *slot) -> int {
            for (int k = 0; k < kSlots; ++k)
                if (slot_win[k] == w) {
                    slot_used[k] = ++clock;
                    *slot = k;
                    return GTC_OK;
                }
            int best = -1;
            for (int k = 0; k < kSlots; ++k) {
                if (slot_win[k] == keep1 || slot_win[k] == keep2) continue;
                if (best < 0 || slot_used[k] < slot_used[best]) best = k;
            }
            const int64_t e0w = G->win_e[w], ne = G->win_e[w + 1] - e0w;
            if (ne > 0) {
                if (G->rebuild) {
                    GTC_TRY(emit_window(G, w, wcol[best], wbin[best], s));
                } else {
                    GTC_HIP_CHECK(hipMemcpyAsync(wcol[best], G->h_col + e0w, sizeof(int32_t) * ne,
                                                 hipMemcpyHostToDevice, s));
                    if (!G->packed)
                        GTC_HIP_CHECK(hipMemcpyAsync(wbin[best], G->h_bin + e0w, ne,
                                                     hipMemcpyHostToDevice, s));
                }
            }
            slot_win[best] = w;
            slot_used[best] = ++clock;
            *slot = best;
            return GTC_OK;
        };
        const int64_t W = (int64_t)G->win.size() - 1;
        a.tiled = 1;
        for (int64_t h = 0; h < W && !rc; ++h) {
            const int64_t nh = G->win_hubs[h + 1] - G->win_hubs[h];
            if (nh <= 0) continue;
            const int64_t smax = G->win_smax[h];
            if (smax <= h + 1) {
                int sh = 0, sn = 0;
                rc = ensure(h, smax, smax, &sh);
                if (!rc) rc = ensure(smax, h, h, &sn);
                if (rc) break;
                a.col_h = a.col_1 = a.col_2 = wcol[sh];
                a.bin_h = a.bin_1 = a.bin_2 = wbin[sh];
                a.base_h = a.base_1 = a.base_2 = G->win_e[h];
                a.w1_lo = a.w2_lo = (int32_t)G->win[h];
                a.w1_hi = a.w2_hi = (int32_t)G->win[smax + 1];
                a.e_split = smax > h ? G->win_e[smax] : INT64_MAX;
                a.base_1b = smax > h ? G->win_e[smax] - ((intptr_t)wcol[sn] - (intptr_t)wcol[sh]) / 4 : 0;
                rc = launch(G->hubs + G->win_hubs[h], nh);
                a.e_split = INT64_MAX;
                a.base_1b = 0;
                continue;
            }
            for (int64_t c1 = h; c1 <= smax && !rc; ++c1)
                for (int64_t c2 = c1; c2 <= smax && !rc; ++c2) {
                    int sh = 0, s1 = 0, s2 = 0;
                    rc = ensure(h, c1, c2, &sh);
                    if (!rc) rc = ensure(c1, h, c2, &s1);
                    if (!rc) rc = ensure(c2, h, c1, &s2);
                    if (rc) break;
                    a.col_h = wcol[sh];
                    a.bin_h = wbin[sh];
                    a.base_h = G->win_e[h];
                    a.col_1 = wcol[s1];
                    a.bin_1 = wbin[s1];
                    a.base_1 = G->win_e[c1];
                    a.w1_lo = (int32_t)G->win[c1];
                    a.w1_hi = (int32_t)G->win[c1 + 1];
                    a.col_2 = wcol[s2];
                    a.bin_2 = wbin[s2];
                    a.base_2 = G->win_e[c2];
                    a.w2_lo = (int32_t)G->win[c2];
                    a.w2_hi = (int32_t)G->win[c2 + 1];
                    rc = launch(G->hubs + G->win_hubs[h], nh);
                }
        }
    }
    if (!rc && WT) rc = finalize_class_sums(wsum, ncfg, copies, 6 * ncfg, scale, d_even_w, d_odd_w, s);
    std::vector<unsigned long long> h_even(ncfg);
    if (!rc) {
        hipError_t e = hipMemcpyAsync(h_even.data(), d_even, 8 * ncfg, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) rc = hip_fail(e, "4pCF readback", __FILE__, __LINE__);
        // launches on two streams overlap: from the first start to the last end
        const size_t k0 = two_streams && kev.size() >= 2 ? kev.size() - 2 * (size_t)tiles_run : 0;
        for (size_t k = 0; !rc && k + 1 < kev.size(); k += 2) {
            float t = 0.f;
            if (two_streams && k >= k0) {
                (void)hipEventElapsedTime(&t, kev[k0], kev[k + 1]);
                kms = std::max(kms, t);
            } else {
                (void)hipEventElapsedTime(&t, kev[k], kev[k + 1]);
                kms += t;
            }
        }
    }
    (void)hipStreamSynchronize(s);
    for (hipEvent_t e : kev) (void)hipEventDestroy(e);
    dev_free(scratch, s);
    if (rc) return rc;
    unsigned long long cl = 0;
    for (auto v : h_even) cl += v;
    if (st) {
        st->launch_waves = waves;
        st->launch_blocks = launched_blocks;
        st->launch_lds_bytes = (int32_t)lds;
        st->cliques4 = cl;
        st->merge_walks = G->walks;
        st->tiles = tiles_run;
        st->kernel_ms = kms;
        st->weight_scale = scale;
    }
    return GTC_OK;
}

}  // namespace gtc

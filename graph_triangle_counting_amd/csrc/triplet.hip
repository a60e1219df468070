// triplet.hip - binned triangle enumeration, the 3pCF numerator (GRAMSCI v2 §II.2, §III.1).
//
// One wavefront per hub i (persistent workgroups); hubs are taken heaviest first, in batches, from
// one counter per work class (HubQueue).  The pages' merge-walk intersects the hub tail
// {k in N(i): k > j} with N(j) for every spoke j by two pointers over both sorted lists.  Here the
// hub side of that walk is held in LDS as a direct-address map over the hub's stencil domain (the
// label ranges of its forward cells, see hub_domain): map[k] = bin(i,k) + 1 for k in N+(i), 0
// otherwise.  The spoke rows are streamed once, in order: 64 spokes at a time, their rows laid end
// to end by a wave scan and read with 8 (or 16) loads in flight per lane.  Each element is one
// O(1) LDS probe, and elements past the hub's last neighbour miss, as the two-pointer walk stops
// when the hub list is exhausted.  Every element of N+(j) exceeds j, so a hit is exactly a triangle
// i < j < k, counted once.
//
// A hit ranks its sorted side-length bins (Fig. 8 key order) and adds 1 to a workgroup LDS
// histogram (32-bit, exchanged out before it could overflow); the histogram is flushed with 64-bit
// global atomics.  Weighted counts add the exact fixed-point value of fl(fl(w1*w2)*w3) as two
// limbs (28 low bits, 30 offset high bits) to 64-bit LDS counters, flushed into 128-bit global
// accumulators, so the sum is exact and independent of order (the pages accumulate fp atomics,
// §III.5.2, and see order-dependent last digits, §IV.8).
//
// Graphs over several hub windows (§III.5.3) run as a loop of tiles (hub window, search windows);
// out-of-core windows are uploaded from pinned host memory on a copy stream, or emitted again by
// the pair search, while the previous tile counts.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gtc_internal.h"

namespace gtc {

struct TripletArgs {
    const int64_t *row_ptr;  // global row offsets [n+1]
    // hub window: rows of hubs, entry e at col_h[e - base_h] (bin_h null: packed entries)
    const int32_t *col_h;
    const uint8_t *bin_h;
    int64_t base_h;
    // search windows: rows of spokes j in [s_lo, s_hi); entry e at col_s[e - base_s] (and
    // bin_s[e - base_s]) when e < e_split, else at col_s[e - base_s2]: a launch may span two
    // search windows held in two buffers of one allocation (base_s2 folds in their distance)
    const int32_t *col_s;
    const uint8_t *bin_s;
    int64_t base_s;
    int64_t e_split, base_s2;
    int32_t s_lo, s_hi;
    const int32_t *hubs;  // hubs of this launch, heaviest first
    int32_t n_hubs;
    int32_t nb, ncfg;
    int32_t map_bytes;   // per-wave map (bytes), multiple of 16, covers every hub's domain
    int32_t wave_bytes;  // per-wave LDS region: map, spoke chunk, (weighted) hub row
    int32_t max_m;       // longest forward row
    const int32_t *key_s;
    const int32_t *cell_start;
    const int64_t *work;
    const uint32_t *slot_off;  // [n][16] forward cell slot starts of every row
    uint8_t band[145];         // banded walk: tlo[14][5], thi[14][5], smax[5]
    Grid gr;
    const double *w_s;  // weights, internal order (weighted only)
    double two_s;       // 2^s
    unsigned int *queue;         // class counters, kQueueStride words apart
    const unsigned int *qcount;  // [kHubClasses] hubs per class in this launch's hub list
    unsigned int batch_cap;      // largest batch of hubs per take
    // banded walk: > 0 splits each hub into one queue entry per key run, taken a group of this
    // many hubs at a time (every hub's run 0, then their run 1, ...), so that the waves of an XCD
    // read one run's spoke rows together
    unsigned int band_group;
    int32_t hist_copies;  // unsorted histogram: 1, or 2 (odd lanes add to the second copy)
    unsigned long long *counts;  // [ncfg]
    unsigned long long *limbs;   // [ncfg][4]: 128-bit sum of low limbs, 128-bit sum of high limbs
    unsigned int flush_at;       // hits (unsorted histogram: walked elements) a wave may add
                                 // between exchanges of the LDS histogram
};

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void add_u128(unsigned long long *p, unsigned long long v) {
    const unsigned long long old = atomicAdd(p, v);
    if (old + v < old) atomicAdd(p + 1, 1ull);
}

__device__ __forceinline__ unsigned int wave_sum(unsigned int v) {
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// LDS layout: rank tables A, B (i32[256] each, at LDS address 0) | band table (tlo, thi [14][5],
// smax [5]) | counts u32[ncfg] | (weighted) low limbs u64[ncfg], high limbs u64[ncfg] | nw
// per-wave regions.  The rank tables hold 4 A[x] + the counts' LDS address and 4 B[y], so that a
// configuration's counter address is A[x] + B[y] + 4 z, read with its bins scaled by 4 as byte
// offsets.  The unsorted histogram (no rank per hit) comes first, and the tables after it,
// unscaled.
// (with a global histogram, GH, only the rank and band tables and the maps are in LDS)
constexpr size_t kBandTableBytes = 160;
constexpr int32_t kHistLds = 2 * 256 * 4 + (int32_t)kBandTableBytes;
// (nhist counters: ncfg times the histogram copies; weighted, as many low limbs and ncfg high ones)
__host__ __device__ inline size_t triplet_lds_fixed(int nhist, int ncfg, bool weighted, bool gh) {
    size_t b = kHistLds;
    if (!gh) {
        b += align_up(sizeof(uint32_t) * nhist, 16);
        if (weighted) b += sizeof(unsigned long long) * ((size_t)nhist + ncfg);
    }
    return b;
}

// Exchange the workgroup histogram out to global memory.  Safe while other waves keep adding:
// each bin is swapped for zero atomically, so every increment is flushed exactly once.
template <bool W>
__device__ __forceinline__ void flush_hist(int ncfg, unsigned long long *counts,
                                           unsigned long long *limbs, uint32_t *hc,
                                           unsigned long long *hl, int copies, int first,
                                           int step) {
    for (int t = first; t < ncfg; t += step) {
        uint32_t v = atomicExch(&hc[t], 0u);
        if (copies > 1) v += atomicExch(&hc[ncfg + t], 0u);
        if (v) atomicAdd(&counts[t], (unsigned long long)v);
        if (W) {
            unsigned long long l = atomicExch(&hl[t], 0ull);
            if (copies > 1) l += atomicExch(&hl[ncfg + t], 0ull);  // (each below 2^61)
            if (l) add_u128(&limbs[4 * t], l);
            const unsigned long long h = atomicExch(&hl[copies * ncfg + t], 0ull);
            if (h) add_u128(&limbs[4 * t + 2], h);
        }
    }
}

// Rows of the histogram over unsorted bin triples (one per b_jk), padded so that the rows of one
// spoke's hits start in different LDS banks: with at most 16 bins a row's b_ik cover at most half
// of the 32 banks and consecutive rows start nb banks apart (nb^2 padded to nb modulo 32); with
// more bins an odd row length suffices.
__host__ __device__ inline int unsorted_row(int nb) {
    return nb <= 16 ? nb * nb + (nb - nb * nb % 32 + 32) % 32 : nb * nb | 1;
}

// The same for a histogram over the unsorted bin triple t = b0 unsorted_row(nb) + b1 nb + b2
// (nb rows): each bin is added to the rank of its sorted triple.
__device__ __forceinline__ void flush_hist_unsorted(int nb, unsigned long long *counts, uint32_t *hu,
                                                    const int32_t *rA, const int32_t *rB, int first,
                                                    int step) {
    const int row = unsorted_row(nb), nh = nb * row;
    for (int t = first; t < nh; t += step) {
        const int r = t % row;
        if (r >= nb * nb) continue;  // (the padding bin)
        const uint32_t v = atomicExch(&hu[t], 0u);
        if (!v) continue;
        const int b0 = t / row, b1 = r / nb, b2 = r % nb;
        const int x = min(b0, min(b1, b2)), z = max(b0, max(b1, b2)), y = b0 + b1 + b2 - x - z;
        atomicAdd(&counts[rA[x] + rB[y] + z], (unsigned long long)v);
    }
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// Per-wave LDS region: hub map | chunk of 64 spokes | (weighted) the hub row's weights.
//   map    : u8 bin+1 per domain label (unsorted histogram: 4 (bin+1)), or (weighted) u32
//            (LDS address of the label's hub weight) | 4 bin << 18.  The flat walk's map holds
//            the domain's five key runs, each after a zero entry, and a zero entry at the end;
//            the banded walk's covers one key run, with a zero entry on each side
//   chunk  : cpre u32[65] flat start of each spoke's row, cbase i64[64] (row start - flat start,
//            relative to the CSR slice), then for the unsorted histogram cbij u8[64] spoke bins,
//            for the sorted one cown u32[64] owner words ((weighted) the LDS address of the
//            spoke's cw entry | 4 bin << 18), and (weighted) cw f64[64]: the spoke weights
constexpr int kChunkPre = 0, kChunkBase = 272, kChunkBij = 784, kChunkOwn = 848, kChunkW = 1104;
__host__ __device__ inline size_t chunk_bytes(bool weighted, bool uh) {
    return weighted ? 1616 : uh ? 848 : 1104;
}
__host__ __device__ inline size_t map_entry_bytes(bool weighted) { return weighted ? 4 : 1; }
__host__ __device__ inline size_t hubrow_bytes(bool weighted, int max_m) {
    return weighted ? align_up(8 * (size_t)max_m, 16) : 0;
}
// LDS addresses below 2^18 (160 KB) leave the top bits of a weighted map entry or owner word to
// 4 x the bin
constexpr int kLdsAddrBits = 18;

// spoke-row loads in flight per lane
constexpr int kUnroll = 8;
// banded walk: probes issued together before their hits (the deep kernel, 16 loads in flight: 8;
// the 8-load kernel: 2).  More LDS reads in flight per wave hide their latency; a whole deep block
// at once measured slower.
constexpr int kProbeBatch = 8;
constexpr int kProbeBatchShallow = 2;

// Banded walk (grids of at least 3 cells per axis).  A hub's forward stencil is five key runs
// ("bands"); band q holds the hub-row slots [kBandSlot[q], kBandSlot[q+1]) (own cell and the
// next cell, then three rows of three cells).  A spoke sitting in hub slot s has its own forward
// cell slots [tlo, thi) = band table[s][q] inside band q, so its elements there form one
// contiguous piece of its row, found from the row's slot offsets, and every label in that piece
// lies in band q's label range: its map address is the label less a per-band constant, clamped
// onto the zero entries beside the band (only the walk's no-element sentinel is clamped).
__host__ __device__ constexpr int band_slot(int q) { return q == 0 ? 0 : 3 * q - 1; }

// Banded walk: hubs of at least 2^kRunSplitLog2 spoke elements are queued once per key run, a
// group of hubs at a time, so that the waves of one XCD read the same run's spoke rows together
// (halves the L2 misses of a 4M-point graph of degree 2250); lighter hubs pay more for the repeated
// hub set-up than they gain.
constexpr int kRunSplitLog2 = 17;

// UH (unweighted, LDS histogram, few bins): hits go to a histogram over the unsorted bin triple
// (bij, bik, bjk) - nb rows, one per b_jk, of nb^2 bins padded (unsorted_row) - with neither a
// sort nor a rank lookup per triangle; the bins are folded onto configuration ranks when the
// histogram is exchanged.
// DEEP: 2 kUnroll loads in flight per lane, for launches whose LDS histogram leaves room for
// only 16 waves per CU (their registers are then free).
template <bool W, bool GH, bool BANDED, bool PK, bool UH, bool DEEP = false>
__global__ void __launch_bounds__(1024) k_triplet(TripletArgs a) {
    constexpr int kUnroll = DEEP ? 2 * gtc::kUnroll : gtc::kUnroll;
    static_assert(!UH || (!W && !GH), "the unsorted histogram is an unweighted LDS histogram");
    // A walk over packed entries keeps each element's whole entry, which the probe and the hit
    // take apart.
    constexpr bool kRawEntry = PK;
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    // (the unsorted histogram, whose hits need no rank, keeps the LDS start and the tables follow)
    const int32_t nhist = a.hist_copies * (UH ? a.nb * unsorted_row(a.nb) : a.ncfg);
    const size_t hbytes = GH ? 0 : align_up(sizeof(uint32_t) * nhist, 16);
    int32_t *rA = reinterpret_cast<int32_t *>(smem + (UH ? hbytes : 0));  // (rank tables)
    int32_t *rB = rA + 256;
    uint8_t *btab = reinterpret_cast<uint8_t *>(rB + 256);  // tlo[14*5] | thi[14*5] | smax[5]
    uint32_t *hc = reinterpret_cast<uint32_t *>(smem + (UH ? 0 : kHistLds));
    size_t off = kHistLds + hbytes;
    // (weighted) low limb sums [nhist], then the high ones [ncfg]
    unsigned long long *hl = nullptr;
    if (W && !GH) {
        hl = reinterpret_cast<unsigned long long *>(smem + off);
        off += sizeof(unsigned long long) * ((size_t)nhist + a.ncfg);
    }
    unsigned char *wb = smem + off + (size_t)wid * a.wave_bytes;
    uint8_t *map8 = wb;
    // the wave's map as an LDS address
    typedef __attribute__((address_space(3))) unsigned char lds_u8;
    typedef __attribute__((address_space(3))) uint32_t lds_u32;
    typedef __attribute__((address_space(3))) int32_t lds_i32;
    typedef __attribute__((address_space(3))) unsigned long long lds_u64;
    typedef __attribute__((address_space(3))) double lds_f64;
    const int32_t map_off = (int32_t)(uint32_t)(uintptr_t)(lds_u8 *)wb;
    const int32_t hc_lds = (int32_t)(uint32_t)(uintptr_t)(lds_u8 *)hc;  // the histogram's LDS address
    // low limb address of the configuration whose count is at LDS address h: 2 (h - hc_lds) past hl
    // (its high limb nhist words further)
    const int32_t hl_lds = W && !GH ? (int32_t)(uint32_t)(uintptr_t)(lds_u8 *)hl - 2 * hc_lds : 0;
    const int32_t hh_lds = hl_lds + 8 * nhist;
    // (histogram in two copies: odd lanes add to the second, so that lanes of one wave that hit the
    // same bin collide half as often; weighted, the counts and low limbs have a second copy)
    const int32_t hc_lane =
        hc_lds + (UH && (lane & 1) ? (a.hist_copies - 1) * 4 * a.nb * unsorted_row(a.nb) : 0);
    const uint32_t cp_lane = W && (lane & 1) ? (uint32_t)((a.hist_copies - 1) * 4 * a.ncfg) : 0u;
    uint32_t *mapw = reinterpret_cast<uint32_t *>(wb);
    unsigned char *ck = wb + a.map_bytes;
    uint32_t *cpre = reinterpret_cast<uint32_t *>(ck + kChunkPre);
    int64_t *cbase = reinterpret_cast<int64_t *>(ck + kChunkBase);
    uint8_t *cbij = ck + kChunkBij;
    uint32_t *cown = reinterpret_cast<uint32_t *>(ck + kChunkOwn);
    double *cw = reinterpret_cast<double *>(ck + kChunkW);
    double *rw = reinterpret_cast<double *>(ck + chunk_bytes(true, false));
    const int32_t cw_lds = (int32_t)(uint32_t)(uintptr_t)(lds_u8 *)(ck + kChunkW);
    const int32_t rw_lds = (int32_t)(uint32_t)(uintptr_t)(lds_u8 *)rw;

    if (!GH)
        for (int t = threadIdx.x; t < nhist + (W ? a.ncfg : 0); t += blockDim.x) {
            if (t < nhist) hc[t] = 0;
            if (W) hl[t] = 0;
        }
    if (threadIdx.x == 0) {
        rank3_tables(a.nb, rA, rB);
        if (!UH)  // (the sorted histogram's hits read them scaled)
            for (int t = 0; t < a.nb; ++t) {
                rA[t] = 4 * rA[t] + hc_lds;
                rB[t] *= 4;
            }
    }
    // fields the walk uses, as plain values (capturing the argument struct by reference would
    // make the compiler keep the whole struct live in registers)
    const int32_t ncfg = a.ncfg;
    const int32_t *const col_s = a.col_s;
    const uint8_t *const bin_s = a.bin_s;
    const int64_t base_s = a.base_s;
    const int64_t e_split = a.e_split, base_s2 = a.base_s2;
    unsigned long long *const g_counts = a.counts;
    unsigned long long *const g_limbs = a.limbs;
    const double two_s = a.two_s;
    const int32_t nbk = a.nb;
    const uint32_t nb4 = 4u * ((uint32_t)nbk & 0xffu);  // (bins below 2^8)
    const uint32_t row4 = 4u * ((uint32_t)unsorted_row(nbk) & 0xffffu);  // (below 2^16)
    if constexpr (BANDED)
        for (int t = threadIdx.x; t < 145; t += blockDim.x) btab[t] = a.band[t];
    __syncthreads();

    unsigned int wave_hits = 0;
    HubQueue hub_queue;
    // classes of at least 2^kRunSplitLog2 spoke elements per hub take one entry per key run
    const bool by_run = BANDED && a.band_group > 0;
    hub_queue.init(a.qcount, a.batch_cap, lane, (int)(blockIdx.x % kQueueParts),
                   by_run && 63 - lane >= kRunSplitLog2 ? 5u : 1u);
    for (;;) {
        uint32_t hq;
        if (!hub_queue.next(a.queue, lane, hq)) break;
        // the hub-list position of the entry's hub, and its key run (5: every run)
        uint32_t run_only = 5;
        if (by_run && 63 - hub_queue.cls >= kRunSplitLog2)
            hub_queue.split(hq, 5u, a.band_group, hq, run_only);
        else if (by_run)
            hq = hub_queue.hub_pos(hq);
        const int32_t i = __builtin_amdgcn_readfirstlane(a.hubs[hq]);
        const int64_t rb = a.row_ptr[i], re = a.row_ptr[i + 1];
        const int32_t key_i = a.key_s[i];
        const double wi = W ? a.w_s[i] : 0.0;
        const int32_t m = (int32_t)(re - rb);
        const int32_t *hrow = a.col_h + (rb - a.base_h);
        const uint8_t *hbin = a.bin_h + (rb - a.base_h);
        // The first 64 positions of the hub row with their spoke rows (and weights), loaded in one
        // pass: the hub map, the hub weights and the first chunk of spokes take them from here,
        // which keeps a hub's set-up to four dependent rounds of global loads.
        int32_t j0 = 0, b0 = 0, len0 = 0;
        int64_t sb0 = 0;
        double wj0 = 0.0;
        // (Banded hubs are long and read their spokes per band: they skip this.)
        // label of hub-row position p (packed entries carry the bin in the top byte)
        auto hlab = [&](int p) __attribute__((always_inline)) {
            return PK ? (int32_t)((uint32_t)hrow[p] & kLabelMask) : hrow[p];
        };
        if (!BANDED && lane < m) csr_entry<PK>(hrow, hbin, lane, j0, b0);
        HubDomain dom;
        hub_domain(i, key_i, a.gr, a.cell_start, dom);
        if (!BANDED && lane < m) {
            sb0 = a.row_ptr[j0];
            len0 = (int32_t)(a.row_ptr[j0 + 1] - sb0);
            if (W) wj0 = a.w_s[j0];
        }
        const int32_t hub_lo = BANDED ? hlab(0) : __shfl(j0, 0, kWave);
        const int32_t hub_hi = !BANDED && m <= kWave ? __shfl(j0, m - 1, kWave) : hlab(m - 1);
        if (W)
            for (int p = lane; p < m; p += kWave)
                rw[p] = !BANDED && p < kWave ? wj0 : a.w_s[hlab(p)];

        // spokes of this tile: hub-row positions [p_lo, p_hi) with j in [s_lo, s_hi)
        int32_t p_lo = 0, p_hi = m;
        if (a.s_lo > hub_lo || a.s_hi <= hub_hi) {
            int32_t l = 0, h = m;
            while (l < h) { const int32_t md = (l + h) >> 1; if (hlab(md) < a.s_lo) l = md + 1; else h = md; }
            p_lo = l;
            h = m;
            while (l < h) { const int32_t md = (l + h) >> 1; if (hlab(md) < a.s_hi) l = md + 1; else h = md; }
            p_hi = l;
        }

        unsigned int my_hits = 0;
        uint32_t hub_elems = 0;  // (unsorted histogram) elements walked, a bound on its hits
        // Flat walk: label k's map index is the number of map entries before it, the sum over the
        // five runs of k - lo + 1 clamped to [0, run size + 1] (a zero entry before each run, one
        // at the end): med3(k, lo - 1, hi) summed, less the sum of lo - 1.  A label in a gap
        // between runs, before the first or past the last reads a zero entry.  (As plain
        // scalars: a select over the arrays is lowered to a stack copy.)
        const int32_t a0 = dom.lo[0] - 1, a1 = dom.lo[1] - 1, a2 = dom.lo[2] - 1, a3 = dom.lo[3] - 1,
                      a4 = dom.lo[4] - 1;
        const int32_t z0 = dom.hi[0], z1 = dom.hi[1], z2 = dom.hi[2], z3 = dom.hi[3], z4 = dom.hi[4];
        const int32_t asum = a0 + a1 + a2 + a3 + a4;
        // map entry bytes (weighted map: 4 bytes per label)
        constexpr int32_t kMapEntry = W ? 4 : 1;
        // the LDS address of map index f is fbase + f kMapEntry, f = (sum of the clamps) - asum
        const int32_t fbase = map_off - kMapEntry * asum;

        // Walk the rows of (up to) 64 spokes laid end to end: lane q describes spoke p0 + q by
        // its element range [sb, sb + len) and bin bj.  A wave scan gives each spoke's start in
        // the flat range; the lanes stream the range with kUnroll loads in flight each, map every
        // label k to its hub-map offset and bin every hit.  Banded: the map holds labels
        // [blo, blo + bsize); otherwise it holds the whole domain, found by comparisons.
        auto walk = [&](int32_t p0, int64_t sb, int32_t len, int32_t bj, int32_t blo,
                        int32_t bsize) __attribute__((always_inline)) {
            const int32_t band_c = blo - map_off - 1, band_hi = map_off + bsize + 1;
            const int32_t incl = wave_incl_scan(len, lane);
            const int32_t total = __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1, kWave));
            if (total == 0) return;
            if (UH) hub_elems += (uint32_t)total;
            cpre[lane] = (uint32_t)(incl - len);
            if (lane == kWave - 1) cpre[kWave] = (uint32_t)incl;
            cbase[lane] = sb - (sb >= e_split ? base_s2 : base_s) - (incl - len);
            if (UH) cbij[lane] = (uint8_t)bj;
            else cown[lane] = (W ? (uint32_t)(cw_lds + 8 * lane) : 0u) | ((uint32_t)bj << (kLdsAddrBits + 2));
            if (W) {
                const double wj = len > 0 ? rw[p0 + lane] : 0.0;
                cw[lane] = wj;
            }
            wave_lds_sync();
            // owner spoke of flat index t: the last q with cpre[q] <= t (then t < cpre[q+1]).  The
            // owner's end and row pointers stay in registers; LDS is read again only when t
            // crosses into the next spoke.
            int q = 0;
            {
                int hi = kWave;
                while (hi - q > 1) {
                    const int md = (q + hi) >> 1;
                    if ((int32_t)cpre[md] <= lane) q = md; else hi = md;
                }
            }
            // The lanes take flat elements t = T + lane, T uniform.  Element T + lane is cpl[T]: the
            // owner's row pointer with the lane folded in, so that a block's loads are one pointer
            // and immediate offsets; the owner changes once T reaches qrel.
            int32_t qend = (int32_t)cpre[q + 1];
            int32_t qrel = qend - lane;
            const int32_t *cpl = col_s + cbase[q] + lane;
            const uint8_t *bpl = PK ? nullptr : bin_s + cbase[q] + lane;
            // owner spoke's word: 4 b_ij << 18 and (weighted) the LDS address of its weights; for
            // the histogram over unsorted triples the LDS address of the owner's histogram row
            // instead, less 4: 4 b_ij nb - 4 past row 0, so that a hit adds its map entry
            // 4 (b_ik + 1) and 4 b_jk row
            auto owner_word = [&](int qq_) __attribute__((always_inline)) -> int32_t {
                if constexpr (UH)  // (24-bit multiply: full rate)
                    return (int32_t)__umul24((uint32_t)cbij[qq_], nb4) + hc_lane - 4;
                else return (int32_t)cown[qq_];
            };
            int32_t own = owner_word(q);
            // the owner of element T + lane, and the block pointers cb, bb_ of a block at t0
            auto seek = [&](int32_t T, int32_t t0, const int32_t *&cb, const uint8_t *&bb_)
                            __attribute__((always_inline)) {
                if (T >= qrel) {
                    const int32_t t = T + lane;
                    do {
                        ++q;
                        qend = (int32_t)cpre[q + 1];
                    } while (t >= qend);
                    qrel = qend - lane;
                    cpl = col_s + cbase[q] + lane;
                    cb = cpl + t0;
                    if (!PK) {
                        bpl = bin_s + cbase[q] + lane;
                        bb_ = bpl + t0;
                    }
                    own = owner_word(q);
                }
            };
            // the label's map entry, 0 when it is no neighbour of the hub
            auto probe = [&](int32_t k) __attribute__((always_inline)) -> uint32_t {
                int32_t mo;
                if constexpr (BANDED && !W) {
                    // label k's entry is byte 1 + k - blo of the map, between zero entries at 0
                    // and bsize + 1: a label outside the band (and k = -1, no element) is clamped
                    // onto one of them (a three-operand median, no branch).  As LDS addresses,
                    // with the wave's map address folded into the bounds.
                    // (the compiler forms no median from a min and a max of variables)
                    if constexpr (PK) {
                        // k is the whole packed entry: a 24-bit multiply-add by one takes its
                        // label (the low 24 bits) less the band start in one instruction
                        asm("v_mad_u32_u24 %0, %1, 1, %2\n\tv_med3_i32 %0, %0, %3, %4"
                            : "=&v"(mo)
                            : "v"(k), "v"(-band_c), "v"(map_off), "v"(band_hi));
                    } else {
                        const int32_t x = (int32_t)((uint32_t)k - (uint32_t)band_c);
                        asm("v_med3_i32 %0, %1, %2, %3" : "=v"(mo) : "v"(x), "v"(map_off), "v"(band_hi));
                    }
                    uint32_t e = *(const lds_u8 *)(uintptr_t)(uint32_t)mo;
                    // (kept a 32-bit value: a 16-bit compare would need a zero extension for the hit)
                    if constexpr (UH) asm("" : "+v"(e));
                    return e;
                } else if constexpr (BANDED) {
                    // a label outside the band (and no element) reads a zero entry
                    const int32_t lab = PK ? (int32_t)((uint32_t)k & kLabelMask) : k;
                    mo = 1 + (int32_t)min((uint32_t)(lab - blo), (uint32_t)bsize);
                    return mapw[mo];
                } else {
                    // four sums of three-operand medians, no compare or branch
                    const int32_t lab = PK ? (int32_t)((uint32_t)k & kLabelMask) : k;
                    int32_t m0, m1, m2, m3, m4;
                    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(m0) : "v"(lab), "v"(a0), "v"(z0));
                    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(m1) : "v"(lab), "v"(a1), "v"(z1));
                    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(m2) : "v"(lab), "v"(a2), "v"(z2));
                    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(m3) : "v"(lab), "v"(a3), "v"(z3));
                    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(m4) : "v"(lab), "v"(a4), "v"(z4));
                    const uint32_t mob = (uint32_t)(fbase + kMapEntry * (m0 + m1 + m2 + m3 + m4));
                    if constexpr (W) return *(const lds_u32 *)(uintptr_t)mob;
                    else return *(const lds_u8 *)(uintptr_t)mob;
                }
            };
            // Sorted-histogram hit in two phases, so that the flat walk can issue the LDS reads of
            // two hits before either waits.  hread: the configuration's count address
            // h = 4 rank + hc_lds from the three bins times 4 (byte offsets into the rank tables,
            // at absolute LDS addresses 0 and 1024: the kernel declares no static LDS, so its
            // dynamic block starts at 0), sorted by a minimum, a median and a maximum of three;
            // and (weighted) the hub and spoke weights in order, wx <= wy, and the third weight.
            // Lanes without a hit (v = 0) read valid addresses.
            auto hread = [&](int32_t bjk, int32_t ow, uint32_t v, uint32_t &h, double &wx, double &wy,
                             double &wk) __attribute__((always_inline)) {
                const uint32_t bij4 = (uint32_t)ow >> kLdsAddrBits;
                const uint32_t bik4 = W ? v >> kLdsAddrBits : 4 * v - 4;
                uint32_t bjk4;
                if constexpr (kRawEntry)  // b_jk is the entry's top byte: a byte-select shift
                    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD "
                        "src0_sel:DWORD src1_sel:BYTE_3"
                        : "=v"(bjk4)
                        : "v"(bjk));
                else bjk4 = (uint32_t)bjk << 2;
                uint32_t x4, y4, z4;
                asm("v_min3_u32 %0, %1, %2, %3" : "=v"(x4) : "v"(bij4), "v"(bik4), "v"(bjk4));
                asm("v_med3_u32 %0, %1, %2, %3" : "=v"(y4) : "v"(bij4), "v"(bik4), "v"(bjk4));
                asm("v_max3_u32 %0, %1, %2, %3" : "=v"(z4) : "v"(bij4), "v"(bik4), "v"(bjk4));
                h = (uint32_t)*(const lds_i32 *)(uintptr_t)x4 +
                    (uint32_t)*(const lds_i32 *)(uintptr_t)(1024 + y4) + z4;
                if constexpr (W) {
                    constexpr uint32_t kAddr = (1u << kLdsAddrBits) - 1;
                    const double wj = *(const lds_f64 *)(uintptr_t)((uint32_t)ow & kAddr);
                    asm("v_min_f64 %0, %1, %2" : "=v"(wx) : "v"(wi), "v"(wj));
                    asm("v_max_f64 %0, %1, %2" : "=v"(wy) : "v"(wi), "v"(wj));
                    wk = *(const lds_f64 *)(uintptr_t)(v & kAddr);
                }
            };
            // hadd: the count and (weighted) the fixed-point limbs of fl(fl(w1 w2) w3) over the
            // three weights ascending: the hub and spoke pair wx <= wy is ordered already, so w3
            // is the larger of wy and wk, and w1 w2 the product of wx and the smaller (weights
            // are finite; a tie of +0 and -0 gives a zero product either way)
            auto hadd = [&](uint32_t v, uint32_t h, double wx, double wy, double wk)
                            __attribute__((always_inline)) {
                if (!v) return;
                const int32_t c = (int32_t)((h - (uint32_t)hc_lds) >> 2);  // (global histogram)
                const uint32_t hq = h + cp_lane;  // (this lane's copy)
                if (GH) atomicAdd(&g_counts[c], 1ull);
                else atomicAdd((uint32_t *)(lds_u32 *)(uintptr_t)hq, 1u);
                if (W) {
                    double mn, mx;
                    asm("v_min_f64 %0, %1, %2" : "=v"(mn) : "v"(wy), "v"(wk));
                    asm("v_max_f64 %0, %1, %2" : "=v"(mx) : "v"(wy), "v"(wk));
                    const double pr = __dmul_rn(__dmul_rn(wx, mn), mx);
                    const double qv = rint(__dmul_rn(pr, two_s));     // exact integer, |qv| < 2^57
                    const double qh = floor(__dmul_rn(qv, 0x1p-28));   // in [-2^29, 2^29)
                    const double ql = __fma_rn(-qh, 0x1p28, qv);       // in [0, 2^28)
                    const unsigned long long ul = (uint32_t)ql;
                    const unsigned long long uh = (uint32_t)((int32_t)qh + (1 << 29));
                    if (GH) {
                        add_u128(&g_limbs[4 * c], ul);
                        add_u128(&g_limbs[4 * c + 2], uh);
                    } else {
                        // the low limb at 2 (h - hc_lds) past hl (in this lane's copy), the high
                        // one nhist words further (an 8-byte stride spreads the 64-bit adds over
                        // twice the banks of 16-byte records)
                        atomicAdd((unsigned long long *)(lds_u64 *)(uintptr_t)(2 * hq + (uint32_t)hl_lds), ul);
                        atomicAdd((unsigned long long *)(lds_u64 *)(uintptr_t)(2 * h + (uint32_t)hh_lds), uh);
                    }
                }
                ++my_hits;
            };
            auto hit = [&](int32_t bjk, int32_t ow, uint32_t v) __attribute__((always_inline)) {
                if (!v) return;
                if constexpr (UH) {
                    // bin b_jk row + b_ij nb + b_ik at LDS address ow + v + 4 b_jk row, v = 4 (b_ik + 1):
                    // one 24-bit multiply (full rate; a 32-bit multiply issues at a quarter).  Hits
                    // are not counted: the walked elements bound them.
                    uint32_t off;
                    if constexpr (kRawEntry)  // b_jk is the entry's top byte: a byte-select multiply
                        asm("v_mul_u32_u24_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD "
                            "src0_sel:DWORD src1_sel:BYTE_3\n\tv_add3_u32 %0, %0, %3, %4"
                            : "=&v"(off)
                            : "s"(row4), "v"(bjk), "v"(ow), "v"(v));
                    else off = ((uint32_t)bjk & 0xffu) * row4 + (uint32_t)ow + v;
                    atomicAdd((uint32_t *)(lds_u32 *)(uintptr_t)off, 1u);
                    return;
                }
                uint32_t h;
                double wx = 0.0, wy = 0.0, wk = 0.0;
                hread(bjk, ow, v, h, wx, wy, wk);
                hadd(v, h, wx, wy, wk);
            };
            // the first r element steps of a block (r uniform: kUnroll but in the last block)
            auto process_block = [&](const int32_t *kk, const int32_t *bb, const int32_t *qq, int r)
                                     __attribute__((always_inline)) {
                if constexpr (BANDED) {
                    // (the raw packed entry stands for its bin in the unsorted-histogram hit)
                    constexpr int PB = DEEP ? kProbeBatch : kProbeBatchShallow;
#pragma unroll
                    for (int u0 = 0; u0 < kUnroll; u0 += PB) {
                        uint32_t vv[PB];
#pragma unroll
                        for (int d = 0; d < PB; ++d) vv[d] = u0 + d < r ? probe(kk[u0 + d]) : 0u;
#pragma unroll
                        for (int d = 0; d < PB; ++d)
                            if (u0 + d < r) hit(kRawEntry ? kk[u0 + d] : bb[u0 + d], qq[u0 + d], vv[d]);
                    }
                } else {  // every probe of the block first, then the hits
                    uint32_t vv[kUnroll];
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u) vv[u] = u < r ? probe(kk[u]) : 0u;
                    if constexpr (UH) {
#pragma unroll
                        for (int u = 0; u < kUnroll; ++u)
                            if (u < r) hit(kRawEntry ? kk[u] : bb[u], qq[u], vv[u]);
                    } else {  // (sorted histogram: hits in pairs, both hits' reads issued first)
#pragma unroll
                        for (int u = 0; u < kUnroll; u += 2) {
                            uint32_t h0 = 0, h1 = 0;
                            double x0 = 0.0, y0 = 0.0, w0 = 0.0, x1 = 0.0, y1 = 0.0, w1 = 0.0;
                            if (u < r) hread(kRawEntry ? kk[u] : bb[u], qq[u], vv[u], h0, x0, y0, w0);
                            if (u + 1 < r)
                                hread(kRawEntry ? kk[u + 1] : bb[u + 1], qq[u + 1], vv[u + 1], h1, x1, y1, w1);
                            if (u < r) hadd(vv[u], h0, x0, y0, w0);
                            if (u + 1 < r) hadd(vv[u + 1], h1, x1, y1, w1);
                        }
                    }
                }
            };
            // element u kWave + lane of a block at cb, bb_: its label and bin (kRawEntry: the whole
            // entry); kNone is no element (packed: a label past the band, 2^24 at most, whose low
            // 24 bits fall below the band; in the flat walk label 0, below every hub's domain).
            auto load_elem = [&](const int32_t *cb, const uint8_t *bb_, int u, int32_t &k, int32_t &b)
                                 __attribute__((always_inline)) {
                if constexpr (kRawEntry) {
                    k = cb[u * kWave];
                    b = 0;
                } else {
                    csr_entry<PK>(cb, bb_, u * kWave, k, b);
                }
            };
            const int32_t kNone = kRawEntry ? blo + bsize : -1;
            // whole blocks of kWave * kUnroll elements need no bounds checks; then one checked tail
            constexpr int kBlock = kWave * kUnroll;
            auto load_block = [&](int32_t tb, int32_t *kk, int32_t *bb, int32_t *qq)
                                  __attribute__((always_inline)) {
                const int32_t *cb = cpl + tb;
                const uint8_t *bb_ = PK ? nullptr : bpl + tb;
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    seek(tb + u * kWave, tb, cb, bb_);
                    qq[u] = own;
                    load_elem(cb, bb_, u, kk[u], bb[u]);
                }
            };
            int32_t t0 = 0;
            if constexpr (DEEP && PK) {
                // two blocks in flight: the next block's loads are issued before this block's
                // probes and hits (two register sets, taken in turn)
                const int32_t nfull = total / kBlock;
                int32_t ka[kUnroll], ba[kUnroll], qa[kUnroll], kb2[kUnroll], bb2[kUnroll], qb[kUnroll];
                if (nfull > 0) load_block(0, ka, ba, qa);
                for (int32_t blk = 0; blk < nfull; blk += 2) {
                    if (blk + 1 < nfull) load_block((blk + 1) * kBlock, kb2, bb2, qb);
                    process_block(ka, ba, qa, kUnroll);
                    if (blk + 1 < nfull) {
                        if (blk + 2 < nfull) load_block((blk + 2) * kBlock, ka, ba, qa);
                        process_block(kb2, bb2, qb, kUnroll);
                    }
                }
                t0 = nfull * kBlock;
            } else {
                for (; t0 + kBlock <= total; t0 += kBlock) {
                    int32_t kk[kUnroll], bb[kUnroll], qq[kUnroll];
                    load_block(t0, kk, bb, qq);
                    process_block(kk, bb, qq, kUnroll);
                }
            }
            if (t0 < total) {
                // only the steps that hold elements (a uniform bound), each checked per lane
                const int r = (total - t0 + kWave - 1) / kWave;
                int32_t kk[kUnroll], bb[kUnroll], qq[kUnroll];
                const int32_t *cb = cpl + t0;
                const uint8_t *bb_ = PK ? nullptr : bpl + t0;
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    kk[u] = kNone;
                    bb[u] = 0;
                    qq[u] = own;
                    if (u < r && lane < total - (t0 + u * kWave)) {
                        seek(t0 + u * kWave, t0, cb, bb_);
                        qq[u] = own;
                        load_elem(cb, bb_, u, kk[u], bb[u]);
                    }
                }
                process_block(kk, bb, qq, r);
            }
            wave_lds_sync();  // the next chunk overwrites the chunk arrays
        };

        uint32_t *map32 = reinterpret_cast<uint32_t *>(wb);
        if constexpr (!BANDED) {
            // one map over the whole domain: k -> run by comparisons against the run starts
            // (the domain's labels and six zero entries)
            const int map_words = W ? dom.size + 6 : (dom.size + 9) >> 2;
            for (int t = lane; t < map_words; t += kWave) map32[t] = 0u;
            wave_lds_sync();
            for (int p = lane; p < m; p += kWave) {
                int32_t k = j0, bk = b0;
                if (p >= kWave) csr_entry<PK>(hrow, hbin, p, k, bk);
                const int32_t f = min(max(k, a0), z0) + min(max(k, a1), z1) + min(max(k, a2), z2) +
                                  min(max(k, a3), z3) + min(max(k, a4), z4) - asum;
                if (W) mapw[f] = (uint32_t)(rw_lds + 8 * p) | ((uint32_t)bk << (kLdsAddrBits + 2));
                else map8[f] = (uint8_t)(UH ? 4 * (bk + 1) : bk + 1);
            }
            wave_lds_sync();
            for (int32_t p0 = p_lo; p0 < p_hi; p0 += kWave) {
                const int32_t p = p0 + lane;
                int64_t sb = 0;
                int32_t len = 0, bj = 0;
                if (p < p_hi) {
                    if (p0 == 0) {  // positions 0..63: loaded with the hub
                        bj = b0;
                        sb = sb0;
                        len = len0;
                    } else {
                        int32_t j;
                        csr_entry<PK>(hrow, hbin, p, j, bj);
                        sb = a.row_ptr[j];
                        len = (int32_t)(a.row_ptr[j + 1] - sb);
                    }
                }
                walk(p0, sb, len, bj, 0, 0);
            }
        } else {
            const uint32_t *hso = a.slot_off + (int64_t)i * 16;  // hub row slot starts, [14] = m
            for (int bq = 0; bq < 5; ++bq) {
                if (run_only < 5 && (uint32_t)bq != run_only) continue;
                const int32_t hp_lo = (int32_t)hso[band_slot(bq)], hp_hi = (int32_t)hso[band_slot(bq + 1)];
                if (hp_lo == hp_hi) continue;  // no neighbour of the hub in this band: no triangle
                const int32_t sp_hi = min(p_hi, (int32_t)hso[btab[140 + bq]]);
                if (p_lo >= sp_hi) continue;
                // run bq's label range, selected without indexing (keeps dom in registers)
                int32_t blo = dom.lo[0], bhi = dom.hi[0];
#pragma unroll
                for (int t = 1; t < 5; ++t)
                    if (bq == t) { blo = dom.lo[t]; bhi = dom.hi[t]; }
                const int32_t bsize = bhi - blo;
                // (and the zero entries at 0 and bsize + 1)
                const int map_words = W ? bsize + 2 : (bsize + 5) >> 2;
                for (int t = lane; t < map_words; t += kWave) map32[t] = 0u;
                wave_lds_sync();
                for (int p = hp_lo + lane; p < hp_hi; p += kWave) {
                    int32_t k, bk;
                    csr_entry<PK>(hrow, hbin, p, k, bk);
                    if (W) mapw[1 + k - blo] = (uint32_t)(rw_lds + 8 * p) | ((uint32_t)bk << (kLdsAddrBits + 2));
                    else map8[1 + k - blo] = (uint8_t)(UH ? 4 * (bk + 1) : bk + 1);
                }
                wave_lds_sync();
                for (int32_t p0 = p_lo; p0 < sp_hi; p0 += kWave) {
                    const int32_t p = p0 + lane;
                    int64_t sb = 0;
                    int32_t len = 0, bj = 0;
                    if (p < sp_hi) {
                        int sj = 0;  // hub slot of position p
#pragma unroll
                        for (int t = 1; t < 14; ++t) sj += (int32_t)hso[t] <= p;
                        const int tlo = btab[sj * 5 + bq], thi = btab[70 + sj * 5 + bq];
                        if (tlo < thi) {
                            int32_t j;
                            csr_entry<PK>(hrow, hbin, p, j, bj);
                            const uint32_t *jso = a.slot_off + (int64_t)j * 16;
                            const uint32_t beg = jso[tlo];
                            sb = a.row_ptr[j] + beg;
                            len = (int32_t)(jso[thi] - beg);
                        }
                    }
                    walk(p0, sb, len, bj, blo, bsize);
                }
                wave_lds_sync();  // map reads done before the next band refills it
            }
        }

        if (!GH) {
            wave_hits += UH ? hub_elems : wave_sum(my_hits);
            if (wave_hits >= a.flush_at) {
                if (UH)
                    for (int cp = 0; cp < a.hist_copies; ++cp)
                        flush_hist_unsorted(nbk, g_counts, hc + cp * nbk * unsorted_row(nbk), rA, rB,
                                            lane, kWave);
                else flush_hist<W>(ncfg, g_counts, g_limbs, hc, hl, a.hist_copies, lane, kWave);
                wave_hits = 0;
            }
        }
        wave_lds_sync();  // this wave's LDS reads complete before the next hub rewrites them
    }
    if (!GH) {
        __syncthreads();
        if (UH)
            for (int cp = 0; cp < a.hist_copies; ++cp)
                flush_hist_unsorted(nbk, g_counts, hc + cp * nbk * unsorted_row(nbk), rA, rB,
                                    threadIdx.x, blockDim.x);
        else flush_hist<W>(ncfg, g_counts, g_limbs, hc, hl, a.hist_copies, threadIdx.x, blockDim.x);
    }
}

// ------------------------------------------------------------------ host side

constexpr int kUnsortedMaxBins = 32;  // nb (nb^2 + 1) 32-bit bins: at most 129 KB of LDS
static_assert(4 * kUnsortedMaxBins <= 255, "map entries 4 (bin + 1) are bytes");

struct DeviceLimits {
    int cus = 0;
    size_t lds_per_block = 0;
};

static int device_limits(DeviceLimits &d) {
    int dev = 0;
    GTC_HIP_CHECK(hipGetDevice(&dev));
    GTC_HIP_CHECK(hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev));
    int lds = 0;
    GTC_HIP_CHECK(hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
    d.lds_per_block = (size_t)lds;
    return GTC_OK;
}

struct TripletPlan {
    int waves = 4;       // waves per workgroup
    size_t lds = 0;      // dynamic LDS bytes per workgroup
    int blocks = 0;      // persistent grid
    int per_cu = 0;      // resident workgroups per CU
};

static const void *triplet_kernel(bool w, bool gh, bool banded, bool pk, bool uh, bool deep = false) {
    if (deep && uh && banded && !w && !gh)
        return pk ? reinterpret_cast<const void *>(&k_triplet<false, false, true, true, true, true>)
                  : reinterpret_cast<const void *>(&k_triplet<false, false, true, false, true, true>);
#define GTC_K(W_, GH_, B_, U_)                                                              \
    (pk ? reinterpret_cast<const void *>(&k_triplet<W_, GH_, B_, true, U_>)                \
        : reinterpret_cast<const void *>(&k_triplet<W_, GH_, B_, false, U_>))
    if (w) return gh ? (banded ? GTC_K(true, true, true, false) : GTC_K(true, true, false, false))
                     : (banded ? GTC_K(true, false, true, false) : GTC_K(true, false, false, false));
    if (gh) return banded ? GTC_K(false, true, true, false) : GTC_K(false, true, false, false);
    if (uh) return banded ? GTC_K(false, false, true, true) : GTC_K(false, false, false, true);
    return banded ? GTC_K(false, false, true, false) : GTC_K(false, false, false, false);
#undef GTC_K
}

// Workgroup shape: the waves of a workgroup share one LDS histogram and each owns a hub map, so
// more waves per workgroup amortise the histogram.  Pick the shape with the most resident waves
// per CU (LDS and registers, from the occupancy API) whose histogram exchange budget still covers
// the largest hub.
static int plan_triplet(const void *kfn, const TripletArgs &a, size_t fixed, bool gh,
                        int64_t n_hubs, unsigned long long max_hub_hits, TripletPlan &pl) {
    DeviceLimits dl;
    GTC_TRY(device_limits(dl));
    int best_waves = 0, best_per_cu = 0;
    size_t best_lds = 0;
    for (int waves = 16; waves >= 1; waves >>= 1) {
        const size_t lds = fixed + (size_t)waves * a.wave_bytes;
        if (lds > dl.lds_per_block) continue;
        if (!gh && max_hub_hits >= (0xffffffffull / (unsigned long long)waves) / 2) continue;
        if (lds > 65536)
            GTC_HIP_CHECK(hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
        int per_cu = 0;
        GTC_HIP_CHECK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, waves * kWave, lds));
        if (per_cu * waves > best_per_cu * best_waves) {
            best_waves = waves;
            best_per_cu = per_cu;
            best_lds = lds;
        }
    }
    if (best_waves == 0) {
        set_error("3pCF needs more LDS per workgroup than the device allows (histogram %d configs, "
                  "%d bytes per wave, %zu available) or a hub is too large for 32-bit LDS bins",
                  a.ncfg, a.wave_bytes, dl.lds_per_block);
        return GTC_E_UNSUPPORTED;
    }
    int64_t blocks = (int64_t)dl.cus * best_per_cu;
    const int64_t need = (n_hubs + best_waves - 1) / best_waves;
    if (blocks > need) blocks = need;
    if (blocks < 1) blocks = 1;
    pl.waves = best_waves;
    pl.lds = best_lds;
    pl.blocks = (int)blocks;
    pl.per_cu = best_per_cu;
    return GTC_OK;
}

static int launch_triplet(const void *kfn, TripletArgs &a, const TripletPlan &pl, hipStream_t s) {
    void *args[] = {&a};
    GTC_HIP_CHECK(hipLaunchKernel(kfn, dim3(pl.blocks), dim3(pl.waves * kWave), args, pl.lds, s));
    return GTC_OK;
}

// Band table of the banded walk for a grid of g >= 3 cells per axis: for a spoke in hub slot s,
// its forward cell slots [tlo, thi) whose keys fall in the hub's key run q; and smax[q], the first
// hub slot whose spokes cannot reach run q.  Key offsets of the 14 forward slots relative to the
// cell: own cell, +x, then the rows (dz, dy) = (0, 1), (1, -1), (1, 0), (1, 1) of three cells.
static void band_table(int64_t g, uint8_t out[145]) {
    const int64_t gg = g * g;
    const int64_t off[14] = {0, 1, g - 1, g, g + 1, gg - g - 1, gg - g, gg - g + 1,
                             gg - 1, gg, gg + 1, gg + g - 1, gg + g, gg + g + 1};
    const int64_t lo[5] = {0, g - 1, gg - g - 1, gg - 1, gg + g - 1};
    for (int q = 0; q < 5; ++q) {
        const int64_t hi = lo[q] + (q == 0 ? 2 : 3);
        int smax = 0;
        for (int sj = 0; sj < 14; ++sj) {
            int tlo = 14, thi = 14;
            for (int t = 13; t >= 0; --t) {
                if (off[sj] + off[t] >= lo[q]) tlo = t;
                if (off[sj] + off[t] >= hi) thi = t;
            }
            out[sj * 5 + q] = (uint8_t)tlo;
            out[70 + sj * 5 + q] = (uint8_t)thi;
            if (off[sj] < hi) smax = sj + 1;
        }
        out[140 + q] = (uint8_t)smax;
    }
}

int gather_weights(const gtc_graph_s *G, const double *d_w, double *w_s, unsigned long long *d_m,
                   int32_t *d_bad, double *maxabs, hipStream_t s);

int count_3pcf_device(gtc_graph_s *G, const double *d_w, uint64_t *d_counts, double *d_weighted,
                      gtc_stats *st, hipStream_t s, const HubSubset *sub,
                      const ExternalScratch *ext) {
    // hubs to count: the graph's (per window), or a caller's subset (one-window graphs)
    const int32_t *hub_list = sub ? sub->hubs : G->hubs;
    const int64_t hub_total = sub ? sub->n_hubs : G->n_hubs;
    const int64_t sub_win[2] = {0, sub ? sub->n_hubs : 0};
    const int64_t *win_hubs = sub ? sub_win : G->win_hubs.data();
    if (ext && G->windowed()) {
        set_error("the allocation-free count needs the CSR in device memory (csr_mode device)");
        return GTC_E_UNSUPPORTED;
    }
    const bool timed = ext == nullptr;  // events and the closing readback (allocating counts only)
    const bool W = d_w != nullptr;
    const int nb = G->nb;
    const int64_t ncfg = gtc_num_configs(3, nb);
    GTC_TRY(fill_u64(d_counts, ncfg, 0ull, s));

    // one block for the call's device scratch: internal-order weights, sum limbs, the hub class
    // queue
    double *w_s = nullptr;
    unsigned long long *limbs = nullptr, *d_maxabs = nullptr;
    int32_t *d_bad = nullptr;
    unsigned int *queue = nullptr, *qcount = nullptr;
    constexpr int kSlots = 3;  // out-of-core window buffers: a tile's two windows and the next one
    int32_t *wcol[kSlots] = {};
    uint8_t *wbin[kSlots] = {};
    void *scratch = nullptr;
    int rc = GTC_OK;
    int scale = 0;
    auto cleanup = [&]() { dev_free(scratch, s); };
#define STEP(expr) do { rc = (expr); if (rc) { cleanup(); return rc; } } while (0)
#define STEP_HIP(call) do { hipError_t e_ = (call); if (e_ != hipSuccess) { rc = hip_fail(e_, #call, __FILE__, __LINE__); cleanup(); return rc; } } while (0)

    auto layout = [&](Carver &c) {
        if (W) {
            c.take(&w_s, G->n);
            c.take(&limbs, 4 * ncfg);
            c.take(&d_maxabs, 1);
            c.take(&d_bad, 1);
        }
        c.take(&queue, (size_t)kQueueWords);
        c.take(&qcount, kHubClasses);
    };
    // out-of-core windows live in the graph's three window buffers
    for (int b2 = 0; b2 < kSlots; ++b2) {
        wcol[b2] = G->slot_col[b2];
        wbin[b2] = G->slot_bin[b2];
    }
    if (ext) {
        Carver need;
        layout(need);
        if (need.off > ext->bytes) {
            set_error("the count needs %zu bytes of device scratch; the static buffer holds %zu "
                      "(weighted counts take 8 bytes per point)", need.off, ext->bytes);
            return GTC_E_UNSUPPORTED;
        }
        Carver give;
        give.base = ext->base;
        layout(give);
    } else {
        STEP(carve_alloc(&scratch, s, layout));
    }
    if (W) {
        double maxabs = 0.0;
        STEP(gather_weights(G, d_w, w_s, d_maxabs, d_bad, &maxabs, s));
        STEP(weight_scale(maxabs, 3, &scale));
        STEP(fill_u64(reinterpret_cast<uint64_t *>(limbs), 4 * ncfg, 0ull, s));
    }

    TripletArgs a{};
    a.row_ptr = G->row_ptr;
    a.col_h = G->col;
    a.bin_h = G->bin;
    a.base_h = 0;
    a.col_s = G->col;
    a.bin_s = G->bin;
    a.base_s = 0;
    a.e_split = INT64_MAX;
    a.base_s2 = 0;
    a.s_lo = 0;
    a.s_hi = (int32_t)G->n;
    a.hubs = hub_list;
    a.n_hubs = (int32_t)hub_total;
    a.nb = nb;
    a.ncfg = (int32_t)ncfg;
    // Walk mode: banded (per key run, one-subtraction map offsets) for grids of >= 3 cells per axis
    // with long spoke rows; otherwise one map over the whole hub domain.  GTC_TRIPLET_MODE=flat or
    // banded forces a mode (banded needs >= 3 cells per axis).
    const double avg_len = G->walks > 0 ? (double)G->spoke_elements / (double)G->walks : 0.0;
    bool banded = G->grid.g >= 3 && avg_len >= 64.0;
    if (const char *env = std::getenv("GTC_TRIPLET_MODE")) {
        if (!std::strcmp(env, "flat")) banded = false;
        else if (!std::strcmp(env, "banded")) banded = G->grid.g >= 3;
    }
    if (banded) band_table(G->grid.g, a.band);
    a.slot_off = G->slot_off;
    a.max_m = (int32_t)std::max<int64_t>(G->max_deg, 1);
    // (banded: the band and a zero entry on each side, which out-of-band labels read)
    // (flat: the domain and a zero entry before each of its five runs and at the end)
    const int64_t map_labels = banded ? G->max_band + 2 : G->max_domain + 6;
    a.map_bytes = (int32_t)align_up(map_entry_bytes(W) * (size_t)map_labels, 16);
    a.wave_bytes = (int32_t)(a.map_bytes + chunk_bytes(W, false) + hubrow_bytes(W, a.max_m));
    if (W && G->max_deg >= 32768) {
        set_error("weighted 3pCF: a forward row of %lld entries exceeds the LDS address range of "
                  "the weighted map",
                  (long long)G->max_deg);
        cleanup();
        return GTC_E_UNSUPPORTED;
    }
    a.key_s = G->key_s;
    a.cell_start = G->cell_start;
    a.work = G->work;
    a.gr = G->grid;
    a.w_s = w_s;
    a.two_s = std::ldexp(1.0, scale);
    a.queue = queue;
    a.qcount = qcount;
    a.counts = reinterpret_cast<unsigned long long *>(d_counts);
    a.limbs = limbs;

    float kms = 0.f, h2d_ms = 0.f;
    TripletPlan used{};
    int64_t slot_win_end[kSlots] = {-2, -2, -2};  // windows in the buffers after the tiles
    bool uh_used = false, deep_used = false;
    int64_t tiles_run = 0;
    std::vector<hipEvent_t> kev, cev;  // kernel and copy event pairs
    // out-of-core: window uploads run on a copy stream; per window buffer, `ready` marks its upload
    // done and `done` the last kernel that read it
    hipStream_t cs = nullptr;
    hipEvent_t slot_ready[kSlots] = {}, slot_done[kSlots] = {};
    auto cleanup_tiles = [&]() {
        if (cs) (void)hipStreamSynchronize(cs);  // (the graph's transfer stream)
        for (int k = 0; k < kSlots; ++k) {
            if (slot_ready[k]) (void)hipEventDestroy(slot_ready[k]);
            if (slot_done[k]) (void)hipEventDestroy(slot_done[k]);
        }
        for (auto e : kev) (void)hipEventDestroy(e);
        for (auto e : cev) (void)hipEventDestroy(e);
        kev.clear();
        cev.clear();
    };
#define TSTEP(expr) do { rc = (expr); if (rc) { cleanup_tiles(); cleanup(); return rc; } } while (0)
#define TSTEP_HIP(call) do { hipError_t e_ = (call); if (e_ != hipSuccess) { rc = hip_fail(e_, #call, __FILE__, __LINE__); cleanup_tiles(); cleanup(); return rc; } } while (0)
    auto event_pair = [&](std::vector<hipEvent_t> &v) -> int {
        hipEvent_t e0, e1;
        GTC_HIP_CHECK(hipEventCreate(&e0));
        GTC_HIP_CHECK(hipEventCreate(&e1));
        v.push_back(e0);
        v.push_back(e1);
        return GTC_OK;
    };
    if (hub_total > 0) {
        // LDS histogram unless it would take more than half of a workgroup's LDS, or a single hub
        // could overflow its 32-bit bins
        DeviceLimits dl;
        TSTEP(device_limits(dl));
        const unsigned long long max_hub_hits =
            (unsigned long long)G->max_deg * (unsigned long long)(G->max_deg - 1) / 2;
        const bool GH = triplet_lds_fixed(a.ncfg, a.ncfg, W, false) > dl.lds_per_block / 2 ||
                        max_hub_hits >= 0x7fffffffull / 2;
        // Unweighted with at most 32 bins: histogram over the unsorted bin triple (nb^3 <= 32768
        // bins) when the spoke elements per CU amortise folding nb^3 bins per workgroup.  Its
        // exchange budget counts walked elements (at most max_deg^2 per hub), not hits.
        // GTC_TRIPLET_HIST=unsorted or sorted forces the choice (unsorted needs the same limits).
        const int64_t walk_elems = sub ? sub->spoke_elements : G->spoke_elements;
        const int64_t nb3 = (int64_t)nb * nb * nb;
        const unsigned long long max_hub_elems =
            (unsigned long long)G->max_deg * (unsigned long long)G->max_deg;
        const bool uh_ok = !W && !GH && nb <= kUnsortedMaxBins &&
                           max_hub_elems < (0xffffffffull / 16) / 2;
        bool UH = uh_ok && walk_elems >= nb3 * 1024 * (int64_t)dl.cus;
        if (const char *env = std::getenv("GTC_TRIPLET_HIST")) {
            if (!std::strcmp(env, "unsorted")) UH = uh_ok;
            else if (!std::strcmp(env, "sorted")) UH = false;
        }
        // (the sorted histogram's walk keeps an owner word per spoke of a chunk)
        a.wave_bytes = (int32_t)(a.map_bytes + chunk_bytes(W, UH) + hubrow_bytes(W, a.max_m));
        TripletPlan pl;
        const void *kfn = triplet_kernel(W, GH, banded, G->packed, UH);
        const unsigned long long max_hub_adds = UH ? max_hub_elems : max_hub_hits;
        // two copies of the unsorted histogram, or of the weighted counts and low limbs, when they
        // cost no waves per CU (GTC_TRIPLET_COPIES)
        a.hist_copies = 1;
        int nhist = UH ? nb * unsorted_row(nb) : a.ncfg;
        TSTEP(plan_triplet(kfn, a, triplet_lds_fixed(nhist, a.ncfg, W, GH), GH, hub_total, max_hub_adds, pl));
        if ((UH || W) && !GH) {
            TripletPlan p2;
            int copies = -1;
            if (const char *env = std::getenv("GTC_TRIPLET_COPIES")) copies = std::atoi(env) == 2 ? 2 : 1;
            const bool fits = triplet_lds_fixed(2 * nhist, a.ncfg, W, GH) + (size_t)a.wave_bytes <=
                              (size_t)dl.lds_per_block;
            if (copies != 1 && fits) {
                TSTEP(plan_triplet(kfn, a, triplet_lds_fixed(2 * nhist, a.ncfg, W, GH), GH, hub_total,
                                   max_hub_adds, p2));
            }
            if (copies != 1 && fits && (copies == 2 || p2.per_cu * p2.waves >= pl.per_cu * pl.waves)) {
                a.hist_copies = 2;
                nhist *= 2;
                pl = p2;
            }
        }
        // the unsorted histogram's LDS leaves room for at most 16 waves per CU: twice the loads in
        // flight per lane (GTC_TRIPLET_DEEP=0 or 1 forces the choice)
        bool deep = UH && banded && pl.per_cu * pl.waves <= 16;
        if (const char *env = std::getenv("GTC_TRIPLET_DEEP")) deep = UH && banded && std::atoi(env) != 0;
        if (deep) {
            kfn = triplet_kernel(W, GH, banded, G->packed, UH, true);
            TSTEP(plan_triplet(kfn, a, triplet_lds_fixed(nhist, a.ncfg, W, GH), GH, hub_total, max_hub_adds, pl));
        }
        // 32-bit LDS bins: all waves of a workgroup together stay below 2^32 between exchanges
        const unsigned long long budget = 0xffffffffull / (unsigned long long)pl.waves;
        a.flush_at = GH ? 0u : (unsigned int)(budget - max_hub_adds);
        // GTC_TRIPLET_FLUSH_AT=n exchanges the LDS histogram at least every n hits of a wave
        if (const char *env = std::getenv("GTC_TRIPLET_FLUSH_AT")) {
            const long long v = std::atoll(env);
            if (!GH && v > 0 && (unsigned long long)v < a.flush_at) a.flush_at = (unsigned int)v;
        }
        used = pl;
        uh_used = UH;
        deep_used = deep;

        // Tile loop (§III.5.3): hub window h against search windows s = h .. smax(h).  A walk
        // (i, j) runs in the tile (window of i, window of j) only; a resident untiled graph is one
        // tile over all spokes.
        const int64_t nw = (int64_t)G->win.size() - 1;
        const bool ooc = G->windowed();
        const std::vector<int64_t> &hr = G->win_e;  // CSR offsets of the window bounds
        // Out-of-core window buffers.  Each tile needs its hub window and its search window in a
        // buffer; while a tile's kernel runs, the next tile's missing window is uploaded (pinned
        // host CSR) or emitted again (no stored CSR) on a second stream, into a buffer no running
        // or next tile needs (§III.5.3, double buffering).
        int64_t slot_win[kSlots], slot_used[kSlots];
        bool slot_read[kSlots] = {};
        for (int k = 0; k < kSlots; ++k) {
            slot_win[k] = ooc ? G->slot_win[k] : -1;  // windows left by the build or a count
            slot_used[k] = -1;
        }
        // window stream: uploads overlap the counting on the graph's upload stream, each after
        // its window's download into the pinned CSR and after the download out of the buffer it
        // overwrites; re-emits run on the counting stream (a pair-search kernel beside the
        // persistent enumeration kernel only takes compute units)
        hipStream_t wst = s;
        if (G->host_csr) {
            cs = G->upl;
            wst = cs;
        }
        if (ooc) {
            for (int k = 0; k < kSlots; ++k) {
                TSTEP_HIP(hipEventCreateWithFlags(&slot_ready[k], hipEventDisableTiming));
                TSTEP_HIP(hipEventCreateWithFlags(&slot_done[k], hipEventDisableTiming));
            }
            // the windows already in the buffers are ready once the build's emits are
            if (G->staged) TSTEP_HIP(hipStreamWaitEvent(s, G->staged, 0));
            for (int k = 0; k < kSlots; ++k)
                if (slot_win[k] >= 0) TSTEP_HIP(hipEventRecord(slot_ready[k], s));
            // the buffers' contents are undefined until this count completes
            for (int k = 0; k < kSlots; ++k) G->slot_win[k] = -1;
        }
        // buffer holding window w, uploading it if needed; windows in keep[] are not evicted.
        // Returns -1 when every buffer holds a kept window.
        auto ensure = [&](int64_t w, const int64_t *keep, int nkeep, int64_t tick, int *slot) -> int {
            *slot = -1;
            for (int k = 0; k < kSlots; ++k)
                if (slot_win[k] == w) {
                    *slot = k;
                    slot_used[k] = tick;
                    return GTC_OK;
                }
            int victim = -1;
            for (int k = 0; k < kSlots; ++k) {
                bool kept = false;
                for (int q = 0; q < nkeep; ++q) kept |= slot_win[k] == keep[q];
                if (kept) continue;
                if (victim < 0 || slot_used[k] < slot_used[victim]) victim = k;
            }
            if (victim < 0) return GTC_OK;
            const int64_t e0 = hr[w], ne = hr[w + 1] - e0;
            if (slot_read[victim]) GTC_HIP_CHECK(hipStreamWaitEvent(wst, slot_done[victim], 0));
            if (G->host_csr && ne > 0) {
                // the window's download, and the build's download out of this buffer
                const int64_t held = slot_win[victim];
                if (held >= 0 && held < (int64_t)G->win_dl.size() && G->win_dl[held])
                    GTC_HIP_CHECK(hipStreamWaitEvent(wst, G->win_dl[held], 0));
                if (w < (int64_t)G->win_dl.size() && G->win_dl[w])
                    GTC_HIP_CHECK(hipStreamWaitEvent(wst, G->win_dl[w], 0));
            }
            GTC_TRY(event_pair(cev));
            GTC_HIP_CHECK(hipEventRecord(cev[cev.size() - 2], wst));
            if (ne > 0 && G->rebuild) {  // emit the window again from the coordinates
                GTC_TRY(emit_window(G, w, wcol[victim], wbin[victim], wst));
            } else if (ne > 0) {
                GTC_HIP_CHECK(hipMemcpyAsync(wcol[victim], G->h_col + e0, sizeof(int32_t) * ne,
                                             hipMemcpyHostToDevice, wst));
                if (!G->packed)
                    GTC_HIP_CHECK(hipMemcpyAsync(wbin[victim], G->h_bin + e0, ne,
                                                 hipMemcpyHostToDevice, wst));
            }
            GTC_HIP_CHECK(hipEventRecord(cev.back(), wst));
            GTC_HIP_CHECK(hipEventRecord(slot_ready[victim], wst));
            slot_win[victim] = w;
            slot_used[victim] = tick;
            *slot = victim;
            return GTC_OK;
        };
        // Launches, hub windows from the last down (the build leaves the last windows in the
        // buffers).  A launch takes hub window h with search windows sa..sb, sb <= sa + 1: with
        // the CSR on the device, every search window of h at once; out of core, windows h and
        // h + 1 together (two buffers, the third takes the next launch's window meanwhile), then
        // each further search window on its own.  Two windows share a launch when their buffers
        // lie the same number of entries apart in col and bin (the build lays them out so).
        struct Launch { int64_t h, sa, sb; };
        std::vector<Launch> tiles;
        const bool span_ok = !ooc || G->packed ||
            ((intptr_t)wcol[1] - (intptr_t)wcol[0]) / 4 == (intptr_t)wbin[1] - (intptr_t)wbin[0] &&
            ((intptr_t)wcol[2] - (intptr_t)wcol[0]) / 4 == (intptr_t)wbin[2] - (intptr_t)wbin[0];
        for (int64_t h = nw - 1; h >= 0; --h) {
            if (win_hubs[h + 1] <= win_hubs[h]) continue;
            const int64_t smax = G->win_smax[h];
            if (!ooc) {
                tiles.push_back({h, h, smax});
                continue;
            }
            int64_t sw = h;
            if (span_ok && smax > h) {
                tiles.push_back({h, h, h + 1});
                sw = h + 2;
            }
            for (; sw <= smax; ++sw) tiles.push_back({h, sw, sw});
        }
        for (size_t t = 0; t < tiles.size(); ++t) {
            const int64_t h = tiles[t].h, sa = tiles[t].sa, sb = tiles[t].sb;
            const int64_t nh = win_hubs[h + 1] - win_hubs[h];
            int kh = -1, ka = -1, kb = -1;
            if (ooc) {
                const int64_t keep[3] = {h, sa, sb};
                TSTEP(ensure(h, keep, 3, (int64_t)t, &kh));
                TSTEP(ensure(sa, keep, 3, (int64_t)t, &ka));
                TSTEP(ensure(sb, keep, 3, (int64_t)t, &kb));
                if (kh < 0 || ka < 0 || kb < 0) {
                    set_error("3pCF tiles: no window buffer free for window %lld", (long long)sb);
                    cleanup_tiles();
                    cleanup();
                    return GTC_E_HIP;
                }
                TSTEP_HIP(hipStreamWaitEvent(s, slot_ready[kh], 0));
                if (ka != kh) TSTEP_HIP(hipStreamWaitEvent(s, slot_ready[ka], 0));
                if (kb != kh && kb != ka) TSTEP_HIP(hipStreamWaitEvent(s, slot_ready[kb], 0));
            }
            if (t == 0 || tiles[t - 1].h != h) {
                a.hubs = hub_list + win_hubs[h];
                a.n_hubs = (int32_t)nh;
                TSTEP(hub_class_counts(a.hubs, nh, G->row_ptr, G->work, qcount, s));
            }
            a.col_h = ooc ? wcol[kh] : G->col;
            a.bin_h = ooc ? wbin[kh] : G->bin;
            a.base_h = ooc ? hr[h] : 0;
            a.col_s = ooc ? wcol[ka] : G->col;
            a.bin_s = ooc ? wbin[ka] : G->bin;
            a.base_s = ooc ? hr[sa] : 0;
            a.e_split = ooc && sb != sa ? hr[sb] : INT64_MAX;
            a.base_s2 = ooc && sb != sa ? hr[sb] - ((intptr_t)wcol[kb] - (intptr_t)wcol[ka]) / 4 : 0;
            a.s_lo = nw == 1 ? 0 : (int32_t)G->win[sa];
            a.s_hi = nw == 1 ? (int32_t)G->n : (int32_t)G->win[sb + 1];
            TSTEP(fill_u32(queue, kQueueWords, 0u, s));
            TripletPlan tp = pl;
            tp.blocks = (int)std::min<int64_t>(pl.blocks, (nh + pl.waves - 1) / pl.waves);
            // banded: one queue entry per hub and key run, a group of one XCD's waves' worth of
            // hubs at a time (GTC_BAND_GROUP=n sets the group, 0 takes whole hubs)
            a.band_group = banded ? (unsigned int)std::max<int64_t>(1, (int64_t)tp.blocks * tp.waves / kQueueParts) : 0u;
            if (const char *env = std::getenv("GTC_BAND_GROUP"); env && banded)
                a.band_group = (unsigned int)std::max(0LL, std::atoll(env));
            a.batch_cap = batch_cap(a.band_group ? 5 * nh : nh, (int64_t)tp.blocks * tp.waves);
            if (timed) {
                TSTEP(event_pair(kev));
                TSTEP_HIP(hipEventRecord(kev[kev.size() - 2], s));
            }
            TSTEP(launch_triplet(kfn, a, tp, s));
            if (timed) TSTEP_HIP(hipEventRecord(kev.back(), s));
            ++tiles_run;
            if (ooc) {
                const int used_slots[3] = {kh, ka, kb};
                for (int u = 0; u < 3; ++u) {
                    const int k = used_slots[u];
                    if ((u > 0 && k == kh) || (u > 1 && k == ka)) continue;
                    TSTEP_HIP(hipEventRecord(slot_done[k], s));
                    slot_read[k] = true;
                }
                if (t + 1 < tiles.size()) {  // prefetch while this tile runs
                    const Launch &n2 = tiles[t + 1];
                    const int64_t keep[6] = {h, sa, sb, n2.h, n2.sa, n2.sb};
                    int k2;
                    TSTEP(ensure(n2.h, keep, 6, (int64_t)t + 1, &k2));
                    TSTEP(ensure(n2.sa, keep, 6, (int64_t)t + 1, &k2));
                    TSTEP(ensure(n2.sb, keep, 6, (int64_t)t + 1, &k2));
                }
            }
        }
        if (ooc)
            for (int k = 0; k < kSlots; ++k) slot_win_end[k] = slot_win[k];
    }
    // exact sums to doubles on the device, one rounding per configuration
    if (W)
        TSTEP(finalize_limbs(limbs, ncfg, 1, 4 * ncfg,
                             reinterpret_cast<const unsigned long long *>(d_counts), scale,
                             d_weighted, s));
    if (!timed) {  // caller scratch: asynchronous, no statistics
        cleanup_tiles();
        return GTC_OK;
    }
    std::vector<unsigned long long> h_counts(ncfg);
    TSTEP_HIP(hipMemcpyAsync(h_counts.data(), d_counts, sizeof(uint64_t) * ncfg,
                             hipMemcpyDeviceToHost, s));
    TSTEP_HIP(hipStreamSynchronize(s));
    if (cs) TSTEP_HIP(hipStreamSynchronize(cs));
    if (G->windowed() && slot_win_end[0] != -2)  // the windows the buffers now hold
        for (int k = 0; k < kSlots; ++k) G->slot_win[k] = slot_win_end[k];
    for (size_t e = 0; e + 1 < kev.size(); e += 2) {
        float t = 0.f;
        TSTEP_HIP(hipEventElapsedTime(&t, kev[e], kev[e + 1]));
        kms += t;
    }
    for (size_t e = 0; e + 1 < cev.size(); e += 2) {
        float t = 0.f;
        TSTEP_HIP(hipEventElapsedTime(&t, cev[e], cev[e + 1]));
        h2d_ms += t;
    }
    unsigned long long tri = 0;
    for (auto v : h_counts) tri += v;
    if (st) {
        st->triangles = tri;
        st->merge_walks = sub ? sub->walks : G->walks;
        st->spoke_elements = sub ? sub->spoke_elements : G->spoke_elements;
        st->tiles = tiles_run;
        st->h2d_ms = h2d_ms;
        st->kernel_ms = kms;
        st->weight_scale = scale;
        st->launch_waves = used.waves;
        st->launch_blocks = used.blocks;
        st->launch_lds_bytes = (int32_t)used.lds;
        st->launch_mode = (banded ? 1 : 0) | (uh_used ? 2 : 0) | (deep_used ? 4 : 0);
        // hub rows read once (5 B per entry), spoke rows once per walk (4 B), a bin per triangle
        st->q_alg_bytes = 5.0 * (double)(sub ? sub->walks : G->E) +
                          4.0 * (double)st->spoke_elements + (double)tri;
    }
    cleanup_tiles();
    cleanup();
#undef STEP
#undef STEP_HIP
#undef TSTEP
#undef TSTEP_HIP
    return GTC_OK;
}

}  // namespace gtc

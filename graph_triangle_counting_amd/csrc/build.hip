// build.hip - the neighbour graph on the GPU (GRAMSCI v2 §II.1, Eq.(1); CSR layout §III.5.1).
//
// The pages build a kd-tree on the CPU; here the points are bucketed into cubic cells of side
// >= r_max (cell counts and their scan give the cell starts; stable counting-sort passes over the
// digits of the cell keys, ties in original order, give the internal labels, so they are the same
// on every run), and each point's forward neighbours
// (larger internal label) are found in its own cell and the 13 forward neighbour cells.  Visiting
// those cells in increasing key order emits every row already ascending, so no sort is needed.
// Two passes over the same traversal: count (degrees, then a 64-bit scan to row offsets), emit.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "gtc_internal.h"

namespace gtc {

// forward neighbour cells (dz, dy, dx) > (0, 0, 0), in increasing key order
__constant__ int8_t kFwd[13][3] = {{0, 0, 1},  {0, 1, -1},  {0, 1, 0},  {0, 1, 1},  {1, -1, -1},
                                   {1, -1, 0}, {1, -1, 1},  {1, 0, -1}, {1, 0, 0},  {1, 0, 1},
                                   {1, 1, -1}, {1, 1, 0},   {1, 1, 1}};

__global__ void k_cellkey(const int32_t *__restrict__ xyz, int64_t n, Grid gr,
                          int32_t *__restrict__ key, int32_t *__restrict__ cell_count,
                          int32_t *__restrict__ err) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= n) return;
    int x = xyz[3 * i], y = xyz[3 * i + 1], z = xyz[3 * i + 2];
    if ((unsigned)x >= (unsigned)kGridSide || (unsigned)y >= (unsigned)kGridSide ||
        (unsigned)z >= (unsigned)kGridSide) {
        atomicOr(err, 1);
        x = y = z = 0;
    }
    const int k = ((z / gr.cs) * gr.g + y / gr.cs) * gr.g + x / gr.cs;
    key[i] = k;
    atomicAdd(&cell_count[k], 1);
}

// ---- stable counting sort of the cell keys (ties keep the original order)
//
// The keys are sorted by kDigitBits-bit digits, least significant first; each pass is a stable
// counting sort of one digit.  Tile t (kSortTile consecutive positions of the pass's input) is one
// wave.  k_digit_count writes the tile's count of each digit value to hist[d * tiles + t]; the
// exclusive scan of hist (digit-major) is then the first output slot of each (digit, tile); and
// k_digit_scatter walks its tile in order, 64 positions at a time, giving each element the next
// slot of its digit.  Lanes with the same digit find each other with one ballot per digit bit and
// take slots in lane order, so the output is stable, and after the last pass the keys are sorted
// with ties in original order: the same labels on every run.
constexpr int kDigitBits = 8;
constexpr int kDigits = 1 << kDigitBits;
constexpr int kSortTile = 2048;

__global__ void __launch_bounds__(kWave) k_digit_count(const int32_t *__restrict__ key, int64_t n,
                                                       int shift, int32_t *__restrict__ hist,
                                                       int64_t tiles) {
    __shared__ int32_t cnt[kDigits];
    const int lane = threadIdx.x;
    for (int d = lane; d < kDigits; d += kWave) cnt[d] = 0;
    __syncthreads();
    const int64_t lo = blockIdx.x * (int64_t)kSortTile;
    const int64_t hi = lo + kSortTile < n ? lo + kSortTile : n;
    for (int64_t i = lo + lane; i < hi; i += kWave)
        atomicAdd(&cnt[(key[i] >> shift) & (kDigits - 1)], 1);
    __syncthreads();
    for (int d = lane; d < kDigits; d += kWave) hist[d * tiles + blockIdx.x] = cnt[d];
}

// val_in null: the values are the input positions (the first pass, whose input is in original
// order).
__global__ void __launch_bounds__(kWave) k_digit_scatter(
    const int32_t *__restrict__ key_in, const int32_t *__restrict__ val_in, int64_t n, int shift,
    int bits, const int32_t *__restrict__ slot0, int64_t tiles, int32_t *__restrict__ key_out,
    int32_t *__restrict__ val_out) {
    __shared__ int32_t next[kDigits];
    const int lane = threadIdx.x;
    for (int d = lane; d < kDigits; d += kWave) next[d] = slot0[d * tiles + blockIdx.x];
    __syncthreads();
    const int64_t lo = blockIdx.x * (int64_t)kSortTile;
    const int64_t hi = lo + kSortTile < n ? lo + kSortTile : n;
    for (int64_t base = lo; base < hi; base += kWave) {
        const int64_t i = base + lane;
        const bool valid = i < hi;
        const int32_t k = valid ? key_in[i] : 0;
        const int32_t v = valid ? (val_in ? val_in[i] : (int32_t)i) : 0;
        const int d = (k >> shift) & (kDigits - 1);
        // lanes holding the same digit value
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < bits; ++b) {
            const uint64_t m = __ballot((d >> b) & 1);
            peers &= ((d >> b) & 1) ? m : ~m;
        }
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0));
        int32_t slot = 0;
        if (valid) slot = next[d] + below;
        __syncthreads();  // every lane has read next[] before the group's last lane moves it on
        if (valid) {
            key_out[slot] = k;
            val_out[slot] = v;
            if (below == __popcll(peers) - 1) next[d] = slot + 1;
        }
        __syncthreads();
    }
}

// sorted position r: the point perm[r] (keys sorted, ties in original order) and its coordinates
__global__ void k_scatter(const int32_t *__restrict__ xyz, int64_t n,
                          const int32_t *__restrict__ perm, const int32_t *__restrict__ key_s,
                          int4 *__restrict__ xyz_s) {
    const int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (r >= n) return;
    const int64_t i = perm[r];
    xyz_s[r] = make_int4(xyz[3 * i], xyz[3 * i + 1], xyz[3 * i + 2], key_s[r]);
}

struct PairArgs {
    const int4 *xyz_s;
    const int32_t *cell_start;
    const int64_t *edges;  // [nb+1]
    int32_t nb;
    int32_t n;
    Grid gr;
    int32_t h_lo, h_hi;      // hubs of this launch: labels [h_lo, h_hi)
    int32_t *deg;            // count pass output
    const int64_t *row_ptr;  // emit pass input
    int64_t col_base;        // emit pass: entry e of the CSR is col[e - col_base] (window buffer)
    int32_t *col;
    uint8_t *bin;            // null: packed entries (bin in the top byte of col)
    uint32_t *slot_off;      // emit pass: [n][16] start of each forward cell slot in the row
                             // (null: not written)
};

// Exact squared distance as a double: coordinates differ by < 2^20, squares are < 2^40 and the
// sum < 2^42, so every step is exact in fp64.
__device__ __forceinline__ double sq_dist(const int4 a, const int4 b) {
    const double dx = (double)(a.x - b.x), dy = (double)(a.y - b.y), dz = (double)(a.z - b.z);
    return dx * dx + dy * dy + dz * dz;
}

constexpr int kPairLoads = 8;
constexpr int kPairEdgeSlots = 256;  // >= the largest power of two P with P / 2 < GTC_MAX_BINS

template <bool EMIT>
__global__ void __launch_bounds__(256) k_pairs(PairArgs a) {
    // squared edges as doubles (integers below 2^53), padded with +inf up to a power of two
    // P >= nb: the bin search then takes log2(P) steps of a size the whole wave shares
    __shared__ double se[kPairEdgeSlots];
    int half = 1;  // P / 2 (0 for nb = 1)
    while (2 * half < a.nb) half *= 2;
    if (a.nb == 1) half = 0;
    for (int t = threadIdx.x; t < kPairEdgeSlots; t += blockDim.x)
        se[t] = t <= a.nb ? (double)a.edges[t] : __longlong_as_double(0x7ff0000000000000ll);
    __syncthreads();
    const int64_t ii = a.h_lo + blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (ii >= a.h_hi) return;
    const int32_t i = (int32_t)ii;
    const int4 pi = a.xyz_s[i];
    const int32_t c = pi.w, g = a.gr.g;
    const int32_t cz = c / (g * g), cy = (c / g) % g, cx = c % g;
    const double e0 = se[0], emax = se[a.nb];
    int32_t cnt = 0;
    int64_t w = EMIT ? a.row_ptr[i] - a.col_base : 0;
    auto test = [&](int32_t j, double d2) __attribute__((always_inline)) {
        if (d2 >= e0 && d2 < emax) {
            if (EMIT) {
                int l = 0;  // se[l] <= d2 < se[l + 1]
                for (int h = half; h > 0; h >>= 1)
                    if (d2 >= se[l + h]) l += h;
                if (a.bin) {
                    a.col[w] = j;
                    a.bin[w] = (uint8_t)l;
                } else {
                    a.col[w] = (int32_t)pack_entry(j, l);
                }
                ++w;
            } else {
                ++cnt;
            }
        }
    };
    // candidates of a cell, kPairLoads coordinate loads in flight per lane
    auto scan = [&](int32_t lo, int32_t hi) {
        int32_t j = lo;
        for (; j + kPairLoads <= hi; j += kPairLoads) {
            int4 pj[kPairLoads];
#pragma unroll
            for (int u = 0; u < kPairLoads; ++u) pj[u] = a.xyz_s[j + u];
#pragma unroll
            for (int u = 0; u < kPairLoads; ++u) test(j + u, sq_dist(pj[u], pi));
        }
        for (; j < hi; ++j) test(j, sq_dist(a.xyz_s[j], pi));
    };
    // slot 0: own cell (labels above i); slots 1..13: the forward cells in key order.  The emit
    // pass records where each slot starts in the row (empty slots for cells outside the grid).
    uint32_t so[16];
    const int64_t w0 = w;
    so[0] = 0;
    scan(i + 1, a.cell_start[c + 1]);
    for (int s = 0; s < 13; ++s) {
        so[s + 1] = (uint32_t)(w - w0);
        const int x = cx + kFwd[s][2], y = cy + kFwd[s][1], z = cz + kFwd[s][0];
        if (x < 0 || y < 0 || x >= g || y >= g || z >= g) continue;
        const int32_t cc = (z * g + y) * g + x;
        scan(a.cell_start[cc], a.cell_start[cc + 1]);
    }
    if (!EMIT) {
        a.deg[i] = cnt;
    } else if (a.slot_off) {  // (null when a window is emitted again for counting)
        so[14] = (uint32_t)(w - w0);
        so[15] = 0;
        uint4 *dst = reinterpret_cast<uint4 *>(a.slot_off + (int64_t)i * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = make_uint4(so[4 * q], so[4 * q + 1], so[4 * q + 2], so[4 * q + 3]);
    }
}

// Per-hub statistics, sixteen lanes per hub: work[i] = sum of d+(j) over the row of i, and the
// graph maxima / totals that size the enumeration kernels.
struct StatsOut {
    unsigned long long max_deg;
    unsigned long long max_domain;
    unsigned long long spoke_elements;
    unsigned long long walks;
    unsigned long long n_hubs;
    unsigned long long max_band;
};

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) {
        const unsigned long long o = __shfl_xor(v, d, kWave);
        v = o > v ? o : v;
    }
    return v;
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

__global__ void __launch_bounds__(256)
    k_degstats(int32_t h_lo, int32_t h_hi, const int64_t *__restrict__ row_ptr,
               const int32_t *__restrict__ col, int64_t col_base, uint32_t label_mask,
               const int32_t *__restrict__ deg,
               const int32_t *__restrict__ key_s, const int32_t *__restrict__ cell_start, Grid gr,
               int64_t *__restrict__ work, StatsOut *out, unsigned long long *win_last) {
    constexpr int L = 16;
    __shared__ unsigned long long red[7][256 / kWave];
    const int sub = threadIdx.x & (L - 1);
    const int64_t hub0 = h_lo + (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / L;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x / L;
    unsigned long long my_max_deg = 0, my_max_dom = 0, my_sum = 0, my_walks = 0, my_hubs = 0,
                       my_max_band = 0, my_last = 0;
    for (int64_t h = hub0; h < h_hi; h += stride) {
        const int64_t b = row_ptr[h], e = row_ptr[h + 1];
        int64_t s = 0;
        for (int64_t t = b + sub; t < e; t += L) s += deg[(uint32_t)col[t - col_base] & label_mask];
#pragma unroll
        for (int d = L / 2; d > 0; d >>= 1) s += __shfl_xor(s, d, L);
        if (sub == 0) {
            work[h] = s;
            const int64_t m = e - b;
            my_max_deg = m > (int64_t)my_max_deg ? m : my_max_deg;
            my_sum += s;
            HubDomain dom;
            hub_domain((int32_t)h, key_s[h], gr, cell_start, dom);
            my_max_dom = dom.size > (int64_t)my_max_dom ? dom.size : my_max_dom;
            for (int t = 0; t < 5; ++t) {
                const unsigned long long bs = (unsigned long long)(dom.hi[t] - dom.lo[t]);
                my_max_band = bs > my_max_band ? bs : my_max_band;
            }
            if (m >= 2 && s > 0) {
                my_walks += m;
                my_hubs += 1;
            }
            if (m > 0) {  // largest spoke label of the window: bounds its search windows
                const unsigned long long last =
                    (unsigned long long)((uint32_t)col[e - 1 - col_base] & label_mask);
                my_last = last > my_last ? last : my_last;
            }
        }
    }
    // block reduction, then one atomic per quantity per block
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    my_max_deg = wave_max_u64(my_max_deg);
    my_max_dom = wave_max_u64(my_max_dom);
    my_sum = wave_sum_u64(my_sum);
    my_walks = wave_sum_u64(my_walks);
    my_hubs = wave_sum_u64(my_hubs);
    my_max_band = wave_max_u64(my_max_band);
    my_last = wave_max_u64(my_last);
    if (lane == 0) {
        red[6][wid] = my_last;
        red[5][wid] = my_max_band;
        red[0][wid] = my_max_deg;
        red[1][wid] = my_max_dom;
        red[2][wid] = my_sum;
        red[3][wid] = my_walks;
        red[4][wid] = my_hubs;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long v[7] = {0, 0, 0, 0, 0, 0, 0};
        for (int w = 0; w < (int)(blockDim.x / kWave); ++w) {
            v[6] = red[6][w] > v[6] ? red[6][w] : v[6];
            v[0] = red[0][w] > v[0] ? red[0][w] : v[0];
            v[1] = red[1][w] > v[1] ? red[1][w] : v[1];
            v[2] += red[2][w];
            v[3] += red[3][w];
            v[4] += red[4][w];
            v[5] = red[5][w] > v[5] ? red[5][w] : v[5];
        }
        atomicMax(&out->max_deg, v[0]);
        atomicMax(&out->max_domain, v[1]);
        atomicAdd(&out->spoke_elements, v[2]);
        atomicAdd(&out->walks, v[3]);
        atomicAdd(&out->n_hubs, v[4]);
        atomicMax(&out->max_band, v[5]);
        if (v[6]) atomicMax(win_last, v[6]);
    }
}

// Hub lists: hubs with a possible triangle (d+ >= 2, work > 0), grouped by hub window and, within
// a window, heaviest first by class (floor(log2(work)), hub_class).  A counting sort on the key
// window * kHubClasses + class, aggregated per block in LDS when the keys fit there.
constexpr int kLdsKeys = 4096;

__device__ __forceinline__ int hub_key(int64_t i, const int64_t *__restrict__ row_ptr,
                                       const int64_t *__restrict__ work,
                                       const int64_t *__restrict__ win, int32_t nwin) {
    const int c = hub_class(row_ptr[i + 1] - row_ptr[i], work[i]);
    if (c < 0) return -1;
    int lo = 0, hi = nwin;  // window k holds labels [win[k], win[k+1])
    while (hi - lo > 1) {
        const int md = (lo + hi) >> 1;
        if (win[md] <= i) lo = md; else hi = md;
    }
    return lo * kHubClasses + c;
}

__global__ void __launch_bounds__(256)
    k_bucket_count(int32_t n, const int64_t *__restrict__ row_ptr, const int64_t *__restrict__ work,
                   const int64_t *__restrict__ win, int32_t nwin, int32_t nkeys,
                   int32_t *__restrict__ count) {
    extern __shared__ int32_t loc[];
    const bool lds = nkeys <= kLdsKeys;
    if (lds)
        for (int t = threadIdx.x; t < nkeys; t += blockDim.x) loc[t] = 0;
    __syncthreads();
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < n) {
        const int b = hub_key(i, row_ptr, work, win, nwin);
        if (b >= 0) atomicAdd(lds ? &loc[b] : &count[b], 1);
    }
    __syncthreads();
    if (lds)
        for (int t = threadIdx.x; t < nkeys; t += blockDim.x)
            if (loc[t]) atomicAdd(&count[t], loc[t]);
}

__global__ void __launch_bounds__(256)
    k_bucket_scatter(int32_t n, const int64_t *__restrict__ row_ptr,
                     const int64_t *__restrict__ work, const int64_t *__restrict__ win,
                     int32_t nwin, int32_t nkeys, int32_t *__restrict__ cursor,
                     int32_t *__restrict__ hubs) {
    extern __shared__ int32_t sh[];
    const bool lds = nkeys <= kLdsKeys;
    int32_t *loc = sh, *base = sh + (lds ? nkeys : 0);
    if (lds)
        for (int t = threadIdx.x; t < nkeys; t += blockDim.x) loc[t] = 0;
    __syncthreads();
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    int b = -1;
    int32_t r = 0;
    if (i < n) {
        b = hub_key(i, row_ptr, work, win, nwin);
        if (b >= 0 && lds) r = atomicAdd(&loc[b], 1);
    }
    __syncthreads();
    if (lds) {
        for (int t = threadIdx.x; t < nkeys; t += blockDim.x)
            base[t] = loc[t] ? atomicAdd(&cursor[t], loc[t]) : 0;
        __syncthreads();
        if (b >= 0) hubs[base[b] + r] = (int32_t)i;
    } else if (b >= 0) {
        hubs[atomicAdd(&cursor[b], 1)] = (int32_t)i;
    }
}

__global__ void __launch_bounds__(256)
    k_class_count(const int32_t *__restrict__ hubs, int64_t n_hubs,
                  const int64_t *__restrict__ row_ptr, const int64_t *__restrict__ work,
                  uint32_t *__restrict__ counts) {
    __shared__ uint32_t loc[kHubClasses];
    for (int t = threadIdx.x; t < kHubClasses; t += blockDim.x) loc[t] = 0;
    __syncthreads();
    for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < n_hubs;
         p += (int64_t)gridDim.x * blockDim.x) {
        const int32_t i = hubs[p];
        const int c = hub_class(row_ptr[i + 1] - row_ptr[i], work[i]);
        if (c >= 0) atomicAdd(&loc[c], 1u);
    }
    __syncthreads();
    for (int t = threadIdx.x; t < kHubClasses; t += blockDim.x)
        if (loc[t]) atomicAdd(&counts[t], loc[t]);
}

int hub_class_counts(const int32_t *hubs, int64_t n_hubs, const int64_t *row_ptr,
                     const int64_t *work, uint32_t *counts, hipStream_t s) {
    GTC_TRY(fill_u32(counts, kHubClasses, 0u, s));
    if (n_hubs <= 0) return GTC_OK;
    int64_t blocks = (n_hubs + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(k_class_count, dim3((unsigned)blocks), dim3(256), 0, s, hubs, n_hubs,
                       row_ptr, work, counts);
    GTC_HIP_CHECK(hipGetLastError());
    return GTC_OK;
}

// ------------------------------------------------------------------ host orchestration

// Hub windows (§III.5.3) on the device, the same greedy plan as plan_windows on the host: each
// window runs from the previous bound a to the largest b with row_ptr[b] - row_ptr[a] <= cap (at
// least one row).  One wave searches each bound 64-ary: the 64 probes that hold form a prefix
// (row_ptr is nondecreasing), so their count narrows the range by 64 per round.  Writes the bounds
// and their CSR offsets, bounds[0..W] and bound_e[0..W] (room for max_w + 1 of each), and W to
// *count, or -1 if W would exceed max_w.
__global__ void __launch_bounds__(kWave)
    k_plan_windows(const int64_t *__restrict__ row_ptr, int64_t n, int64_t cap, int64_t max_w,
                   int64_t *__restrict__ bounds, int64_t *__restrict__ bound_e,
                   int64_t *__restrict__ count) {
    const int lane = threadIdx.x;
    int64_t a = 0, W = 0;
    if (lane == 0) {
        bounds[0] = 0;
        bound_e[0] = row_ptr[0];
    }
    while (a < n) {
        const int64_t limit = row_ptr[a] + cap;
        // the bound lies in [lo, hi]: the largest b there with row_ptr[b] <= limit, else lo
        int64_t lo = a + 1, hi = n;
        while (lo < hi) {
            const int64_t step = (hi - lo + kWave - 1) / kWave;
            const int64_t p = lo + (int64_t)(lane + 1) * step;
            const bool ok = p <= hi && row_ptr[p] <= limit;
            const int k = __popcll(__ballot(ok));
            hi = std::min(hi, lo + (int64_t)(k + 1) * step - 1);
            lo += (int64_t)k * step;
        }
        a = lo;
        if (++W > max_w) break;
        if (lane == 0) {
            bounds[W] = a;
            bound_e[W] = row_ptr[a];
        }
    }
    if (lane == 0) *count = W > max_w ? -1 : W;
}

static Grid choose_grid(int64_t n, int64_t r2) {
    // integer cell side cs = ceil(sqrt(r2)), so two neighbours are at most one cell apart per axis
    int64_t cs = (int64_t)std::sqrt((double)r2);
    while (cs * cs < r2) ++cs;
    while (cs > 1 && (cs - 1) * (cs - 1) >= r2) --cs;
    if (cs < 1) cs = 1;
    int64_t g = (kGridSide + cs - 1) / cs;
    // at most ~2n cells (at least 1) and 512 per axis: finer cells than that only cost memory
    int64_t cap = 1;
    while ((cap + 1) * (cap + 1) * (cap + 1) <= 2 * (n > 0 ? n : 1) && cap < 512) ++cap;
    if (g > cap) {
        g = cap;
        cs = (kGridSide + g - 1) / g;
    }
    Grid gr;
    gr.g = (int32_t)g;
    gr.cs = (int32_t)cs;
    gr.ncell = g * g * g;
    return gr;
}

static inline unsigned grid_for(int64_t n, int threads) {
    return (unsigned)((n + threads - 1) / threads);
}

int build_graph_device(gtc_graph_s *G, const int32_t *d_xyz, hipStream_t s) {
    const int64_t n = G->n;
    // packed CSR entries when labels fit 24 bits (GTC_CSR_LAYOUT=split keeps two arrays)
    G->packed = n <= kPackedMaxN;
    if (const char *env = std::getenv("GTC_CSR_LAYOUT"))
        if (!std::strcmp(env, "split")) G->packed = false;
    G->grid = choose_grid(n, G->edges[G->nb]);
    const Grid gr = G->grid;

    // the graph's per-point arrays (hubs: at most one per point)
    GTC_TRY(carve_alloc(&G->arena_pts, s, [&](Carver &c) {
        c.take(&G->d_edges, G->nb + 1);
        c.take(&G->cell_start, gr.ncell + 1);
        c.take(&G->perm, n);
        c.take(&G->key_s, n);
        c.take(&G->row_ptr, n + 1);
        c.take(&G->deg, n);
        c.take(&G->work, n);
        c.take(&G->slot_off, 16 * (size_t)n);
        c.take(&G->hubs, n);
    }));
    GTC_TRY(dev_alloc_n(&G->xyz_s, n, s));
    GTC_HIP_CHECK(hipMemcpyAsync(G->d_edges, G->edges, sizeof(int64_t) * (G->nb + 1),
                                 hipMemcpyHostToDevice, s));

    // build scratch: keys and the sort's ping-pong arrays, cell counts, error flag, stats, scan
    // partials, the sort's digit counts
    int32_t *key = nullptr, *key_t = nullptr, *val_t = nullptr, *val_u = nullptr;
    int32_t *ccount = nullptr, *err = nullptr, *hist = nullptr;
    StatsOut *d_stats = nullptr;
    int64_t *scan_ws = nullptr;
    void *scratch = nullptr;
    int rc = GTC_OK;
    auto cleanup = [&]() { dev_free(scratch, s); };
#define STEP(expr)            \
    do {                      \
        rc = (expr);          \
        if (rc) {             \
            cleanup();        \
            return rc;        \
        }                     \
    } while (0)
#define STEP_HIP(call)                                                   \
    do {                                                                 \
        hipError_t e_ = (call);                                          \
        if (e_ != hipSuccess) {                                          \
            rc = hip_fail(e_, #call, __FILE__, __LINE__);                \
            cleanup();                                                   \
            return rc;                                                   \
        }                                                                \
    } while (0)

    // counting-sort passes over the key digits, only as many bits as the largest key needs
    int key_bits = 1;
    while (key_bits < 31 && ((int64_t)1 << key_bits) < gr.ncell) ++key_bits;
    const int passes = (key_bits + kDigitBits - 1) / kDigitBits;
    const int64_t tiles = (n + kSortTile - 1) / kSortTile;
    const int64_t hist_n = tiles * kDigits;
    const size_t scan_ws_bytes = std::max({scan_workspace_bytes(n), scan_workspace_bytes(gr.ncell),
                                           scan_workspace_bytes(hist_n)});
    STEP(carve_alloc(&scratch, s, [&](Carver &c) {
        c.take(&key, n);
        c.take(&key_t, n);
        c.take(&val_t, n);
        c.take(&val_u, n);
        c.take(&hist, hist_n + 1);
        c.take(&ccount, gr.ncell);
        c.take(&err, 1);
        c.take(&d_stats, 1);
        c.take(&scan_ws, scan_ws_bytes / sizeof(int64_t));
    }));
    STEP(fill_u32(reinterpret_cast<uint32_t *>(ccount), gr.ncell, 0u, s));
    STEP(fill_u32(reinterpret_cast<uint32_t *>(err), 1, 0u, s));
    STEP(fill_u64(reinterpret_cast<uint64_t *>(d_stats), sizeof(StatsOut) / 8, 0ull, s));

    if (n > 0) {
        hipLaunchKernelGGL(k_cellkey, dim3(grid_for(n, 256)), dim3(256), 0, s, d_xyz, n, gr, key,
                           ccount, err);
        STEP_HIP(hipGetLastError());
    }
    STEP(exclusive_scan_i32_to_i32(ccount, G->cell_start, gr.ncell, scan_ws, s));
    if (n > 0) {
        // pass p reads (kin, vin) and writes the next pair; the last pass writes (key_s, perm)
        int32_t *kin = key, *vin = nullptr;
        for (int p = 0; p < passes; ++p) {
            const int shift = p * kDigitBits;
            const int bits = std::min(kDigitBits, key_bits - shift);
            int32_t *kout = p == passes - 1 ? G->key_s : (kin == key_t ? key : key_t);
            int32_t *vout = p == passes - 1 ? G->perm : (vin == val_t ? val_u : val_t);
            hipLaunchKernelGGL(k_digit_count, dim3((unsigned)tiles), dim3(kWave), 0, s, kin, n,
                               shift, hist, tiles);
            STEP_HIP(hipGetLastError());
            STEP(exclusive_scan_i32_to_i32(hist, hist, hist_n, scan_ws, s));
            hipLaunchKernelGGL(k_digit_scatter, dim3((unsigned)tiles), dim3(kWave), 0, s, kin, vin,
                               n, shift, bits, hist, tiles, kout, vout);
            STEP_HIP(hipGetLastError());
            kin = kout;
            vin = vout;
        }
        hipLaunchKernelGGL(k_scatter, dim3(grid_for(n, 256)), dim3(256), 0, s, d_xyz, n, G->perm,
                           G->key_s, G->xyz_s);
        STEP_HIP(hipGetLastError());
    }

    PairArgs pa{};
    pa.xyz_s = G->xyz_s;
    pa.cell_start = G->cell_start;
    pa.edges = G->d_edges;
    pa.nb = G->nb;
    pa.n = (int32_t)n;
    pa.gr = gr;
    pa.deg = G->deg;
    pa.h_lo = 0;
    pa.h_hi = (int32_t)n;
    if (n > 0) {
        hipLaunchKernelGGL(k_pairs<false>, dim3(grid_for(n, 256)), dim3(256), 0, s, pa);
        STEP_HIP(hipGetLastError());
    }
    STEP(exclusive_scan_i32_to_i64(G->deg, G->row_ptr, n, scan_ws, s));

    int32_t h_err = 0;
    STEP_HIP(hipMemcpyAsync(&G->E, G->row_ptr + n, sizeof(int64_t), hipMemcpyDeviceToHost, s));
    STEP_HIP(hipMemcpyAsync(&h_err, err, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    STEP_HIP(hipStreamSynchronize(s));
    if (h_err) {
        set_error("a coordinate is outside [0, 2^20)");
        cleanup();
        return GTC_E_INVALID;
    }
    // Automatic chunking (§III.5.3): a build given no window budget keeps the CSR out of core when
    // it would take more than 3/4 of the free device memory (free memory plus what the stream-
    // ordered pool holds unused; GTC_DEVICE_FREE_BYTES=n replaces that figure, for tests).  The
    // windows are then emitted again per tile (the coordinates are kept) or held in pinned host
    // memory (coordinates dropped), with a budget of 1/8 of the free memory per window.
    if (G->auto_tiles && n > 0) {
        size_t free_b = 0, total_b = 0;
        STEP_HIP(hipMemGetInfo(&free_b, &total_b));
        int dev = 0;
        hipMemPool_t pool;
        if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
            uint64_t reserved = 0, used = 0;
            if (hipMemPoolGetAttribute(pool, hipMemPoolAttrReservedMemCurrent, &reserved) == hipSuccess &&
                hipMemPoolGetAttribute(pool, hipMemPoolAttrUsedMemCurrent, &used) == hipSuccess &&
                reserved > used)
                free_b += reserved - used;
        }
        (void)hipGetLastError();
        if (const char *env = std::getenv("GTC_DEVICE_FREE_BYTES")) {
            const long long v = std::atoll(env);
            if (v > 0) free_b = (size_t)v;
        }
        const int64_t csr_bytes = G->E * (G->packed ? 4 : 5);
        if ((double)csr_bytes > 0.75 * (double)free_b) {
            G->tile_bytes = std::max<int64_t>((int64_t)(free_b / 8), (int64_t)1 << 20);
            if (G->keep_coords_requested) G->rebuild = true;
            else G->host_csr = true;
        }
    }
    // hub windows: one window unless a tile budget is set (§III.5.3)
    G->win.assign({0, n});
    G->win_e.assign({0, G->E});
    G->max_window_edges = G->E;
    if (G->tile_bytes > 0 && n > 0) {
        // Greedy windows, planned on the device: only the bounds travel to the host.  Two
        // consecutive windows hold more than cap entries together (the second's first row did not
        // fit the first), so W <= 2E / (cap + 1) + 1, and W <= n.
        const int64_t cap = G->tile_bytes / (G->packed ? 4 : 5);
        const int64_t max_w = std::min<int64_t>(n, 2 * (G->E / (cap + 1)) + 3);
        int64_t *d_bounds = nullptr, *d_bound_e = nullptr, *d_count = nullptr;
        void *plan_ws = nullptr;
        STEP(carve_alloc(&plan_ws, s, [&](Carver &c) {
            c.take(&d_bounds, max_w + 1);
            c.take(&d_bound_e, max_w + 1);
            c.take(&d_count, 1);
        }));
        hipLaunchKernelGGL(k_plan_windows, dim3(1), dim3(kWave), 0, s, G->row_ptr, n, cap, max_w,
                           d_bounds, d_bound_e, d_count);
        int64_t Wn = 0;
        hipError_t e = hipGetLastError();
        if (e == hipSuccess)
            e = hipMemcpyAsync(&Wn, d_count, sizeof(int64_t), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e == hipSuccess && Wn > 0) {
            G->win.resize(Wn + 1);
            G->win_e.resize(Wn + 1);
            e = hipMemcpyAsync(G->win.data(), d_bounds, sizeof(int64_t) * (Wn + 1),
                               hipMemcpyDeviceToHost, s);
            if (e == hipSuccess)
                e = hipMemcpyAsync(G->win_e.data(), d_bound_e, sizeof(int64_t) * (Wn + 1),
                                   hipMemcpyDeviceToHost, s);
            if (e == hipSuccess) e = hipStreamSynchronize(s);
        }
        dev_free(plan_ws, s);
        if (e != hipSuccess) STEP(hip_fail(e, "window plan", __FILE__, __LINE__));
        if (Wn <= 0) {
            set_error("window plan: more than %lld windows", (long long)max_w);
            cleanup();
            return GTC_E_HIP;
        }
        G->max_window_edges = 0;
        for (int64_t k = 0; k < Wn; ++k)
            G->max_window_edges = std::max(G->max_window_edges, G->win_e[k + 1] - G->win_e[k]);
    }
    const int64_t W = (int64_t)G->win.size() - 1;
    unsigned long long *win_last = nullptr;
    // Out-of-core staging: the graph's three window buffers, which end up holding the last three
    // windows, and with a pinned CSR a fourth buffer for the build alone, so that window
    // downloads (on the graph's transfer stream) overlap the next windows' emits.  A buffer is
    // emitted into again once its download has completed.
    constexpr int kStage = 4;
    int32_t *st_col[kStage] = {};
    uint8_t *st_bin[kStage] = {};
    int64_t st_win[kStage] = {-1, -1, -1, -1};  // window each staging buffer holds
    int64_t st_seq[kStage] = {-1, -1, -1, -1};  // order of its last download (-1: none)
    void *extra_block = nullptr;                // the fourth buffer (freed on the transfer stream)
    hipStream_t cs = nullptr;
    hipEvent_t emitted[kStage] = {}, copied[kStage] = {}, extra_ready = nullptr;
    bool copy_pending[kStage] = {};
    const int64_t nkeys = W * kHubClasses;  // hub-list keys: window * classes + class
    int32_t *key_count = nullptr, *key_start = nullptr;
    int64_t *d_win = nullptr, *key_scan_ws = nullptr;
    void *scratch2 = nullptr;
    auto cleanup2 = [&]() {
        if (cs) (void)hipStreamSynchronize(cs);  // (the stream is the graph's)
        for (int b = 0; b < kStage; ++b) {
            if (emitted[b]) (void)hipEventDestroy(emitted[b]);
            if (copied[b]) (void)hipEventDestroy(copied[b]);
        }
        if (extra_ready) (void)hipEventDestroy(extra_ready);
        if (extra_block) dev_free(extra_block, G->xfer);
        dev_free(scratch2, s);
    };
#define STEP2(expr) do { rc = (expr); if (rc) { cleanup2(); cleanup(); return rc; } } while (0)
#define STEP2_HIP(call) do { hipError_t e_ = (call); if (e_ != hipSuccess) { rc = hip_fail(e_, #call, __FILE__, __LINE__); cleanup2(); cleanup(); return rc; } } while (0)
    STEP2(carve_alloc(&scratch2, s, [&](Carver &c) {
        c.take(&win_last, W);
        c.take(&key_count, nkeys);
        c.take(&key_start, nkeys + 1);
        c.take(&d_win, W + 1);
        c.take(&key_scan_ws, scan_workspace_bytes(nkeys) / sizeof(int64_t));
    }));
    if (G->windowed()) {  // the graph's window buffers, which stage the build's windows
        // buffers of a multiple of 256 entries back to back, labels then bins: buffer b starts
        // b * stride entries after buffer 0 in both arrays, so one launch can address two of them
        const int64_t stride = (std::max<int64_t>(G->max_window_edges, 1) + 255) & ~(int64_t)255;
        STEP2(carve_alloc(&G->slot_block, s, [&](Carver &c) {
            for (int b = 0; b < 3; ++b) c.take(&G->slot_col[b], stride);
            if (!G->packed)
                for (int b = 0; b < 3; ++b) c.take(&G->slot_bin[b], stride);
        }));
        for (int b = 0; b < 3; ++b) {
            st_col[b] = G->slot_col[b];
            st_bin[b] = G->slot_bin[b];
        }
    }
    STEP2(fill_u64(reinterpret_cast<uint64_t *>(win_last), W, 0ull, s));
    if (G->host_csr) {
        // out-of-core: the CSR lives in pinned host memory; each window is emitted into a device
        // staging buffer and copied out
        STEP2(host_alloc_pinned(reinterpret_cast<void **>(&G->h_col),
                                sizeof(int32_t) * std::max<int64_t>(G->E, 1)));
        if (!G->packed)
            STEP2(host_alloc_pinned(reinterpret_cast<void **>(&G->h_bin),
                                    std::max<int64_t>(G->E, 1)));
        STEP2_HIP(hipStreamCreateWithFlags(&G->xfer, hipStreamNonBlocking));
        STEP2_HIP(hipStreamCreateWithFlags(&G->upl, hipStreamNonBlocking));
        G->win_dl.assign(W, nullptr);
        cs = G->xfer;
        for (int b = 0; b < kStage; ++b) {
            STEP2_HIP(hipEventCreateWithFlags(&emitted[b], hipEventDisableTiming));
            STEP2_HIP(hipEventCreateWithFlags(&copied[b], hipEventDisableTiming));
        }
        if (W > 3) {  // windows that do not stay on the device: the fourth buffer stages one
            STEP2(carve_alloc(&extra_block, cs, [&](Carver &c) {
                c.take(&st_col[3], G->max_window_edges);
                if (!G->packed) c.take(&st_bin[3], G->max_window_edges);
            }));
            STEP2_HIP(hipEventCreateWithFlags(&extra_ready, hipEventDisableTiming));
            STEP2_HIP(hipEventRecord(extra_ready, cs));
            STEP2_HIP(hipStreamWaitEvent(s, extra_ready, 0));
        }
    } else if (!G->rebuild) {  // (rebuild: the emit pass only feeds the statistics)
        STEP2(carve_alloc(&G->arena_csr, s, [&](Carver &c) {
            c.take(&G->col, G->E);
            if (!G->packed) c.take(&G->bin, G->E);
        }));
    }
    pa.row_ptr = G->row_ptr;
    pa.slot_off = G->slot_off;
    // Emit order.  A pinned CSR: the windows that leave the device first, then the three that
    // stay from the last down, so that their downloads end in the order a count (which walks hub
    // windows from the last down) gives their buffers up to its uploads.
    std::vector<int64_t> order(W);
    for (int64_t k = 0; k < W; ++k) order[k] = k;
    if (G->host_csr && W > 3) std::reverse(order.end() - 3, order.end());
    for (int64_t oi = 0; oi < W && n > 0; ++oi) {
        const int64_t k = order[oi];
        const int64_t lo = G->win[k], hi = G->win[k + 1];
        if (hi <= lo) continue;
        const int64_t e_lo = G->windowed() ? G->win_e[k] : 0;
        // staging buffer of this window.  Resident or re-emitted windows: the three in turn.  A
        // pinned CSR: the last window that leaves the device takes the fourth buffer, earlier
        // ones the three in turn, and each of the last three windows the buffer among the three
        // whose download was queued first, so that the emits wait for the earliest downloads.
        int sb = (int)(k % 3);
        if (G->host_csr && W > 3) {
            if (k == W - 4) {
                sb = 3;
            } else if (k > W - 4) {
                sb = -1;
                for (int b = 0; b < 3; ++b) {
                    if (st_win[b] >= W - 3) continue;  // holds a window that stays
                    if (sb < 0 || st_seq[b] < st_seq[sb]) sb = b;
                }
            }
        }
        st_win[sb] = k;
        if (G->host_csr && copy_pending[sb])  // its previous window has been downloaded
            STEP2_HIP(hipStreamWaitEvent(s, copied[sb], 0));
        pa.h_lo = (int32_t)lo;
        pa.h_hi = (int32_t)hi;
        pa.col_base = e_lo;
        pa.col = G->windowed() ? st_col[sb] : G->col;
        pa.bin = G->windowed() ? st_bin[sb] : G->bin;
        hipLaunchKernelGGL(k_pairs<true>, dim3(grid_for(hi - lo, 256)), dim3(256), 0, s, pa);
        STEP2_HIP(hipGetLastError());
        const int64_t dsb = std::min<int64_t>(((hi - lo) * 16 + 255) / 256, 2048);
        hipLaunchKernelGGL(k_degstats, dim3((unsigned)dsb), dim3(256), 0, s, (int32_t)lo,
                           (int32_t)hi, G->row_ptr, (const int32_t *)pa.col, e_lo,
                           G->packed ? kLabelMask : 0xffffffffu, G->deg, G->key_s,
                           G->cell_start, gr, G->work, d_stats, win_last + k);
        STEP2_HIP(hipGetLastError());
        if (G->host_csr) {
            const int64_t ne = G->win_e[k + 1] - e_lo;
            if (ne > 0) {
                STEP2_HIP(hipEventRecord(emitted[sb], s));
                STEP2_HIP(hipStreamWaitEvent(cs, emitted[sb], 0));
                STEP2_HIP(hipMemcpyAsync(G->h_col + e_lo, st_col[sb], sizeof(int32_t) * ne,
                                         hipMemcpyDeviceToHost, cs));
                if (!G->packed)
                    STEP2_HIP(hipMemcpyAsync(G->h_bin + e_lo, st_bin[sb], ne,
                                             hipMemcpyDeviceToHost, cs));
                STEP2_HIP(hipEventRecord(copied[sb], cs));
                STEP2_HIP(hipEventCreateWithFlags(&G->win_dl[k], hipEventDisableTiming));
                STEP2_HIP(hipEventRecord(G->win_dl[k], cs));
                copy_pending[sb] = true;
                st_seq[sb] = oi;
            }
        }
    }
    if (extra_block) {  // freed in order after its downloads
        dev_free(extra_block, cs);
        extra_block = nullptr;
    }
    StatsOut hs{};
    std::vector<unsigned long long> h_last(W);
    STEP2_HIP(hipMemcpyAsync(&hs, d_stats, sizeof(hs), hipMemcpyDeviceToHost, s));
    STEP2_HIP(hipMemcpyAsync(h_last.data(), win_last, sizeof(unsigned long long) * W,
                             hipMemcpyDeviceToHost, s));
    STEP2_HIP(hipStreamSynchronize(s));
    G->max_deg = (int64_t)hs.max_deg;
    G->max_domain = (int64_t)hs.max_domain;
    G->spoke_elements = (int64_t)hs.spoke_elements;
    G->walks = (int64_t)hs.walks;
    G->n_hubs = (int64_t)hs.n_hubs;
    G->max_band = (int64_t)hs.max_band;
    // search windows of each hub window: from itself to the window of its largest spoke label
    G->win_smax.assign(W, 0);
    for (int64_t k = 0; k < W; ++k) {
        const int64_t last = std::max<int64_t>((int64_t)h_last[k], G->win[k]);
        const int64_t t = std::upper_bound(G->win.begin(), G->win.end(), last) - G->win.begin() - 1;
        G->win_smax[k] = (int32_t)std::min<int64_t>(std::max<int64_t>(t, k), W - 1);
    }

    // hub lists by (window, class): window k's hubs are hubs[win_hubs[k], win_hubs[k+1])
    G->win_hubs.assign(W + 1, 0);
    G->win_hubs[W] = G->n_hubs;
    if (n > 0 && G->n_hubs > 0) {
        if (nkeys > INT32_MAX / 2) {
            set_error("too many hub windows (%lld)", (long long)W);
            cleanup2();
            cleanup();
            return GTC_E_UNSUPPORTED;
        }
        STEP2_HIP(hipMemcpyAsync(d_win, G->win.data(), sizeof(int64_t) * (W + 1),
                                 hipMemcpyHostToDevice, s));
        STEP2(fill_u32(reinterpret_cast<uint32_t *>(key_count), nkeys, 0u, s));
        const size_t lds_keys = nkeys <= kLdsKeys ? sizeof(int32_t) * (size_t)nkeys : 0;
        hipLaunchKernelGGL(k_bucket_count, dim3(grid_for(n, 256)), dim3(256), lds_keys, s,
                           (int32_t)n, G->row_ptr, G->work, d_win, (int32_t)W, (int32_t)nkeys,
                           key_count);
        STEP2_HIP(hipGetLastError());
        STEP2(exclusive_scan_i32_to_i32(key_count, key_start, nkeys, key_scan_ws, s));
        std::vector<int32_t> h_start(nkeys + 1);
        STEP2_HIP(hipMemcpyAsync(h_start.data(), key_start, sizeof(int32_t) * (nkeys + 1),
                                 hipMemcpyDeviceToHost, s));
        hipLaunchKernelGGL(k_bucket_scatter, dim3(grid_for(n, 256)), dim3(256), 2 * lds_keys, s,
                           (int32_t)n, G->row_ptr, G->work, d_win, (int32_t)W, (int32_t)nkeys,
                           key_start, G->hubs);
        STEP2_HIP(hipGetLastError());
        STEP2_HIP(hipStreamSynchronize(s));
        for (int64_t k = 0; k < W; ++k) G->win_hubs[k] = h_start[k * kHubClasses];
        if (h_start[nkeys] != G->n_hubs) {
            set_error("hub list: %d hubs bucketed, %lld expected", h_start[nkeys],
                      (long long)G->n_hubs);
            cleanup2();
            cleanup();
            return GTC_E_HIP;
        }
    }
    // The downloads into the pinned CSR may still run: readers wait for `downloaded`.  The last
    // windows stay in the staging buffers for the first tiles of a count.
    if (cs) {
        STEP2_HIP(hipEventCreateWithFlags(&G->downloaded, hipEventDisableTiming));
        STEP2_HIP(hipEventRecord(G->downloaded, cs));
        cs = nullptr;
    }
    if (G->windowed()) {
        STEP2_HIP(hipEventCreateWithFlags(&G->staged, hipEventDisableTiming));
        STEP2_HIP(hipEventRecord(G->staged, s));
        for (int b = 0; b < 3; ++b) G->slot_win[b] = st_win[b];
    }
    cleanup2();
#undef STEP2
#undef STEP2_HIP
    cleanup();
#undef STEP
#undef STEP_HIP
    return GTC_OK;
}

// Keep the listed hubs that can close a triangle (hub_class >= 0), and sum their forward degrees
// (merge-walks) and spoke elements.
__global__ void __launch_bounds__(256)
    k_filter_hubs(const int32_t *__restrict__ in, int64_t n_in, const int64_t *__restrict__ row_ptr,
                  const int64_t *__restrict__ work, int32_t *__restrict__ out,
                  unsigned long long *__restrict__ sums /* [3]: kept, walks, spoke elements */) {
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (t >= n_in) return;
    const int32_t i = in[t];
    const int64_t m = row_ptr[i + 1] - row_ptr[i];
    if (hub_class(m, work[i]) < 0) return;
    out[atomicAdd(&sums[0], 1ull)] = i;
    atomicAdd(&sums[1], (unsigned long long)m);
    atomicAdd(&sums[2], (unsigned long long)work[i]);
}

int filter_hubs(const gtc_graph_s *G, const int32_t *in, int64_t n_in, int32_t *out,
                unsigned long long *d_sums, HubSubset *res, hipStream_t s) {
    GTC_TRY(fill_u64(reinterpret_cast<uint64_t *>(d_sums), 3, 0ull, s));
    if (n_in > 0) {
        hipLaunchKernelGGL(k_filter_hubs, dim3(grid_for(n_in, 256)), dim3(256), 0, s, in, n_in,
                           G->row_ptr, G->work, out, d_sums);
        GTC_HIP_CHECK(hipGetLastError());
    }
    unsigned long long h[3];
    GTC_HIP_CHECK(hipMemcpyAsync(h, d_sums, sizeof(h), hipMemcpyDeviceToHost, s));
    GTC_HIP_CHECK(hipStreamSynchronize(s));
    res->hubs = out;
    res->n_hubs = (int64_t)h[0];
    res->walks = (int64_t)h[1];
    res->spoke_elements = (int64_t)h[2];
    return GTC_OK;
}

int emit_window(const gtc_graph_s *G, int64_t w, int32_t *col, uint8_t *bin, hipStream_t s) {
    const int64_t lo = G->win[w], hi = G->win[w + 1];
    if (hi <= lo) return GTC_OK;
    PairArgs pa{};
    pa.xyz_s = G->xyz_s;
    pa.cell_start = G->cell_start;
    pa.edges = G->d_edges;
    pa.nb = G->nb;
    pa.n = (int32_t)G->n;
    pa.gr = G->grid;
    pa.h_lo = (int32_t)lo;
    pa.h_hi = (int32_t)hi;
    pa.row_ptr = G->row_ptr;
    pa.col_base = G->win_e[w];
    pa.col = col;
    pa.bin = G->packed ? nullptr : bin;
    pa.slot_off = nullptr;
    hipLaunchKernelGGL(k_pairs<true>, dim3(grid_for(hi - lo, 256)), dim3(256), 0, s, pa);
    GTC_HIP_CHECK(hipGetLastError());
    return GTC_OK;
}

// Weights into internal order: w_s[pos] = w[perm[pos]], and max |w| (bit pattern of a
// non-negative double orders like its value) plus a flag for non-finite values.
// w_s[i] = w[perm[i]]; max |w| and a non-finite flag reduced per workgroup, then one atomic per
// workgroup (atomics on one address serialise: one per wave cost ~0.2 ms per million points)
constexpr int kGatherThreads = 256;
__global__ void __launch_bounds__(kGatherThreads)
k_gather_weights(int64_t n, const double *__restrict__ w, const int32_t *__restrict__ perm,
                 double *__restrict__ w_s, unsigned long long *__restrict__ maxabs_bits,
                 int32_t *__restrict__ bad) {
    __shared__ unsigned long long wmax[kGatherThreads / kWave];
    __shared__ int32_t wbad[kGatherThreads / kWave];
    unsigned long long m = 0;
    int32_t nf = 0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const double v = w[perm[i]];
        w_s[i] = v;
        nf |= !isfinite(v);
        const unsigned long long b = (unsigned long long)__double_as_longlong(fabs(v));
        m = b > m ? b : m;
    }
    for (int d = kWave / 2; d > 0; d >>= 1) {
        const unsigned long long o = __shfl_xor(m, d, kWave);
        m = o > m ? o : m;
        nf |= __shfl_xor(nf, d, kWave);
    }
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    if (lane == 0) {
        wmax[wid] = m;
        wbad[wid] = nf;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int t = 1; t < kGatherThreads / kWave; ++t) {
            m = wmax[t] > m ? wmax[t] : m;
            nf |= wbad[t];
        }
        if (m) atomicMax(maxabs_bits, m);
        if (nf) atomicOr(bad, 1);
    }
}

int gather_weights(const gtc_graph_s *G, const double *d_w, double *w_s, unsigned long long *d_m,
                   int32_t *d_bad, double *maxabs, hipStream_t s) {
    int rc = fill_u64(reinterpret_cast<uint64_t *>(d_m), 1, 0ull, s);
    if (!rc) rc = fill_u32(reinterpret_cast<uint32_t *>(d_bad), 1, 0u, s);
    unsigned long long hm = 0;
    int32_t hb = 0;
    if (!rc && G->n > 0) {
        const unsigned blocks = (unsigned)std::min<int64_t>((G->n + kGatherThreads - 1) / kGatherThreads, 2048);
        hipLaunchKernelGGL(k_gather_weights, dim3(blocks), dim3(kGatherThreads), 0, s, G->n, d_w,
                           G->perm, w_s, d_m, d_bad);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) rc = hip_fail(e, "k_gather_weights", __FILE__, __LINE__);
    }
    if (!rc) {
        hipError_t e = hipMemcpyAsync(&hm, d_m, sizeof(hm), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipMemcpyAsync(&hb, d_bad, sizeof(hb), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) rc = hip_fail(e, "weight readback", __FILE__, __LINE__);
    }
    if (rc) return rc;
    if (hb) {
        set_error("a weight is not finite");
        return GTC_E_INVALID;
    }
    double v;
    std::memcpy(&v, &hm, sizeof(v));
    *maxabs = v;
    return GTC_OK;
}

}  // namespace gtc

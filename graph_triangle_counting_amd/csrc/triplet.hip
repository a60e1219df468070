// triplet.hip - binned triangle enumeration, the 3pCF numerator (GRAMSCI v2 §II.2, §III.1).
//
// One wavefront per hub i, hubs popped heaviest-first from a global queue (persistent
// workgroups).  The pages' merge-walk intersects the hub tail {k in N(i): k > j} with N(j) for
// every spoke j by two pointers over both sorted lists.  Here the hub side of that walk is held in
// LDS as a direct-address map over the hub's stencil domain (the label ranges of its forward
// cells, see hub_domain): map[k] = bin(i,k) + 1 for k in N+(i), 0 otherwise.  The spoke row
// N+(j) is then streamed once, in order, by a group of G lanes; each element is one O(1) LDS
// probe, and the walk stops at the first element past the hub's last neighbour, as the two-pointer
// walk does when the hub list is exhausted.  Every element of N+(j) exceeds j, so a hit is exactly
// a triangle i < j < k, counted once.
//
// A hit ranks its sorted side-length bins (Fig. 8 key order) and adds 1 to a workgroup LDS
// histogram (32-bit, exchanged out before it could overflow); the histogram is flushed with 64-bit
// global atomics.  Weighted counts add the exact fixed-point value of fl(fl(w1*w2)*w3) as two
// limbs (28 low bits, 30 offset high bits) to 64-bit LDS counters, flushed into 128-bit global
// accumulators, so the sum is exact and independent of order (the pages accumulate fp atomics,
// §III.5.2, and see order-dependent last digits, §IV.8).
#include <algorithm>
#include <climits>
#include <cmath>
#include <vector>

#include "gtc_internal.h"

namespace gtc {

struct TripletArgs {
    const int64_t *row_ptr;  // global row offsets [n+1]
    // hub window: rows of hubs, entry e at col_h[e - base_h]
    const int32_t *col_h;
    const uint8_t *bin_h;
    int64_t base_h;
    // search window: rows of spokes, entry e at col_s[e - base_s]; spokes j in [s_lo, s_hi)
    const int32_t *col_s;
    const uint8_t *bin_s;
    int64_t base_s;
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
    Grid gr;
    const double *w_s;  // weights, internal order (weighted only)
    double two_s;       // 2^s
    unsigned int *queue;
    unsigned long long *counts;  // [ncfg]
    unsigned long long *limbs;   // [ncfg][4]: 128-bit sum of low limbs, 128-bit sum of high limbs
    unsigned int flush_at;       // hits a wave may add between exchanges of the LDS histogram
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

// LDS layout: counts u32[ncfg] | (weighted) lo u64[ncfg], hi u64[ncfg] | A i32[256], B i32[256]
//             | nw maps of map_bytes
// (with a global histogram, GH, only the rank tables and the maps are in LDS)
__host__ __device__ inline size_t triplet_lds_fixed(int ncfg, bool weighted, bool gh) {
    size_t b = 0;
    if (!gh) {
        b += align_up(sizeof(uint32_t) * ncfg, 16);
        if (weighted) b += 2 * align_up(sizeof(unsigned long long) * ncfg, 16);
    }
    return b + 2 * 256 * sizeof(int32_t);
}

// Exchange the workgroup histogram out to global memory.  Safe while other waves keep adding:
// each bin is swapped for zero atomically, so every increment is flushed exactly once.
template <bool W>
__device__ void flush_hist(const TripletArgs &a, uint32_t *hc, unsigned long long *hlo,
                           unsigned long long *hhi, int first, int step) {
    for (int t = first; t < a.ncfg; t += step) {
        const uint32_t v = atomicExch(&hc[t], 0u);
        if (v) atomicAdd(&a.counts[t], (unsigned long long)v);
        if (W) {
            const unsigned long long l = atomicExch(&hlo[t], 0ull);
            if (l) add_u128(&a.limbs[4 * t], l);
            const unsigned long long h = atomicExch(&hhi[t], 0ull);
            if (h) add_u128(&a.limbs[4 * t + 2], h);
        }
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

// Per-wave LDS region: hub map | chunk of 64 spokes | (weighted) the hub row's bins and weights.
//   map    : u8 bin+1 per domain label, or (weighted) u16 row position+1
//   chunk  : cpre u32[65] flat start of each spoke's row, cbase i64[64] (row start - flat start),
//            cbij u8[64] spoke bins, (weighted) cw f64[64] spoke weights
constexpr int kChunkPre = 0, kChunkBase = 272, kChunkBij = 784, kChunkW = 848;
__host__ __device__ inline size_t chunk_bytes(bool weighted) { return weighted ? 1360 : 848; }
__host__ __device__ inline size_t hubrow_bytes(bool weighted, int max_m) {
    return weighted ? align_up(8 * (size_t)max_m, 16) + align_up((size_t)max_m, 16) : 0;
}

constexpr int kUnroll = 4;  // loads in flight per lane

// GH: bins go straight to the global histogram (configuration counts too large for LDS).
template <bool W, bool GH>
__global__ void __launch_bounds__(256) k_triplet(TripletArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    size_t off = 0;
    uint32_t *hc = reinterpret_cast<uint32_t *>(smem);
    if (!GH) off += align_up(sizeof(uint32_t) * a.ncfg, 16);
    unsigned long long *hlo = nullptr, *hhi = nullptr;
    if (W && !GH) {
        hlo = reinterpret_cast<unsigned long long *>(smem + off);
        off += align_up(sizeof(unsigned long long) * a.ncfg, 16);
        hhi = reinterpret_cast<unsigned long long *>(smem + off);
        off += align_up(sizeof(unsigned long long) * a.ncfg, 16);
    }
    int32_t *rA = reinterpret_cast<int32_t *>(smem + off);
    int32_t *rB = rA + 256;
    off += 2 * 256 * sizeof(int32_t);
    unsigned char *wb = smem + off + (size_t)wid * a.wave_bytes;
    uint8_t *map8 = wb;
    uint16_t *map16 = reinterpret_cast<uint16_t *>(wb);
    unsigned char *ck = wb + a.map_bytes;
    uint32_t *cpre = reinterpret_cast<uint32_t *>(ck + kChunkPre);
    int64_t *cbase = reinterpret_cast<int64_t *>(ck + kChunkBase);
    uint8_t *cbij = ck + kChunkBij;
    double *cw = reinterpret_cast<double *>(ck + kChunkW);
    double *rw = reinterpret_cast<double *>(ck + chunk_bytes(true));
    uint8_t *rbn = ck + chunk_bytes(true) + align_up(8 * (size_t)a.max_m, 16);

    if (!GH)
        for (int t = threadIdx.x; t < a.ncfg; t += blockDim.x) {
            hc[t] = 0;
            if (W) hlo[t] = hhi[t] = 0;
        }
    if (threadIdx.x == 0) rank3_tables(a.nb, rA, rB);
    __syncthreads();

    unsigned int wave_hits = 0;
    for (;;) {
        unsigned int hq = 0;
        if (lane == 0) hq = atomicAdd(a.queue, 1u);
        hq = __builtin_amdgcn_readfirstlane(__shfl(hq, 0, kWave));
        if (hq >= (unsigned int)a.n_hubs) break;
        const int32_t i = __builtin_amdgcn_readfirstlane(a.hubs[hq]);
        const int64_t rb = a.row_ptr[i], re = a.row_ptr[i + 1];
        const int32_t m = (int32_t)(re - rb);
        HubDomain dom;
        hub_domain(i, a.key_s[i], a.gr, a.cell_start, dom);

        // hub side of the walk: clear the map over the domain, then mark N+(i)
        uint32_t *map32 = reinterpret_cast<uint32_t *>(wb);
        const int map_words = ((W ? 2 : 1) * dom.size + 3) >> 2;
        for (int t = lane; t < map_words; t += kWave) map32[t] = 0u;
        wave_lds_sync();
        const int32_t *hrow = a.col_h + (rb - a.base_h);
        const uint8_t *hbin = a.bin_h + (rb - a.base_h);
        for (int p = lane; p < m; p += kWave) {
            const int32_t k = hrow[p];
            int32_t d = dom.delta[0];
#pragma unroll
            for (int t = 1; t < 5; ++t)
                if (k >= dom.lo[t]) d = dom.delta[t];
            if (W) {
                map16[k + d] = (uint16_t)(p + 1);
                rw[p] = a.w_s[k];
                rbn[p] = hbin[p];
            } else {
                map8[k + d] = (uint8_t)(hbin[p] + 1);
            }
        }
        wave_lds_sync();
        const int32_t hub_hi = hrow[m - 1];
        const double wi = W ? a.w_s[i] : 0.0;

        // spokes of this tile: hub-row positions [p_lo, p_hi) with j in [s_lo, s_hi)
        int32_t p_lo = 0, p_hi = m;
        if (a.s_lo > hrow[0] || a.s_hi <= hub_hi) {
            int32_t l = 0, h = m;
            while (l < h) { const int32_t md = (l + h) >> 1; if (hrow[md] < a.s_lo) l = md + 1; else h = md; }
            p_lo = l;
            h = m;
            while (l < h) { const int32_t md = (l + h) >> 1; if (hrow[md] < a.s_hi) l = md + 1; else h = md; }
            p_hi = l;
        }

        unsigned int my_hits = 0;
        // spokes in chunks of 64: lane q fetches spoke q's row bounds, a wave scan lays the 64
        // spoke rows end to end, and the lanes walk that flat range with kUnroll loads in flight.
        for (int32_t p0 = p_lo; p0 < p_hi; p0 += kWave) {
            const int32_t p = p0 + lane;
            int64_t sb = 0;
            int32_t len = 0, bj = 0;
            double wj = 0.0;
            if (p < p_hi) {
                const int32_t j = hrow[p];
                bj = hbin[p];
                sb = a.row_ptr[j];
                len = (int32_t)(a.row_ptr[j + 1] - sb);
                if (W) wj = a.w_s[j];
            }
            const int32_t incl = wave_incl_scan(len, lane);
            const int32_t total = __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1, kWave));
            cpre[lane] = (uint32_t)(incl - len);
            if (lane == kWave - 1) cpre[kWave] = (uint32_t)incl;
            cbase[lane] = sb - (incl - len);
            cbij[lane] = (uint8_t)bj;
            if (W) cw[lane] = wj;
            wave_lds_sync();
            // owner spoke of flat index t: the last q with cpre[q] <= t (then t < cpre[q+1])
            int q = 0;
            {
                int hi = kWave;
                while (hi - q > 1) {
                    const int md = (q + hi) >> 1;
                    if ((int32_t)cpre[md] <= lane) q = md; else hi = md;
                }
            }
            for (int32_t t0 = 0; t0 < total; t0 += kWave * kUnroll) {
                int32_t kk[kUnroll], bb[kUnroll], qq[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int32_t t = t0 + u * kWave + lane;
                    kk[u] = INT32_MAX;
                    bb[u] = 0;
                    qq[u] = q;
                    if (t < total) {
                        while ((int32_t)cpre[q + 1] <= t) ++q;
                        qq[u] = q;
                        const int64_t e = cbase[q] + t - a.base_s;
                        kk[u] = a.col_s[e];
                        bb[u] = a.bin_s[e];
                    }
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int32_t k = kk[u];
                    if (k > hub_hi) continue;  // past the hub's last neighbour (or no element)
                    int32_t d = dom.delta[0], lim = dom.hi[0];
#pragma unroll
                    for (int t = 1; t < 5; ++t)
                        if (k >= dom.lo[t]) { d = dom.delta[t]; lim = dom.hi[t]; }
                    if (k >= lim) continue;  // in a gap between the hub's stencil runs
                    const uint32_t v = W ? (uint32_t)map16[k + d] : (uint32_t)map8[k + d];
                    if (!v) continue;
                    const int32_t bij = cbij[qq[u]];
                    const int32_t bik = W ? (int32_t)rbn[v - 1] : (int32_t)v - 1;
                    const int32_t bjk = bb[u];
                    const int32_t x = min(bij, min(bik, bjk)), z = max(bij, max(bik, bjk));
                    const int32_t y = bij + bik + bjk - x - z;
                    const int32_t c = rA[x] + rB[y] + z;
                    if (GH) atomicAdd(&a.counts[c], 1ull);
                    else atomicAdd(&hc[c], 1u);
                    if (W) {
                        const double wjj = cw[qq[u]], wk = rw[v - 1];
                        const double x1 = fmin(wi, wjj), x2 = fmax(wi, wjj);
                        const double w1 = fmin(x1, wk), tt = fmax(x1, wk);
                        const double w2 = fmin(x2, tt), w3 = fmax(x2, tt);
                        const double pr = __dmul_rn(__dmul_rn(w1, w2), w3);
                        const double qv = rint(__dmul_rn(pr, a.two_s));     // exact integer
                        const double qh = floor(__dmul_rn(qv, 0x1p-28));   // in [-2^29, 2^29)
                        const double ql = __fma_rn(-qh, 0x1p28, qv);       // in [0, 2^28)
                        const unsigned long long ul = (unsigned long long)ql;
                        const unsigned long long uh = (unsigned long long)((long long)qh + (1ll << 29));
                        if (GH) {
                            add_u128(&a.limbs[4 * c], ul);
                            add_u128(&a.limbs[4 * c + 2], uh);
                        } else {
                            atomicAdd(&hlo[c], ul);
                            atomicAdd(&hhi[c], uh);
                        }
                    }
                    ++my_hits;
                }
            }
            wave_lds_sync();  // the next chunk overwrites the chunk arrays
        }
        if (!GH) {
            wave_hits += wave_sum(my_hits);
            if (wave_hits >= a.flush_at) {
                flush_hist<W>(a, hc, hlo, hhi, lane, kWave);
                wave_hits = 0;
            }
        }
        wave_lds_sync();  // this wave's map reads complete before the next hub clears it
    }
    if (!GH) {
        __syncthreads();
        flush_hist<W>(a, hc, hlo, hhi, threadIdx.x, blockDim.x);
    }
}

// ------------------------------------------------------------------ host side

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
};

template <bool W, bool GH>
static int plan_triplet(const TripletArgs &a, int64_t n_hubs, TripletPlan &pl) {
    DeviceLimits dl;
    GTC_TRY(device_limits(dl));
    const size_t fixed = triplet_lds_fixed(a.ncfg, W, GH);
    int waves = 4;
    while (waves > 1 && fixed + (size_t)waves * a.wave_bytes > dl.lds_per_block) waves >>= 1;
    const size_t lds = fixed + (size_t)waves * a.wave_bytes;
    if (lds > dl.lds_per_block) {
        set_error("3pCF needs %zu bytes of LDS per workgroup (histogram %d configs, %d bytes per "
                  "wave); the device allows %zu",
                  lds, a.ncfg, a.wave_bytes, dl.lds_per_block);
        return GTC_E_UNSUPPORTED;
    }
    if (lds > 65536)
        GTC_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void *>(&k_triplet<W, GH>),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    int per_cu = 0;
    GTC_HIP_CHECK(hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void *>(&k_triplet<W, GH>), waves * kWave, lds));
    if (per_cu < 1) per_cu = 1;
    int64_t blocks = (int64_t)dl.cus * per_cu;
    const int64_t need = (n_hubs + waves - 1) / waves;
    if (blocks > need) blocks = need;
    if (blocks < 1) blocks = 1;
    pl.waves = waves;
    pl.lds = lds;
    pl.blocks = (int)blocks;
    return GTC_OK;
}

template <bool W, bool GH>
static int launch_triplet(const TripletArgs &a, const TripletPlan &pl, hipStream_t s) {
    hipLaunchKernelGGL((k_triplet<W, GH>), dim3(pl.blocks), dim3(pl.waves * kWave), pl.lds, s, a);
    GTC_HIP_CHECK(hipGetLastError());
    return GTC_OK;
}

int gather_weights(const gtc_graph_s *G, const double *d_w, double *w_s, double *maxabs,
                   hipStream_t s);

// Scale exponent of the exact weighted sums: s = 57 - e, with M = fl(fl(a*a)*a) = f 2^e,
// f in [0.5, 1), for a = max |w|; then |p * 2^s| < 2^57 for every triangle product p.
static int weight_scale_for(double maxabs) {
    volatile double a2 = maxabs * maxabs;
    volatile double m = a2 * maxabs;
    if (m == 0.0) return 0;
    int e = 0;
    std::frexp((double)m, &e);
    return 57 - e;
}

static double limbs_to_double(const unsigned long long *l, unsigned long long count, int s) {
    const unsigned __int128 lo = ((unsigned __int128)l[1] << 64) | l[0];
    const unsigned __int128 hi = ((unsigned __int128)l[3] << 64) | l[2];
    const unsigned __int128 u = (hi << 28) + lo - ((unsigned __int128)count << 57);
    const __int128 v = (__int128)u;  // exact sum of q, two's complement
    return std::ldexp((double)v, -s);
}

int count_3pcf_device(gtc_graph_s *G, const double *d_w, uint64_t *d_counts, double *d_weighted,
                      gtc_stats *st, hipStream_t s) {
    const bool W = d_w != nullptr;
    const int nb = G->nb;
    const int64_t ncfg = gtc_num_configs(3, nb);
    GTC_TRY(fill_u64(d_counts, ncfg, 0ull, s));

    double *w_s = nullptr;
    unsigned long long *limbs = nullptr;
    unsigned int *queue = nullptr;
    int rc = GTC_OK;
    int scale = 0;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    auto cleanup = [&]() {
        dev_free(w_s, s);
        dev_free(limbs, s);
        dev_free(queue, s);
        if (ev0) (void)hipEventDestroy(ev0);
        if (ev1) (void)hipEventDestroy(ev1);
    };
#define STEP(expr) do { rc = (expr); if (rc) { cleanup(); return rc; } } while (0)
#define STEP_HIP(call) do { hipError_t e_ = (call); if (e_ != hipSuccess) { rc = hip_fail(e_, #call, __FILE__, __LINE__); cleanup(); return rc; } } while (0)

    if (W) {
        double maxabs = 0.0;
        STEP(dev_alloc_n(&w_s, G->n, s));
        STEP(gather_weights(G, d_w, w_s, &maxabs, s));
        scale = weight_scale_for(maxabs);
        STEP(dev_alloc_n(&limbs, 4 * ncfg, s));
        STEP(fill_u64(reinterpret_cast<uint64_t *>(limbs), 4 * ncfg, 0ull, s));
    }
    STEP(dev_alloc_n(&queue, 1, s));
    STEP(fill_u32(queue, 1, 0u, s));
    STEP_HIP(hipEventCreate(&ev0));
    STEP_HIP(hipEventCreate(&ev1));

    TripletArgs a{};
    a.row_ptr = G->row_ptr;
    a.col_h = G->col;
    a.bin_h = G->bin;
    a.base_h = 0;
    a.col_s = G->col;
    a.bin_s = G->bin;
    a.base_s = 0;
    a.s_lo = 0;
    a.s_hi = (int32_t)G->n;
    a.hubs = G->hubs;
    a.n_hubs = (int32_t)G->n_hubs;
    a.nb = nb;
    a.ncfg = (int32_t)ncfg;
    a.max_m = (int32_t)std::max<int64_t>(G->max_deg, 1);
    a.map_bytes = (int32_t)align_up((W ? 2 : 1) * (size_t)std::max<int64_t>(G->max_domain, 1), 16);
    a.wave_bytes = (int32_t)(a.map_bytes + chunk_bytes(W) + hubrow_bytes(W, a.max_m));
    if (W && G->max_deg >= 65535) {
        set_error("weighted 3pCF: a forward row of %lld entries exceeds the 16-bit position map",
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
    a.counts = reinterpret_cast<unsigned long long *>(d_counts);
    a.limbs = limbs;

    float kms = 0.f;
    if (G->n_hubs > 0) {
        // LDS histogram unless it would take more than half of a workgroup's LDS
        DeviceLimits dl;
        STEP(device_limits(dl));
        const bool GH = triplet_lds_fixed(a.ncfg, W, false) > dl.lds_per_block / 2;
        TripletPlan pl;
        STEP(W ? (GH ? plan_triplet<true, true>(a, G->n_hubs, pl) : plan_triplet<true, false>(a, G->n_hubs, pl))
               : (GH ? plan_triplet<false, true>(a, G->n_hubs, pl) : plan_triplet<false, false>(a, G->n_hubs, pl)));
        // 32-bit LDS bins: all waves of a workgroup together stay below 2^32 between exchanges
        const unsigned long long max_hub_hits =
            (unsigned long long)G->max_deg * (unsigned long long)(G->max_deg - 1) / 2;
        const unsigned long long budget = 0xffffffffull / (unsigned long long)pl.waves;
        if (!GH && max_hub_hits >= budget / 2) {
            set_error("a hub has %lld forward neighbours; its triangles could overflow the 32-bit "
                      "LDS histogram", (long long)G->max_deg);
            cleanup();
            return GTC_E_UNSUPPORTED;
        }
        a.flush_at = GH ? 0u : (unsigned int)(budget - max_hub_hits);
        STEP_HIP(hipEventRecord(ev0, s));
        STEP(W ? (GH ? launch_triplet<true, true>(a, pl, s) : launch_triplet<true, false>(a, pl, s))
               : (GH ? launch_triplet<false, true>(a, pl, s) : launch_triplet<false, false>(a, pl, s)));
        STEP_HIP(hipEventRecord(ev1, s));
    }
    std::vector<unsigned long long> h_counts(ncfg), h_limbs(W ? 4 * ncfg : 0);
    STEP_HIP(hipMemcpyAsync(h_counts.data(), d_counts, sizeof(uint64_t) * ncfg,
                            hipMemcpyDeviceToHost, s));
    if (W)
        STEP_HIP(hipMemcpyAsync(h_limbs.data(), limbs, sizeof(unsigned long long) * 4 * ncfg,
                                hipMemcpyDeviceToHost, s));
    STEP_HIP(hipStreamSynchronize(s));
    if (G->n_hubs > 0) STEP_HIP(hipEventElapsedTime(&kms, ev0, ev1));
    if (W) {
        std::vector<double> h_w(ncfg);
        for (int64_t c = 0; c < ncfg; ++c) h_w[c] = limbs_to_double(&h_limbs[4 * c], h_counts[c], scale);
        STEP_HIP(hipMemcpyAsync(d_weighted, h_w.data(), sizeof(double) * ncfg,
                                hipMemcpyHostToDevice, s));
        STEP_HIP(hipStreamSynchronize(s));
    }
    unsigned long long tri = 0;
    for (auto v : h_counts) tri += v;
    if (st) {
        st->triangles = tri;
        st->merge_walks = G->walks;
        st->spoke_elements = G->spoke_elements;
        st->tiles = G->n_hubs > 0 ? 1 : 0;
        st->kernel_ms = kms;
        st->weight_scale = scale;
        st->q_alg_bytes = 5.0 * (double)G->E + 4.0 * (double)G->spoke_elements + (double)tri;
    }
    cleanup();
#undef STEP
#undef STEP_HIP
    return GTC_OK;
}

}  // namespace gtc

// twopoint.hip - the 2pCF pair histogram over the graph's edges (GRAMSCI v2 §II.1, §III.3).
//
// Each forward edge (i, j), j > i, is one pair, counted once in its bin.  With weights, the pair
// adds p = fl(w_i * w_j) as the exact integer q = rint(p * 2^s), s = 57 - e for M = fl(a * a) =
// f * 2^e and a = max |w|, so |q| < 2^57; q goes into two limbs (28 low bits, 30 offset high
// bits) summed in 64-bit counters, and the host rounds each bin's exact sum once.  With data
// weights summing to +1 and random weights to -1 the sums are the Landy-Szalay numerator
// DD - 2DR + RR of the signed-weight estimator.
//
// One wave per row (rows taken in blocks from a grid-stride loop); the lanes stream the row's
// entries and add to per-wave LDS bins, so waves never contend; the workgroup adds its bins to the
// global totals at the end with 64-bit atomics (limbs into 128-bit accumulators with carry).
#include <cmath>
#include <vector>

#include "gtc_internal.h"

namespace gtc {

int gather_weights(const gtc_graph_s *G, const double *d_w, double *w_s, unsigned long long *d_m,
                   int32_t *d_bad, double *maxabs, hipStream_t s);

namespace {

constexpr int kPairWaves = 4;  // waves per workgroup

struct PairHistArgs {
    const int64_t *row_ptr;
    const int32_t *col;    // entry e at col[e - base]
    const uint8_t *bin;    // null: packed entries
    int64_t base;
    int32_t row_lo, row_hi;  // rows of this launch
    int32_t nb;
    const double *w_s;       // weights in internal order (weighted only)
    double two_s;
    unsigned long long *counts;  // [nb]
    unsigned long long *limbs;   // [nb][4]: 128-bit sums of the low and of the high limbs
};

__device__ __forceinline__ void add_u128_pair(unsigned long long *p, unsigned long long v) {
    const unsigned long long old = atomicAdd(p, v);
    if (old + v < old) atomicAdd(p + 1, 1ull);
}

template <bool W, bool PK>
__global__ void __launch_bounds__(kPairWaves * kWave) k_pair_hist(PairHistArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int per_wave = (W ? 3 : 1) * a.nb;  // u64 words: counts | low limbs | high limbs
    unsigned long long *h = reinterpret_cast<unsigned long long *>(smem) + (size_t)wid * per_wave;
    for (int t = lane; t < per_wave; t += kWave) h[t] = 0ull;
    __builtin_amdgcn_wave_barrier();

    const int64_t nrows = (int64_t)a.row_hi - a.row_lo;
    const int64_t stride = (int64_t)gridDim.x * kPairWaves;
    for (int64_t r = (int64_t)blockIdx.x * kPairWaves + wid; r < nrows; r += stride) {
        const int32_t i = a.row_lo + (int32_t)r;
        const int64_t rb = a.row_ptr[i] - a.base, re = a.row_ptr[i + 1] - a.base;
        const double wi = W ? a.w_s[i] : 0.0;
        for (int64_t e = rb + lane; e < re; e += kWave) {
            int32_t j, b;
            csr_entry<PK>(a.col, a.bin, e, j, b);
            atomicAdd(&h[b], 1ull);
            if (W) {
                const double p = __dmul_rn(wi, a.w_s[j]);
                const double qv = rint(__dmul_rn(p, a.two_s));     // exact integer, |qv| < 2^57
                const double qh = floor(__dmul_rn(qv, 0x1p-28));   // in [-2^29, 2^29)
                const double ql = __fma_rn(-qh, 0x1p28, qv);       // in [0, 2^28)
                atomicAdd(&h[a.nb + b], (unsigned long long)(uint32_t)ql);
                atomicAdd(&h[2 * a.nb + b],
                          (unsigned long long)(uint32_t)((int32_t)qh + (1 << 29)));
            }
        }
    }
    __syncthreads();
    // the workgroup's waves together, then one global add per bin
    for (int t = threadIdx.x; t < per_wave; t += blockDim.x) {
        unsigned long long v = 0;
        for (int w2 = 0; w2 < kPairWaves; ++w2)
            v += reinterpret_cast<unsigned long long *>(smem)[(size_t)w2 * per_wave + t];
        if (!v) continue;
        if (t < a.nb) atomicAdd(&a.counts[t], v);
        else if (t < 2 * a.nb) add_u128_pair(&a.limbs[4 * (t - a.nb)], v);
        else add_u128_pair(&a.limbs[4 * (t - 2 * a.nb) + 2], v);
    }
}

const void *pair_kernel(bool w, bool pk) {
    if (w) return pk ? reinterpret_cast<const void *>(&k_pair_hist<true, true>)
                     : reinterpret_cast<const void *>(&k_pair_hist<true, false>);
    return pk ? reinterpret_cast<const void *>(&k_pair_hist<false, true>)
              : reinterpret_cast<const void *>(&k_pair_hist<false, false>);
}

}  // namespace

int count_2pcf_device(gtc_graph_s *G, const double *d_w, uint64_t *d_counts, double *d_weighted,
                      gtc_stats *st, hipStream_t s) {
    const bool W = d_w != nullptr;
    const int nb = G->nb;
    GTC_TRY(fill_u64(d_counts, nb, 0ull, s));
    double *w_s = nullptr;
    unsigned long long *limbs = nullptr, *d_maxabs = nullptr;
    int32_t *d_bad = nullptr, *wcol = nullptr;
    uint8_t *wbin = nullptr;
    void *scratch = nullptr;
    GTC_TRY(carve_alloc(&scratch, s, [&](Carver &c) {
        if (W) {
            c.take(&w_s, G->n);
            c.take(&limbs, 4 * (size_t)nb);
            c.take(&d_maxabs, 1);
            c.take(&d_bad, 1);
        }
        if (G->windowed()) {  // one window's rows at a time
            c.take(&wcol, G->max_window_edges);
            if (!G->packed) c.take(&wbin, G->max_window_edges);
        }
    }));
    int rc = GTC_OK;
    int scale = 0;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    auto finish = [&](int code) {
        if (e0) (void)hipEventDestroy(e0);
        if (e1) (void)hipEventDestroy(e1);
        (void)hipStreamSynchronize(s);
        dev_free(scratch, s);
        return code;
    };
    if (W) {
        double maxabs = 0.0;
        rc = gather_weights(G, d_w, w_s, d_maxabs, d_bad, &maxabs, s);
        if (rc) return finish(rc);
        rc = weight_scale(maxabs, 2, &scale);
        if (rc) return finish(rc);
        rc = fill_u64(reinterpret_cast<uint64_t *>(limbs), 4 * (int64_t)nb, 0ull, s);
        if (rc) return finish(rc);
    }
    PairHistArgs a{};
    a.row_ptr = G->row_ptr;
    a.nb = nb;
    a.w_s = w_s;
    a.two_s = std::ldexp(1.0, scale);
    a.counts = reinterpret_cast<unsigned long long *>(d_counts);
    a.limbs = limbs;
    const void *kfn = pair_kernel(W, G->packed);
    const size_t lds = sizeof(unsigned long long) * (W ? 3 : 1) * nb * kPairWaves;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return finish(hip_fail(hipGetLastError(), "device query", __FILE__, __LINE__));
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)
        return finish(hip_fail(hipGetLastError(), "hipEventCreate", __FILE__, __LINE__));
    float kms = 0.f;
    const int64_t nw = (int64_t)G->win.size() - 1;
    rc = wait_host_csr(G, s);  // uploads read the pinned CSR after the build's downloads
    if (rc) return finish(rc);
    for (int64_t w = 0; w < nw; ++w) {  // the whole graph is one window unless it is tiled
        const int64_t lo = G->win[w], hi = G->win[w + 1];
        if (hi <= lo) continue;
        if (G->windowed()) {
            const int64_t e0w = G->win_e[w], ne = G->win_e[w + 1] - e0w;
            if (ne <= 0) continue;
            if (G->rebuild) {
                rc = emit_window(G, w, wcol, wbin, s);
            } else {
                hipError_t e = hipMemcpyAsync(wcol, G->h_col + e0w, sizeof(int32_t) * ne,
                                              hipMemcpyHostToDevice, s);
                if (e == hipSuccess && !G->packed)
                    e = hipMemcpyAsync(wbin, G->h_bin + e0w, ne, hipMemcpyHostToDevice, s);
                if (e != hipSuccess) rc = hip_fail(e, "window upload", __FILE__, __LINE__);
            }
            if (rc) return finish(rc);
            a.col = wcol;
            a.bin = wbin;
            a.base = e0w;
        } else {
            a.col = G->col;
            a.bin = G->bin;
            a.base = 0;
        }
        a.row_lo = (int32_t)lo;
        a.row_hi = (int32_t)hi;
        const int64_t rows = hi - lo;
        int64_t blocks = std::min<int64_t>((rows + kPairWaves - 1) / kPairWaves, (int64_t)cus * 8);
        if (blocks < 1) blocks = 1;
        void *args[] = {&a};
        float t = 0.f;
        if (hipEventRecord(e0, s) != hipSuccess ||
            hipLaunchKernel(kfn, dim3((unsigned)blocks), dim3(kPairWaves * kWave), args, lds, s) !=
                hipSuccess ||
            hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&t, e0, e1) != hipSuccess)
            return finish(hip_fail(hipGetLastError(), "k_pair_hist", __FILE__, __LINE__));
        kms += t;
    }
    if (W) {  // exact sums to doubles on the device, one rounding per bin
        rc = finalize_limbs(limbs, nb, 1, 4 * nb, reinterpret_cast<const unsigned long long *>(d_counts),
                            scale, d_weighted, s);
        if (rc) return finish(rc);
        hipError_t e = hipStreamSynchronize(s);
        if (e != hipSuccess) return finish(hip_fail(e, "2pCF finalize", __FILE__, __LINE__));
    }
    if (st) {
        st->kernel_ms = kms;
        st->weight_scale = scale;
        st->launch_waves = kPairWaves;
        // every entry read once (4 B packed, 5 B split); weighted: a weight gather per pair
        st->q_alg_bytes = (G->packed ? 4.0 : 5.0) * (double)G->E + (W ? 8.0 * (double)G->E : 0.0);
    }
    return finish(GTC_OK);
}

void disconnected_4pcf_s4(int nb, const double *xi, double *disc) {
    const int64_t ncfg = num_configs_s4(nb);
    std::vector<int32_t> bins(6 * (size_t)ncfg);
    config_bins_s4(nb, bins.data());
    for (int64_t c = 0; c < ncfg; ++c) {
        const int32_t *t = &bins[6 * (size_t)c];  // edges 01 02 03 12 13 23
        disc[c] = xi[t[0]] * xi[t[5]] + xi[t[1]] * xi[t[4]] + xi[t[2]] * xi[t[3]];
    }
}

}  // namespace gtc

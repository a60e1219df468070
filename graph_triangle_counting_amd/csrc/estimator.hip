// estimator.hip - the data-minus-random estimators of the 3pCF and 4pCF (GRAMSCI v2 §II.1,
// §III.3, the compute_3pcf / compute_4pcf interface of §II.2).
//
// One graph over the union of a data catalogue D and a random catalogue R.  The numerators take
// the signed, normalised weights of the Szapudi-Szalay estimator: data w / sum_D w, randoms
// -w / sum_R w.  The normalisation takes the random weights alone, w / sum_R w on R and 0 on D;
// only all-random cliques add to it, so it is counted on a graph of R alone, which has the same
// all-random cliques, bins and scale (max |w| over R), hence the same exact sums, at a fraction
// of the cliques.  Then zeta = NNN / RRR (3pCF), zeta_even = NNNN_even / RRRR and zeta_odd =
// NNNN_odd / RRRR (4pCF, S4 configurations), xi = NN / RR (internal 2pCF), and the connected
// 4pCF zeta_even - disc(xi) of Eq. (4) and (5).  The catalogue sums are correctly rounded, so the
// normalised weights are reproducible bit for bit.
#include <cmath>
#include <cstring>
#include <vector>

#include "gtc_internal.h"

namespace gtc {

namespace {

// Correctly rounded sum of doubles: an exact expansion of non-overlapping partials (two-sum
// steps), rounded once at the end with the half-way correction.
double exact_sum(const std::vector<double> &x) {
    std::vector<double> p;
    for (double v : x) {
        size_t k = 0;
        for (double y : p) {
            if (std::fabs(v) < std::fabs(y)) std::swap(v, y);
            const double hi = v + y;
            const double lo = y - (hi - v);
            if (lo != 0.0) p[k++] = lo;
            v = hi;
        }
        p.resize(k);
        p.push_back(v);
    }
    double hi = 0.0;
    if (!p.empty()) {
        size_t n = p.size();
        hi = p[--n];
        double lo = 0.0;
        while (n > 0) {
            const double x2 = hi, y = p[--n];
            hi = x2 + y;
            const double yr = hi - x2;
            lo = y - yr;
            if (lo != 0.0) break;
        }
        // half-way case: round the way the remaining partials point
        if (n > 0 && ((lo < 0 && p[n - 1] < 0) || (lo > 0 && p[n - 1] > 0))) {
            const double y = lo * 2.0;
            const double x2 = hi + y;
            if (y == x2 - hi) hi = x2;
        }
    }
    return hi;
}

struct Catalogue {
    std::vector<double> w_signed;  // host, n_data + n_rand: data then randoms
    std::vector<double> w_rand;    // host, n_rand: w / sum_R w
};

// the estimator weights from the raw weights (NULL: unit weights)
int make_weights(const double *d_w_data, int64_t nd, const double *d_w_rand, int64_t nr,
                 hipStream_t s, Catalogue *cat) {
    std::vector<double> wd(nd, 1.0), wr(nr, 1.0);
    if (d_w_data && nd)
        GTC_HIP_CHECK(hipMemcpyAsync(wd.data(), d_w_data, sizeof(double) * nd,
                                     hipMemcpyDeviceToHost, s));
    if (d_w_rand && nr)
        GTC_HIP_CHECK(hipMemcpyAsync(wr.data(), d_w_rand, sizeof(double) * nr,
                                     hipMemcpyDeviceToHost, s));
    GTC_HIP_CHECK(hipStreamSynchronize(s));
    for (double v : wd)
        if (!std::isfinite(v)) { set_error("a data weight is not finite"); return GTC_E_INVALID; }
    for (double v : wr)
        if (!std::isfinite(v)) { set_error("a random weight is not finite"); return GTC_E_INVALID; }
    const double sd = exact_sum(wd), sr = exact_sum(wr);
    if (nd > 0 && sd == 0.0) { set_error("the data weights sum to zero"); return GTC_E_INVALID; }
    if (sr == 0.0) { set_error("the random weights sum to zero"); return GTC_E_INVALID; }
    cat->w_signed.resize(nd + nr);
    cat->w_rand.resize(nr);
    for (int64_t i = 0; i < nd; ++i) cat->w_signed[i] = wd[i] / sd;
    for (int64_t i = 0; i < nr; ++i) {
        cat->w_rand[i] = wr[i] / sr;
        cat->w_signed[nd + i] = -cat->w_rand[i];
    }
    return GTC_OK;
}

// D then R, concatenated on the device; the signed weights over D then R, the random weights
// over R
struct DeviceUnion {
    void *block = nullptr;
    int32_t *xyz = nullptr;
    double *w_signed = nullptr, *w_rand = nullptr;
};

int make_union(const int32_t *d_xd, int64_t nd, const int32_t *d_xr, int64_t nr,
               const Catalogue &cat, hipStream_t s, DeviceUnion *u) {
    const int64_t n = nd + nr;
    GTC_TRY(carve_alloc(&u->block, s, [&](Carver &c) {
        c.take(&u->xyz, 3 * (size_t)n);
        c.take(&u->w_signed, n);
        c.take(&u->w_rand, nr);
    }));
    if (nd)
        GTC_HIP_CHECK(hipMemcpyAsync(u->xyz, d_xd, sizeof(int32_t) * 3 * nd,
                                     hipMemcpyDeviceToDevice, s));
    if (nr)
        GTC_HIP_CHECK(hipMemcpyAsync(u->xyz + 3 * nd, d_xr, sizeof(int32_t) * 3 * nr,
                                     hipMemcpyDeviceToDevice, s));
    GTC_HIP_CHECK(hipMemcpyAsync(u->w_signed, cat.w_signed.data(), sizeof(double) * n,
                                 hipMemcpyHostToDevice, s));
    GTC_HIP_CHECK(hipMemcpyAsync(u->w_rand, cat.w_rand.data(), sizeof(double) * nr,
                                 hipMemcpyHostToDevice, s));
    return GTC_OK;
}

int check_catalogues(const char *fn, const int32_t *d_xd, int64_t nd, const int32_t *d_xr,
                     int64_t nr) {
    if (nd < 0 || nr <= 0 || (nd > 0 && !d_xd) || !d_xr || nd + nr >= ((int64_t)1 << 31)) {
        set_error("%s: need n_data >= 0 data points, n_rand > 0 random points, n_data + n_rand "
                  "< 2^31, and their coordinates", fn);
        return GTC_E_INVALID;
    }
    return GTC_OK;
}

template <class T>
int to_host(std::vector<T> &h, const T *d, int64_t n, hipStream_t s) {
    h.resize(n);
    GTC_HIP_CHECK(hipMemcpyAsync(h.data(), d, sizeof(T) * n, hipMemcpyDeviceToHost, s));
    GTC_HIP_CHECK(hipStreamSynchronize(s));
    return GTC_OK;
}

}  // namespace
}  // namespace gtc

using namespace gtc;

int gtc_linear_edges_sq(int64_t r_min, int64_t r_max, int32_t nbins, int64_t *h_edges_sq) {
    if (nbins < 1 || nbins > GTC_MAX_BINS || !h_edges_sq || r_min < 0 || r_max <= r_min ||
        r_max > 2 * (int64_t)kGridSide) {
        set_error("gtc_linear_edges_sq: need 0 <= r_min < r_max <= 2^21, nbins in [1, %d]",
                  GTC_MAX_BINS);
        return GTC_E_INVALID;
    }
    // r_b = (r_min nb + b (r_max - r_min)) / nb; e_b = ceil(r_b^2), so d^2 >= e_b <=> d >= r_b
    const int64_t nb = nbins, den = nb * nb;
    for (int64_t b = 0; b <= nb; ++b) {
        const int64_t num = r_min * nb + b * (r_max - r_min);  // < 2^29
        const int64_t sq = num * num;                          // < 2^58
        h_edges_sq[b] = (sq + den - 1) / den;
    }
    for (int b = 0; b < nbins; ++b)
        if (h_edges_sq[b + 1] <= h_edges_sq[b]) {
            set_error("gtc_linear_edges_sq: bins narrower than the integer grid");
            return GTC_E_INVALID;
        }
    return GTC_OK;
}

int gtc_compute_3pcf(const int32_t *d_xyz_data, int64_t n_data, const double *d_w_data,
                     const int32_t *d_xyz_rand, int64_t n_rand, const double *d_w_rand,
                     const int64_t *h_edges_sq, int32_t nbins, const gtc_options *opt,
                     double *h_zeta, double *h_nnn, double *h_rrr, gtc_stats *st,
                     void *hip_stream) {
    GTC_TRY(check_catalogues("gtc_compute_3pcf", d_xyz_data, n_data, d_xyz_rand, n_rand));
    if (!h_zeta) {
        set_error("gtc_compute_3pcf: h_zeta is NULL");
        return GTC_E_INVALID;
    }
    const int64_t ncfg = gtc_num_configs(3, nbins);
    if (ncfg < 0) {
        set_error("gtc_compute_3pcf: nbins %d out of range", nbins);
        return GTC_E_INVALID;
    }
    AllocScope alloc_scope(opt ? opt->allocator : nullptr);
    hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
    Catalogue cat;
    GTC_TRY(make_weights(d_w_data, n_data, d_w_rand, n_rand, s, &cat));
    DeviceUnion u;
    int rc = make_union(d_xyz_data, n_data, d_xyz_rand, n_rand, cat, s, &u);
    gtc_graph g = nullptr, gr = nullptr;
    if (!rc) rc = gtc_build_graph(u.xyz, n_data + n_rand, h_edges_sq, nbins, opt, hip_stream, &g);
    if (!rc) rc = gtc_build_graph(d_xyz_rand, n_rand, h_edges_sq, nbins, opt, hip_stream, &gr);
    uint64_t *d_counts = nullptr;
    double *d_sum = nullptr;
    void *blk = nullptr;
    if (!rc) rc = carve_alloc(&blk, s, [&](Carver &c) {
        c.take(&d_counts, ncfg);
        c.take(&d_sum, ncfg);
    });
    std::vector<double> nnn, rrr;
    gtc_stats st1{}, st2{};
    if (!rc) rc = gtc_count_3pcf(g, u.w_signed, d_counts, d_sum, &st1, hip_stream);
    if (!rc) rc = to_host(nnn, d_sum, ncfg, s);
    if (!rc) rc = gtc_count_3pcf(gr, u.w_rand, d_counts, d_sum, &st2, hip_stream);
    if (!rc) rc = to_host(rrr, d_sum, ncfg, s);
    if (!rc) {
        for (int64_t c = 0; c < ncfg; ++c) {
            h_zeta[c] = nnn[c] / rrr[c];  // no random triple in a configuration: not a number
            if (h_nnn) h_nnn[c] = nnn[c];
            if (h_rrr) h_rrr[c] = rrr[c];
        }
        if (st) {
            *st = st1;
            st->kernel_ms = st1.kernel_ms + st2.kernel_ms;
            st->count_ms = st1.count_ms + st2.count_ms;
        }
    }
    if (g) gtc_graph_free(g);
    if (gr) gtc_graph_free(gr);
    dev_free(blk, s);
    dev_free(u.block, s);
    (void)hipStreamSynchronize(s);
    return rc;
}

int gtc_compute_4pcf(const int32_t *d_xyz_data, int64_t n_data, const double *d_w_data,
                     const int32_t *d_xyz_rand, int64_t n_rand, const double *d_w_rand,
                     const int64_t *h_edges_sq, int32_t nbins, const gtc_options *opt,
                     double *h_zeta_even, double *h_zeta_odd, double *h_zeta_conn, double *h_xi,
                     gtc_stats *st, void *hip_stream) {
    GTC_TRY(check_catalogues("gtc_compute_4pcf", d_xyz_data, n_data, d_xyz_rand, n_rand));
    if (!h_zeta_even || !h_zeta_odd) {
        set_error("gtc_compute_4pcf: h_zeta_even and h_zeta_odd are required");
        return GTC_E_INVALID;
    }
    const int64_t ncfg = gtc_num_configs_s4(nbins);
    if (ncfg < 0) {
        set_error("gtc_compute_4pcf: nbins %d out of range [1, %d]", nbins, GTC_MAX_BINS_4PCF);
        return GTC_E_INVALID;
    }
    if (opt && opt->drop_coords) {
        set_error("gtc_compute_4pcf: the 4-clique kernel needs the coordinates (drop_coords)");
        return GTC_E_INVALID;
    }
    AllocScope alloc_scope(opt ? opt->allocator : nullptr);
    hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
    Catalogue cat;
    GTC_TRY(make_weights(d_w_data, n_data, d_w_rand, n_rand, s, &cat));
    DeviceUnion u;
    int rc = make_union(d_xyz_data, n_data, d_xyz_rand, n_rand, cat, s, &u);
    gtc_graph g = nullptr, gr = nullptr;
    if (!rc) rc = gtc_build_graph(u.xyz, n_data + n_rand, h_edges_sq, nbins, opt, hip_stream, &g);
    if (!rc) rc = gtc_build_graph(d_xyz_rand, n_rand, h_edges_sq, nbins, opt, hip_stream, &gr);
    uint64_t *d_even = nullptr, *d_pairs = nullptr;
    int64_t *d_odd = nullptr;
    double *d_ew = nullptr, *d_ow = nullptr, *d_pw = nullptr;
    void *blk = nullptr;
    if (!rc) rc = carve_alloc(&blk, s, [&](Carver &c) {
        c.take(&d_even, ncfg);
        c.take(&d_odd, ncfg);
        c.take(&d_ew, ncfg);
        c.take(&d_ow, ncfg);
        c.take(&d_pairs, nbins);
        c.take(&d_pw, nbins);
    });
    std::vector<double> ne, no, rr4, nn, rr;
    gtc_stats st1{}, st2{}, st3{}, st4{};
    if (!rc) rc = gtc_count_4pcf_weighted(g, u.w_signed, 1, d_even, d_odd, d_ew, d_ow, &st1, hip_stream);
    if (!rc) rc = to_host(ne, d_ew, ncfg, s);
    if (!rc) rc = to_host(no, d_ow, ncfg, s);
    if (!rc) rc = gtc_count_4pcf_weighted(gr, u.w_rand, 1, d_even, d_odd, d_ew, d_ow, &st2, hip_stream);
    if (!rc) rc = to_host(rr4, d_ew, ncfg, s);
    if (!rc) rc = gtc_count_2pcf(g, u.w_signed, d_pairs, d_pw, &st3, hip_stream);
    if (!rc) rc = to_host(nn, d_pw, nbins, s);
    if (!rc) rc = gtc_count_2pcf(gr, u.w_rand, d_pairs, d_pw, &st4, hip_stream);
    if (!rc) rc = to_host(rr, d_pw, nbins, s);
    if (!rc) {
        std::vector<double> xi(nbins), disc(ncfg);
        for (int b = 0; b < nbins; ++b) xi[b] = nn[b] / rr[b];
        disconnected_4pcf_s4(nbins, xi.data(), disc.data());
        for (int64_t c = 0; c < ncfg; ++c) {
            h_zeta_even[c] = ne[c] / rr4[c];
            h_zeta_odd[c] = no[c] / rr4[c];
            if (h_zeta_conn) h_zeta_conn[c] = h_zeta_even[c] - disc[c];  // Eq. (5)
        }
        if (h_xi) std::memcpy(h_xi, xi.data(), sizeof(double) * nbins);
        if (st) {
            *st = st1;
            st->kernel_ms = st1.kernel_ms + st2.kernel_ms + st3.kernel_ms + st4.kernel_ms;
            st->count_ms = st1.count_ms + st2.count_ms + st3.count_ms + st4.count_ms;
        }
    }
    if (g) gtc_graph_free(g);
    if (gr) gtc_graph_free(gr);
    dev_free(blk, s);
    dev_free(u.block, s);
    (void)hipStreamSynchronize(s);
    return rc;
}

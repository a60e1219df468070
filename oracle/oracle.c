/* oracle.c - plain CPU reference for the graph-based 3pCF / 4pCF counts.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): used by the tests, the smoke check and the benchmark's
 * CPU-baseline leg; never by the product library.  Written for obviousness, not speed: a cell
 * list to find neighbours, sorted rows, and the pages' own two- and three-pointer walks.
 *
 * Citations are to GRAMSCI v2, "Fast Graph-based Higher-Order Clustering Statistics on the GPU".
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (oracle/build.py).  -ffp-contract=off
 * keeps the weight product as two separately rounded multiplies.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GRID_SIDE (1 << 20)

struct oracle_graph_s {
    int64_t n;
    int32_t nb;
    int64_t edges[ORACLE_MAX_BINS + 1];
    int64_t *row_ptr; /* [n+1] */
    int32_t *col;     /* [nnz], each row ascending (Eq.(1)) */
    uint8_t *bin;     /* [nnz] radial-bin byte per edge (§II.1) */
};

/* ---------------------------------------------------------------- small helpers */

static int64_t sq_dist(const int32_t *p, const int32_t *q) {
    int64_t dx = (int64_t)p[0] - q[0], dy = (int64_t)p[1] - q[1], dz = (int64_t)p[2] - q[2];
    return dx * dx + dy * dy + dz * dz;
}

/* The bin of squared distance d2: the b with e_b <= d2 < e_{b+1}; -1 when outside [e_0, e_nb). */
static int bin_of(const int64_t *edges, int nb, int64_t d2) {
    if (d2 < edges[0] || d2 >= edges[nb]) return -1;
    int b = 0;
    while (d2 >= edges[b + 1]) b++;
    return b;
}

static int set_threads(int32_t nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

static int cmp_i64(const void *a, const void *b) {
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

static int64_t binom(int64_t n, int64_t k) {
    if (k < 0 || n < k) return 0;
    int64_t r = 1;
    for (int64_t t = 1; t <= k; t++) r = r * (n - k + t) / t;
    return r;
}

int64_t oracle_num_configs(int32_t order, int32_t nbins) {
    if (nbins < 1) return 0;
    if (order == 3) return binom(nbins + 2, 3);
    if (order == 4) return binom(nbins + 5, 6);
    return 0;
}

/* ---------------------------------------------------------------- graph (§II.1, Eq.(1)) */

static int validate_inputs(int64_t n, const int32_t *xyz, int32_t nb, const int64_t *edges) {
    if (n < 0 || n >= ((int64_t)1 << 31) || (n > 0 && !xyz) || !edges) return ORACLE_E_INVALID;
    if (nb < 1 || nb > ORACLE_MAX_BINS || edges[0] < 0) return ORACLE_E_INVALID;
    for (int b = 0; b < nb; b++)
        if (edges[b + 1] <= edges[b]) return ORACLE_E_INVALID;
    if (edges[nb] > 3 * (int64_t)GRID_SIDE * GRID_SIDE + 1) return ORACLE_E_INVALID;
    for (int64_t i = 0; i < 3 * n; i++)
        if (xyz[i] < 0 || xyz[i] >= GRID_SIDE) return ORACLE_E_INVALID;
    return 0;
}

static int build_graph_impl(int64_t n, const int32_t *xyz, int32_t nb, const int64_t *edges,
                            int32_t nthreads, int forward, oracle_graph **out) {
    if (!out) return ORACLE_E_INVALID;
    *out = NULL;
    int rc = validate_inputs(n, xyz, nb, edges);
    if (rc) return rc;
    int nt = set_threads(nthreads);

    oracle_graph *g = (oracle_graph *)calloc(1, sizeof(*g));
    if (!g) return ORACLE_E_NOMEM;
    g->n = n;
    g->nb = nb;
    memcpy(g->edges, edges, sizeof(int64_t) * (size_t)(nb + 1));

    /* Cell list: cubic cells of integer side cs >= r_max, so every neighbour is in one of the 27
     * cells around a point.  The grid is kept to at most ~2n cells (and 256 per axis). */
    int64_t cs = (int64_t)sqrt((double)edges[nb]);
    while (cs * cs < edges[nb]) cs++;
    if (cs < 1) cs = 1;
    int64_t gdim = (GRID_SIDE + cs - 1) / cs;
    int64_t gcap = 1;
    while ((gcap + 1) * (gcap + 1) * (gcap + 1) <= 2 * (n > 0 ? n : 1) && gcap < 256) gcap++;
    if (gdim > gcap) {
        gdim = gcap;
        cs = (GRID_SIDE + gdim - 1) / gdim;
    }
    int64_t ncell = gdim * gdim * gdim;

    int64_t *cell_start = (int64_t *)calloc((size_t)ncell + 1, sizeof(int64_t));
    int32_t *by_cell = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int64_t *cell_of = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    int64_t *deg = (int64_t *)calloc((size_t)(n > 0 ? n : 1), sizeof(int64_t));
    g->row_ptr = (int64_t *)calloc((size_t)n + 1, sizeof(int64_t));
    if (!cell_start || !by_cell || !cell_of || !deg || !g->row_ptr) {
        free(cell_start); free(by_cell); free(cell_of); free(deg);
        oracle_graph_free(g);
        return ORACLE_E_NOMEM;
    }
    for (int64_t i = 0; i < n; i++) {
        const int32_t *p = xyz + 3 * i;
        cell_of[i] = ((p[2] / cs) * gdim + p[1] / cs) * gdim + p[0] / cs;
        cell_start[cell_of[i] + 1]++;
    }
    for (int64_t c = 0; c < ncell; c++) cell_start[c + 1] += cell_start[c];
    {
        int64_t *fill = (int64_t *)malloc(sizeof(int64_t) * (size_t)ncell);
        if (!fill) { free(cell_start); free(by_cell); free(cell_of); free(deg); oracle_graph_free(g); return ORACLE_E_NOMEM; }
        memcpy(fill, cell_start, sizeof(int64_t) * (size_t)ncell);
        for (int64_t i = 0; i < n; i++) by_cell[fill[cell_of[i]]++] = (int32_t)i;
        free(fill);
    }

    /* Two passes over the same traversal: count, then fill. */
    for (int pass = 0; pass < 2; pass++) {
        #pragma omp parallel for schedule(dynamic, 256) num_threads(nt)
        for (int64_t i = 0; i < n; i++) {
            const int32_t *p = xyz + 3 * i;
            int64_t cx = p[0] / cs, cy = p[1] / cs, cz = p[2] / cs;
            int64_t cnt = 0;
            int64_t w = pass ? g->row_ptr[i] : 0;
            for (int64_t dz = -1; dz <= 1; dz++)
                for (int64_t dy = -1; dy <= 1; dy++)
                    for (int64_t dx = -1; dx <= 1; dx++) {
                        int64_t x = cx + dx, y = cy + dy, z = cz + dz;
                        if (x < 0 || y < 0 || z < 0 || x >= gdim || y >= gdim || z >= gdim) continue;
                        int64_t c = (z * gdim + y) * gdim + x;
                        for (int64_t t = cell_start[c]; t < cell_start[c + 1]; t++) {
                            int32_t j = by_cell[t];
                            if (j == i || (forward && j < i)) continue;
                            int b = bin_of(edges, nb, sq_dist(p, xyz + 3 * (int64_t)j));
                            if (b < 0) continue;
                            if (pass) {
                                g->col[w] = j;
                                g->bin[w] = (uint8_t)b;
                                w++;
                            } else {
                                cnt++;
                            }
                        }
                    }
            if (!pass) deg[i] = cnt;
        }
        if (!pass) {
            for (int64_t i = 0; i < n; i++) g->row_ptr[i + 1] = g->row_ptr[i] + deg[i];
            int64_t nnz = g->row_ptr[n];
            g->col = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
            g->bin = (uint8_t *)malloc((size_t)(nnz > 0 ? nnz : 1));
            if (!g->col || !g->bin) {
                free(cell_start); free(by_cell); free(cell_of); free(deg);
                oracle_graph_free(g);
                return ORACLE_E_NOMEM;
            }
        }
    }
    free(cell_start); free(by_cell); free(cell_of); free(deg);

    /* Sort each row by neighbour label (Eq.(1)), carrying the bin byte along. */
    int fail = 0;
    #pragma omp parallel for schedule(dynamic, 256) num_threads(nt) reduction(|:fail)
    for (int64_t i = 0; i < n; i++) {
        int64_t a = g->row_ptr[i], e = g->row_ptr[i + 1];
        if (e - a < 2) continue;
        int64_t *tmp = (int64_t *)malloc(sizeof(int64_t) * (size_t)(e - a));
        if (!tmp) { fail = 1; continue; }
        for (int64_t t = a; t < e; t++) tmp[t - a] = ((int64_t)g->col[t] << 8) | g->bin[t];
        qsort(tmp, (size_t)(e - a), sizeof(int64_t), cmp_i64);
        for (int64_t t = a; t < e; t++) {
            g->col[t] = (int32_t)(tmp[t - a] >> 8);
            g->bin[t] = (uint8_t)(tmp[t - a] & 0xff);
        }
        free(tmp);
    }
    if (fail) { oracle_graph_free(g); return ORACLE_E_NOMEM; }
    *out = g;
    return 0;
}

int oracle_build_graph(int64_t n, const int32_t *xyz, int32_t nb, const int64_t *edges,
                       int32_t nthreads, oracle_graph **out) {
    return build_graph_impl(n, xyz, nb, edges, nthreads, 0, out);
}

/* Only the neighbours above each point are kept: every walk of the 3pCF and 4pCF counts reads
 * row entries beyond the spoke's own label, so the counts are those of the full graph. */
int oracle_build_graph_forward(int64_t n, const int32_t *xyz, int32_t nb, const int64_t *edges,
                               int32_t nthreads, oracle_graph **out) {
    return build_graph_impl(n, xyz, nb, edges, nthreads, 1, out);
}

void oracle_graph_free(oracle_graph *g) {
    if (!g) return;
    free(g->row_ptr);
    free(g->col);
    free(g->bin);
    free(g);
}

int64_t oracle_graph_n(const oracle_graph *g) { return g ? g->n : -1; }
int64_t oracle_graph_nnz(const oracle_graph *g) { return g ? g->row_ptr[g->n] : -1; }

int oracle_graph_export(const oracle_graph *g, int64_t *row_ptr, int32_t *col, uint8_t *bin) {
    if (!g || !row_ptr || !col || !bin) return ORACLE_E_INVALID;
    int64_t nnz = g->row_ptr[g->n];
    memcpy(row_ptr, g->row_ptr, sizeof(int64_t) * (size_t)(g->n + 1));
    memcpy(col, g->col, sizeof(int32_t) * (size_t)nnz);
    memcpy(bin, g->bin, (size_t)nnz);
    return 0;
}

int oracle_forward_degrees(const oracle_graph *g, int32_t *deg_out) {
    if (!g || !deg_out) return ORACLE_E_INVALID;
    for (int64_t i = 0; i < g->n; i++) {
        int32_t c = 0;
        for (int64_t t = g->row_ptr[i]; t < g->row_ptr[i + 1]; t++) c += g->col[t] > i;
        deg_out[i] = c;
    }
    return 0;
}

/* ---------------------------------------------------------------- configuration ranks */

/* rank3[(b1*nb + b2)*nb + b3] for b1 <= b2 <= b3, numbered in nested-loop order (§V.1). */
static int32_t *make_rank3(int nb) {
    int32_t *t = (int32_t *)malloc(sizeof(int32_t) * (size_t)nb * nb * nb);
    if (!t) return NULL;
    int32_t r = 0;
    for (int a = 0; a < nb; a++)
        for (int b = a; b < nb; b++)
            for (int c = b; c < nb; c++) t[((size_t)a * nb + b) * nb + c] = r++;
    return t;
}

/* rank6 over nondecreasing 6-tuples, indexed in base nb, nested-loop order. */
static int32_t *make_rank6(int nb) {
    size_t sz = 1;
    for (int k = 0; k < 6; k++) sz *= (size_t)nb;
    int32_t *t = (int32_t *)malloc(sizeof(int32_t) * sz);
    if (!t) return NULL;
    int32_t r = 0;
    for (int a = 0; a < nb; a++)
        for (int b = a; b < nb; b++)
            for (int c = b; c < nb; c++)
                for (int d = c; d < nb; d++)
                    for (int e = d; e < nb; e++)
                        for (int f = e; f < nb; f++)
                            t[(((((size_t)a * nb + b) * nb + c) * nb + d) * nb + e) * nb + f] = r++;
    return t;
}

static void sort_small_int(int *v, int k) {
    for (int x = 1; x < k; x++)
        for (int y = x; y > 0 && v[y - 1] > v[y]; y--) {
            int t = v[y]; v[y] = v[y - 1]; v[y - 1] = t;
        }
}

/* ---------------------------------------------------------------- weights */

/* Scale exponent s of the exact weighted sums (see oracle.h). */
static int weight_scale(const double *w, int64_t n) {
    double a = 0.0;
    for (int64_t i = 0; i < n; i++) a = fmax(a, fabs(w[i]));
    double m = (a * a) * a;
    if (m == 0.0) return 0;
    int e;
    frexp(m, &e);
    return 57 - e;
}

static int weights_finite(const double *w, int64_t n) {
    for (int64_t i = 0; i < n; i++)
        if (!isfinite(w[i])) return 0;
    return 1;
}

/* q = rint(p * 2^s) for p = fl(fl(w1*w2)*w3), w1 <= w2 <= w3. */
static int64_t triangle_q(double wa, double wb, double wc, int s) {
    double t;
    if (wa > wb) { t = wa; wa = wb; wb = t; }
    if (wb > wc) { t = wb; wb = wc; wc = t; }
    if (wa > wb) { t = wa; wa = wb; wb = t; }
    volatile double p12 = wa * wb; /* two separately rounded products, no fusion */
    volatile double p = p12 * wc;
    return (int64_t)rint(ldexp(p, s));
}

/* ---------------------------------------------------------------- 3pCF (§II.2, §III.1) */

static int count_3pcf_impl(const oracle_graph *g, const double *w, int64_t hub_stride,
                           int64_t hub_offset, int32_t nthreads, uint64_t *counts, __int128 *acc,
                           int *scale_out, uint64_t *walks_out) {
    if (!g || !counts || hub_stride < 1 || hub_offset < 0 || hub_offset >= hub_stride)
        return ORACLE_E_INVALID;
    if (w && !weights_finite(w, g->n)) return ORACLE_E_INVALID;
    const int nb = g->nb;
    const int64_t ncfg = oracle_num_configs(3, nb);
    int32_t *rank3 = make_rank3(nb);
    if (!rank3) return ORACLE_E_NOMEM;
    const int s = w ? weight_scale(w, g->n) : 0;
    int nt = set_threads(nthreads);
    memset(counts, 0, sizeof(uint64_t) * (size_t)ncfg);
    if (acc) memset(acc, 0, sizeof(__int128) * (size_t)ncfg);
    uint64_t walks = 0;
    int fail = 0;

    #pragma omp parallel num_threads(nt) reduction(+:walks) reduction(|:fail)
    {
        uint64_t *my = (uint64_t *)calloc((size_t)ncfg, sizeof(uint64_t));
        __int128 *myacc = acc ? (__int128 *)calloc((size_t)ncfg, sizeof(__int128)) : NULL;
        if (!my || (acc && !myacc)) fail = 1;
        #pragma omp for schedule(dynamic, 64)
        for (int64_t i = 0; i < g->n; i++) {
            if (fail || i % hub_stride != hub_offset) continue;
            const int64_t ie = g->row_ptr[i + 1];
            for (int64_t sj = g->row_ptr[i]; sj < ie; sj++) {
                const int32_t j = g->col[sj];
                if (j <= i) continue; /* spoke j > i; the triangle's hub is its smallest label */
                walks++;
                /* Merge-walk (§III.1): pointer a on the hub tail {k in N(i): k > j}, pointer b on
                 * N(j) from its start.  Equal -> triangle, advance both; else advance the smaller. */
                int64_t a = sj + 1, b = g->row_ptr[j];
                const int64_t je = g->row_ptr[j + 1];
                while (a < ie && b < je) {
                    const int32_t ka = g->col[a], kb = g->col[b];
                    if (ka == kb) {
                        int v[3] = {g->bin[sj], g->bin[a], g->bin[b]}; /* r_ij, r_ik, r_jk */
                        sort_small_int(v, 3);
                        const int32_t c = rank3[((size_t)v[0] * nb + v[1]) * nb + v[2]];
                        my[c]++;
                        if (myacc) myacc[c] += triangle_q(w[i], w[j], w[ka], s);
                        a++;
                        b++;
                    } else if (ka < kb) {
                        a++;
                    } else {
                        b++;
                    }
                }
            }
        }
        #pragma omp critical
        {
            if (my)
                for (int64_t c = 0; c < ncfg; c++) counts[c] += my[c];
            if (myacc)
                for (int64_t c = 0; c < ncfg; c++) acc[c] += myacc[c];
        }
        free(my);
        free(myacc);
    }
    free(rank3);
    if (fail) return ORACLE_E_NOMEM;
    if (scale_out) *scale_out = s;
    if (walks_out) *walks_out = walks;
    return 0;
}

int oracle_count_3pcf(const oracle_graph *g, const double *w, int64_t hub_stride,
                      int32_t nthreads, uint64_t *counts, double *weighted, int32_t *scale_out,
                      uint64_t *walks_out) {
    return oracle_count_3pcf_part(g, w, hub_stride, 0, nthreads, counts, weighted, scale_out,
                                  walks_out);
}

int oracle_count_3pcf_part(const oracle_graph *g, const double *w, int64_t hub_stride,
                           int64_t hub_offset, int32_t nthreads, uint64_t *counts,
                           double *weighted, int32_t *scale_out, uint64_t *walks_out) {
    if (!g) return ORACLE_E_INVALID;
    const int64_t ncfg = oracle_num_configs(3, g->nb);
    __int128 *acc = NULL;
    if (w) {
        if (!weighted) return ORACLE_E_INVALID;
        acc = (__int128 *)malloc(sizeof(__int128) * (size_t)ncfg);
        if (!acc) return ORACLE_E_NOMEM;
    }
    int s = 0;
    int rc = count_3pcf_impl(g, w, hub_stride, hub_offset, nthreads, counts, acc, &s, walks_out);
    if (!rc && w) {
        /* one rounding of the exact sum, then an exact power-of-two scaling */
        for (int64_t c = 0; c < ncfg; c++) weighted[c] = ldexp((double)acc[c], -s);
    }
    if (!rc && scale_out) *scale_out = s;
    free(acc);
    return rc;
}

int oracle_count_3pcf_exact(const oracle_graph *g, const double *w, int64_t hub_stride,
                            int32_t nthreads, uint64_t *counts, int64_t *sum_q128,
                            int32_t *scale_out) {
    if (!g || !w || !sum_q128) return ORACLE_E_INVALID;
    const int64_t ncfg = oracle_num_configs(3, g->nb);
    __int128 *acc = (__int128 *)malloc(sizeof(__int128) * (size_t)ncfg);
    if (!acc) return ORACLE_E_NOMEM;
    int s = 0;
    int rc = count_3pcf_impl(g, w, hub_stride, 0, nthreads, counts, acc, &s, NULL);
    if (!rc) {
        for (int64_t c = 0; c < ncfg; c++) {
            unsigned __int128 u = (unsigned __int128)acc[c];
            sum_q128[2 * c] = (int64_t)(uint64_t)u;
            sum_q128[2 * c + 1] = (int64_t)(uint64_t)(u >> 64);
        }
        if (scale_out) *scale_out = s;
    }
    free(acc);
    return rc;
}

/* ---------------------------------------------------------------- 2pCF (§II.1, §III.3) */

/* Pairs per bin, each pair once; weighted: sum of p = fl(w_i * w_j), each scaled to the integer
 * q = rint(p * 2^s) and summed exactly, then rounded once (s = 57 - e for M = fl(a * a) = f 2^e,
 * a = max |w|, so |q| < 2^57). */
int oracle_count_2pcf(const oracle_graph *g, const double *w, uint64_t *counts, double *weighted,
                      int32_t *scale_out) {
    if (!g || !counts || (w && !weighted)) return ORACLE_E_INVALID;
    if (w && !weights_finite(w, g->n)) return ORACLE_E_INVALID;
    const int nb = g->nb;
    __int128 *acc = w ? (__int128 *)calloc((size_t)nb, sizeof(__int128)) : NULL;
    if (w && !acc) return ORACLE_E_NOMEM;
    int s = 0;
    if (w) {
        double a = 0.0;
        for (int64_t i = 0; i < g->n; i++) a = fmax(a, fabs(w[i]));
        const double m = a * a;
        if (m != 0.0) {
            int e;
            frexp(m, &e);
            s = 57 - e;
        }
    }
    memset(counts, 0, sizeof(uint64_t) * (size_t)nb);
    for (int64_t i = 0; i < g->n; i++)
        for (int64_t e = g->row_ptr[i]; e < g->row_ptr[i + 1]; e++) {
            const int32_t j = g->col[e];
            if (j <= i) continue; /* each pair once */
            counts[g->bin[e]]++;
            if (w) {
                volatile double p = w[i] * w[j];
                acc[g->bin[e]] += (int64_t)rint(ldexp(p, s));
            }
        }
    if (w)
        for (int b = 0; b < nb; b++) weighted[b] = ldexp((double)acc[b], -s);
    free(acc);
    if (scale_out) *scale_out = s;
    return 0;
}

/* Eq. (4) per S4 configuration: the three ways of splitting the four vertices into two pairs are
 * the edge pairs (01, 23), (02, 13), (03, 12) of the canonical tuple. */
int oracle_disconnected_4pcf_s4(int32_t nb, const double *xi, double *disc) {
    if (nb < 1 || nb > ORACLE_MAX_BINS_4PCF || !xi || !disc) return ORACLE_E_INVALID;
    const int64_t ncfg = oracle_num_configs_s4(nb);
    int32_t *bins = (int32_t *)malloc(sizeof(int32_t) * 6 * (size_t)ncfg);
    if (!bins) return ORACLE_E_NOMEM;
    oracle_config_bins_s4(nb, bins);
    for (int64_t c = 0; c < ncfg; c++) {
        const int32_t *t = bins + 6 * c;
        disc[c] = xi[t[0]] * xi[t[5]] + xi[t[1]] * xi[t[4]] + xi[t[2]] * xi[t[3]];
    }
    free(bins);
    return 0;
}

/* ---------------------------------------------------------------- 3pCF at chosen hubs */

/* The definition written out, with no graph: the forward neighbours of hub h are the points j > h
 * with e_0 <= d^2(h, j) < e_nb (all n points are tested); every pair j < k of them that are
 * neighbours of each other closes the triangle {h, j, k}, whose smallest label is h (§II.2). */
int oracle_count_3pcf_hubs(int64_t n, const int32_t *xyz, int32_t nb, const int64_t *edges,
                           const double *w, const int32_t *hubs, int64_t nh, int32_t nthreads,
                           uint64_t *counts, double *weighted, int32_t *scale_out) {
    int rc = validate_inputs(n, xyz, nb, edges);
    if (rc) return rc;
    if (nh < 0 || (nh > 0 && !hubs) || !counts || (w && !weighted)) return ORACLE_E_INVALID;
    if (w && !weights_finite(w, n)) return ORACLE_E_INVALID;
    uint8_t *seen = (uint8_t *)calloc((size_t)(n > 0 ? n : 1), 1);
    if (!seen) return ORACLE_E_NOMEM;
    for (int64_t t = 0; t < nh; t++) {
        if (hubs[t] < 0 || hubs[t] >= n || seen[hubs[t]]) {
            free(seen);
            return ORACLE_E_INVALID; /* labels in range and distinct */
        }
        seen[hubs[t]] = 1;
    }
    free(seen);
    const int64_t ncfg = oracle_num_configs(3, nb);
    int32_t *rank3 = make_rank3(nb);
    __int128 *acc = w ? (__int128 *)calloc((size_t)ncfg, sizeof(__int128)) : NULL;
    if (!rank3 || (w && !acc)) {
        free(rank3);
        free(acc);
        return ORACLE_E_NOMEM;
    }
    const int s = w ? weight_scale(w, n) : 0;
    memset(counts, 0, sizeof(uint64_t) * (size_t)ncfg);
    int nt = set_threads(nthreads);
    int fail = 0;

    #pragma omp parallel num_threads(nt) reduction(|:fail)
    {
        uint64_t *my = (uint64_t *)calloc((size_t)ncfg, sizeof(uint64_t));
        __int128 *myacc = w ? (__int128 *)calloc((size_t)ncfg, sizeof(__int128)) : NULL;
        int64_t cap = 1024, m = 0;
        int32_t *fj = (int32_t *)malloc(sizeof(int32_t) * (size_t)cap);
        int *fb = (int *)malloc(sizeof(int) * (size_t)cap);
        if (!my || (w && !myacc) || !fj || !fb) fail = 1;
        #pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nh; t++) {
            if (fail) continue;
            const int32_t h = hubs[t];
            m = 0;
            for (int64_t j = (int64_t)h + 1; j < n; j++) {
                const int b = bin_of(edges, nb, sq_dist(xyz + 3 * (int64_t)h, xyz + 3 * j));
                if (b < 0) continue;
                if (m == cap) {
                    cap *= 2;
                    int32_t *nj = (int32_t *)realloc(fj, sizeof(int32_t) * (size_t)cap);
                    int *nbp = (int *)realloc(fb, sizeof(int) * (size_t)cap);
                    if (nj) fj = nj;
                    if (nbp) fb = nbp;
                    if (!nj || !nbp) { fail = 1; break; }
                }
                fj[m] = (int32_t)j;
                fb[m] = b;
                m++;
            }
            if (fail) continue;
            for (int64_t a = 0; a < m; a++)
                for (int64_t c2 = a + 1; c2 < m; c2++) {
                    const int bjk = bin_of(edges, nb,
                                           sq_dist(xyz + 3 * (int64_t)fj[a], xyz + 3 * (int64_t)fj[c2]));
                    if (bjk < 0) continue;
                    int v[3] = {fb[a], fb[c2], bjk}; /* r_hj, r_hk, r_jk */
                    sort_small_int(v, 3);
                    const int32_t c = rank3[((size_t)v[0] * nb + v[1]) * nb + v[2]];
                    my[c]++;
                    if (myacc) myacc[c] += triangle_q(w[h], w[fj[a]], w[fj[c2]], s);
                }
        }
        #pragma omp critical
        {
            if (my)
                for (int64_t c = 0; c < ncfg; c++) counts[c] += my[c];
            if (myacc)
                for (int64_t c = 0; c < ncfg; c++) acc[c] += myacc[c];
        }
        free(my);
        free(myacc);
        free(fj);
        free(fb);
    }
    free(rank3);
    if (!fail && w)
        for (int64_t c = 0; c < ncfg; c++) weighted[c] = ldexp((double)acc[c], -s);
    free(acc);
    if (fail) return ORACLE_E_NOMEM;
    if (scale_out) *scale_out = s;
    return 0;
}

/* ---------------------------------------------------------------- parity 4pCF (§III.1.1, §III.2) */

/* Sign of the signed volume Eq.(3) in the label-free vertex order (see oracle.h). */
static int parity_sign(const int32_t *xyz, const int32_t v_in[4]) {
    int64_t d2[4][4];
    for (int a = 0; a < 4; a++)
        for (int b = 0; b < 4; b++)
            d2[a][b] = sq_dist(xyz + 3 * (int64_t)v_in[a], xyz + 3 * (int64_t)v_in[b]);
    int64_t key[4];
    int ord[4];
    for (int a = 0; a < 4; a++) {
        key[a] = 0;
        for (int b = 0; b < 4; b++) key[a] += d2[a][b]; /* d2[a][a] == 0 */
        ord[a] = a;
    }
    for (int x = 1; x < 4; x++)
        for (int y = x; y > 0 && key[ord[y - 1]] > key[ord[y]]; y--) {
            int t = ord[y]; ord[y] = ord[y - 1]; ord[y - 1] = t;
        }
    for (int x = 0; x < 3; x++)
        if (key[ord[x]] == key[ord[x + 1]]) return 0; /* tied keys: no label-free orientation */
    const int32_t *p0 = xyz + 3 * (int64_t)v_in[ord[0]];
    int64_t m[3][3];
    for (int r = 0; r < 3; r++) {
        const int32_t *p = xyz + 3 * (int64_t)v_in[ord[r + 1]];
        for (int c = 0; c < 3; c++) m[r][c] = (int64_t)p[c] - p0[c];
    }
    /* (m0 x m1) . m2 */
    int64_t vol = m[2][0] * (m[0][1] * m[1][2] - m[0][2] * m[1][1])
                + m[2][1] * (m[0][2] * m[1][0] - m[0][0] * m[1][2])
                + m[2][2] * (m[0][0] * m[1][1] - m[0][1] * m[1][0]);
    return (vol > 0) - (vol < 0);
}

/* ---------------------------------------------------------------- S4 configurations (§III.3) */

/* A tetrahedron's six edge bins in the edge order (01, 02, 03, 12, 13, 23) of its vertices 0..3.
 * Relabelling the vertices by a permutation p of {0,1,2,3} moves the bin of edge (u, v) to edge
 * (p(u), p(v)).  A configuration is an orbit of 6-tuples under the 24 relabellings (Eq. (4) and
 * the text after it); its canonical tuple is the lexicographically smallest member. */
static const int S4_EDGE[4][4] = {{-1, 0, 1, 2}, {0, -1, 3, 4}, {1, 3, -1, 5}, {2, 4, 5, -1}};
static const int S4_EU[6] = {0, 0, 0, 1, 1, 2}, S4_EV[6] = {1, 2, 3, 2, 3, 3};

static void s4_canonical(const int t[6], int out[6]) {
    int first = 1;
    for (int p0 = 0; p0 < 4; p0++)
        for (int p1 = 0; p1 < 4; p1++)
            for (int p2 = 0; p2 < 4; p2++)
                for (int p3 = 0; p3 < 4; p3++) {
                    const int p[4] = {p0, p1, p2, p3};
                    if (p0 == p1 || p0 == p2 || p0 == p3 || p1 == p2 || p1 == p3 || p2 == p3) continue;
                    int r[6];
                    for (int e = 0; e < 6; e++) r[S4_EDGE[p[S4_EU[e]]][p[S4_EV[e]]]] = t[e];
                    int less = first;
                    for (int e = 0; e < 6 && !first; e++) {
                        if (r[e] != out[e]) {
                            less = r[e] < out[e];
                            break;
                        }
                    }
                    if (less)
                        for (int e = 0; e < 6; e++) out[e] = r[e];
                    first = 0;
                }
}

static size_t tuple_key(const int t[6], int nb) {
    size_t key = 0;
    for (int e = 0; e < 6; e++) key = key * (size_t)nb + (size_t)t[e];
    return key;
}

static void tuple_of_key(size_t key, int nb, int t[6]) {
    for (int e = 5; e >= 0; e--) {
        t[e] = (int)(key % (size_t)nb);
        key /= (size_t)nb;
    }
}

/* canonical key of every 6-tuple key (all threads), then the configuration ranks: canonical keys
 * numbered in key (lexicographic) order */
static uint32_t *make_canon_s4(int nb, size_t *sz_out) {
    size_t sz = 1;
    for (int k = 0; k < 6; k++) sz *= (size_t)nb;
    uint32_t *c = (uint32_t *)malloc(sizeof(uint32_t) * sz);
    if (!c) return NULL;
    #pragma omp parallel for schedule(static)
    for (int64_t key = 0; key < (int64_t)sz; key++) {
        int v[6], cv[6];
        tuple_of_key((size_t)key, nb, v);
        s4_canonical(v, cv);
        c[key] = (uint32_t)tuple_key(cv, nb);
    }
    *sz_out = sz;
    return c;
}

static int32_t *make_rank_s4(int nb, int64_t *ncfg_out) {
    size_t sz = 0;
    uint32_t *c = make_canon_s4(nb, &sz);
    if (!c) return NULL;
    int32_t *t = (int32_t *)malloc(sizeof(int32_t) * sz);
    if (!t) {
        free(c);
        return NULL;
    }
    int32_t r = 0;
    for (size_t key = 0; key < sz; key++) t[key] = c[key] == key ? r++ : -1;
    #pragma omp parallel for schedule(static)
    for (int64_t key = 0; key < (int64_t)sz; key++)
        if (t[key] < 0) t[key] = t[c[key]];
    free(c);
    if (ncfg_out) *ncfg_out = r;
    return t;
}

int64_t oracle_num_configs_s4(int32_t nbins) {
    if (nbins < 1 || nbins > ORACLE_MAX_BINS_4PCF) return 0;
    size_t sz = 0;
    uint32_t *c = make_canon_s4(nbins, &sz);
    if (!c) return ORACLE_E_NOMEM;
    int64_t n = 0;
    for (size_t key = 0; key < sz; key++) n += c[key] == key;
    free(c);
    return n;
}

int oracle_config_bins_s4(int32_t nb, int32_t *bins) {
    if (nb < 1 || nb > ORACLE_MAX_BINS_4PCF || !bins) return ORACLE_E_INVALID;
    size_t sz = 0;
    uint32_t *c = make_canon_s4(nb, &sz);
    if (!c) return ORACLE_E_NOMEM;
    int64_t r = 0;
    for (size_t key = 0; key < sz; key++) {
        if (c[key] != key) continue;
        int v[6];
        tuple_of_key(key, nb, v);
        for (int e = 0; e < 6; e++) bins[6 * r + e] = v[e];
        r++;
    }
    free(c);
    return 0;
}

/* Cayley-Menger determinants: 16 A^2 of a triangle and 288 V^2 of a tetrahedron from squared
 * edge lengths (5x5 bordered matrix, expanded by Gaussian elimination in long double). */
static long double cm_triangle(long double a, long double b, long double c) {
    return 2 * a * b + 2 * b * c + 2 * c * a - a * a - b * b - c * c;
}

static long double cm_tetrahedron(long double d[4][4]) {
    long double m[5][5];
    for (int i = 0; i < 5; i++)
        for (int j = 0; j < 5; j++) m[i][j] = (i == 0 || j == 0) ? (i == j ? 0 : 1) : d[i - 1][j - 1];
    long double det = 1;
    for (int c = 0; c < 5; c++) {
        int piv = c;
        for (int r = c + 1; r < 5; r++)
            if (fabsl(m[r][c]) > fabsl(m[piv][c])) piv = r;
        if (m[piv][c] == 0) return 0;
        if (piv != c) {
            for (int k = 0; k < 5; k++) { long double t = m[c][k]; m[c][k] = m[piv][k]; m[piv][k] = t; }
            det = -det;
        }
        det *= m[c][c];
        for (int r = c + 1; r < 5; r++) {
            const long double f = m[r][c] / m[c][c];
            for (int k = c; k < 5; k++) m[r][k] -= f * m[c][k];
        }
    }
    return det;
}

int oracle_config_realizable_s4(int32_t nb, const int64_t *edges, uint8_t *mask) {
    if (nb < 1 || nb > ORACLE_MAX_BINS_4PCF || !edges || !mask) return ORACLE_E_INVALID;
    const int64_t ncfg = oracle_num_configs_s4(nb);
    int32_t *bins = (int32_t *)malloc(sizeof(int32_t) * 6 * (size_t)ncfg);
    if (!bins) return ORACLE_E_NOMEM;
    oracle_config_bins_s4(nb, bins);
    for (int64_t c = 0; c < ncfg; c++) {
        long double d[4][4] = {{0}};
        for (int e = 0; e < 6; e++) {
            const int b = bins[6 * c + e];
            const long double r = 0.5L * (sqrtl((long double)edges[b]) + sqrtl((long double)edges[b + 1]));
            d[S4_EU[e]][S4_EV[e]] = d[S4_EV[e]][S4_EU[e]] = r * r; /* bin centre in r, squared */
        }
        int ok = cm_tetrahedron(d) > 0;
        for (int f = 0; f < 4 && ok; f++) { /* the face opposite vertex f */
            int u[3], k = 0;
            for (int q = 0; q < 4; q++)
                if (q != f) u[k++] = q;
            ok = cm_triangle(d[u[0]][u[1]], d[u[1]][u[2]], d[u[0]][u[2]]) > 0;
        }
        mask[c] = (uint8_t)ok;
    }
    free(bins);
    return 0;
}

/* Scale of the exact 4pCF weighted sums: s = 57 - e with M = fl(fl(fl(a*a)*a)*a) = f * 2^e for
 * a = max|w|, so |q| < 2^57 for every product of four weights (s = 0 if M == 0). */
static int weight_scale4(const double *w, int64_t n) {
    double a = 0.0;
    for (int64_t i = 0; i < n; i++) a = fmax(a, fabs(w[i]));
    volatile double a2 = a * a;
    volatile double a3 = a2 * a;
    volatile double m = a3 * a;
    if (m == 0.0) return 0;
    int e;
    frexp(m, &e);
    return 57 - e;
}

/* q = rint(p * 2^s) for p = fl(fl(fl(w1*w2)*w3)*w4), the four weights ascending. */
static int64_t tetra_q(const double *wv, int s) {
    double v[4] = {wv[0], wv[1], wv[2], wv[3]};
    for (int x = 1; x < 4; x++)
        for (int y = x; y > 0 && v[y - 1] > v[y]; y--) {
            double t = v[y]; v[y] = v[y - 1]; v[y - 1] = t;
        }
    volatile double p12 = v[0] * v[1];
    volatile double p123 = p12 * v[2];
    volatile double p = p123 * v[3];
    return (int64_t)rint(ldexp(p, s));
}

static int count_4pcf_impl(const oracle_graph *g, const int32_t *xyz, int64_t hub_stride,
                           int32_t nthreads, int s4, uint64_t *even, int64_t *odd,
                           uint64_t *cliques_out, const double *w, __int128 *acc_e,
                           __int128 *acc_o, int *scale_out) {
    if (!g || !xyz || !even || !odd || hub_stride < 1) return ORACLE_E_INVALID;
    if (w && (!acc_e || !acc_o || !weights_finite(w, g->n))) return ORACLE_E_INVALID;
    const int nb = g->nb;
    if (nb > ORACLE_MAX_BINS_4PCF) return ORACLE_E_INVALID;
    int64_t ncfg = oracle_num_configs(4, nb);
    int32_t *rank6 = s4 ? make_rank_s4(nb, &ncfg) : make_rank6(nb);
    if (!rank6) return ORACLE_E_NOMEM;
    const int sc = w ? weight_scale4(w, g->n) : 0;
    int nt = set_threads(nthreads);
    memset(even, 0, sizeof(uint64_t) * (size_t)ncfg);
    memset(odd, 0, sizeof(int64_t) * (size_t)ncfg);
    if (w) {
        memset(acc_e, 0, sizeof(__int128) * (size_t)ncfg);
        memset(acc_o, 0, sizeof(__int128) * (size_t)ncfg);
    }
    uint64_t cliques = 0;
    int fail = 0;

    #pragma omp parallel num_threads(nt) reduction(+:cliques) reduction(|:fail)
    {
        uint64_t *my_e = (uint64_t *)calloc((size_t)ncfg, sizeof(uint64_t));
        int64_t *my_o = (int64_t *)calloc((size_t)ncfg, sizeof(int64_t));
        __int128 *my_ae = w ? (__int128 *)calloc((size_t)ncfg, sizeof(__int128)) : NULL;
        __int128 *my_ao = w ? (__int128 *)calloc((size_t)ncfg, sizeof(__int128)) : NULL;
        if (!my_e || !my_o || (w && (!my_ae || !my_ao))) fail = 1;
        #pragma omp for schedule(dynamic, 64)
        for (int64_t i = 0; i < g->n; i++) {
            if (fail || i % hub_stride) continue;
            const int64_t ie = g->row_ptr[i + 1];
            for (int64_t s1 = g->row_ptr[i]; s1 < ie; s1++) {
                const int32_t j1 = g->col[s1];
                if (j1 <= i) continue;
                const int64_t e1 = g->row_ptr[j1 + 1];
                /* k2 walk: hub tail after j1 against N(j1) (§III.1). */
                int64_t a = s1 + 1, b = g->row_ptr[j1];
                while (a < ie && b < e1) {
                    if (g->col[a] < g->col[b]) { a++; continue; }
                    if (g->col[a] > g->col[b]) { b++; continue; }
                    const int32_t j2 = g->col[a];
                    const int64_t e2 = g->row_ptr[j2 + 1];
                    /* Three-pointer walk (§III.1.1, Eq.(2)): alpha on the hub tail beyond j2,
                     * beta on N(j1) just after j2, gamma on N(j2) past j2's own index. */
                    int64_t al = a + 1, be = b + 1, ga = g->row_ptr[j2];
                    while (ga < e2 && g->col[ga] <= j2) ga++;
                    while (al < ie && be < e1 && ga < e2) {
                        const int32_t ha = g->col[al], hb = g->col[be], hc = g->col[ga];
                        if (ha == hb && hb == hc) {
                            int v[6] = {g->bin[s1], g->bin[a], g->bin[al], /* i-j1, i-j2, i-j3 */
                                        g->bin[b], g->bin[be], g->bin[ga]}; /* j1-j2, j1-j3, j2-j3 */
                            if (!s4) sort_small_int(v, 6); /* S4: the table maps every tuple */
                            const int32_t c = rank6[tuple_key(v, nb)];
                            const int32_t vv[4] = {(int32_t)i, j1, j2, ha};
                            const int sg = parity_sign(xyz, vv);
                            my_e[c]++;
                            my_o[c] += sg;
                            if (w) {
                                const double wv[4] = {w[i], w[j1], w[j2], w[ha]};
                                const int64_t q = tetra_q(wv, sc);
                                my_ae[c] += q;
                                my_ao[c] += (__int128)sg * q;
                            }
                            cliques++;
                            al++; be++; ga++;
                        } else {
                            const int32_t mn = ha < hb ? (ha < hc ? ha : hc) : (hb < hc ? hb : hc);
                            if (ha == mn) al++;
                            if (hb == mn) be++;
                            if (hc == mn) ga++;
                        }
                    }
                    a++;
                    b++;
                }
            }
        }
        #pragma omp critical
        {
            if (my_e && my_o)
                for (int64_t c = 0; c < ncfg; c++) {
                    even[c] += my_e[c];
                    odd[c] += my_o[c];
                }
            if (my_ae && my_ao)
                for (int64_t c = 0; c < ncfg; c++) {
                    acc_e[c] += my_ae[c];
                    acc_o[c] += my_ao[c];
                }
        }
        free(my_e);
        free(my_o);
        free(my_ae);
        free(my_ao);
    }
    free(rank6);
    if (fail) return ORACLE_E_NOMEM;
    if (cliques_out) *cliques_out = cliques;
    if (scale_out) *scale_out = sc;
    return 0;
}

int oracle_count_4pcf_parity(const oracle_graph *g, const int32_t *xyz, int64_t hub_stride,
                             int32_t nthreads, uint64_t *even, int64_t *odd,
                             uint64_t *cliques_out) {
    return count_4pcf_impl(g, xyz, hub_stride, nthreads, 0, even, odd, cliques_out, NULL, NULL,
                           NULL, NULL);
}

int oracle_count_4pcf_parity_s4(const oracle_graph *g, const int32_t *xyz, int64_t hub_stride,
                                int32_t nthreads, uint64_t *even, int64_t *odd,
                                uint64_t *cliques_out) {
    return count_4pcf_impl(g, xyz, hub_stride, nthreads, 1, even, odd, cliques_out, NULL, NULL,
                           NULL, NULL);
}

int oracle_count_4pcf_weighted(const oracle_graph *g, const int32_t *xyz, const double *w,
                               int32_t s4, int32_t nthreads, uint64_t *even, int64_t *odd,
                               double *even_w, double *odd_w, int32_t *scale_out) {
    if (!g || !w || !even_w || !odd_w) return ORACLE_E_INVALID;
    const int64_t ncfg = s4 ? oracle_num_configs_s4(g->nb) : oracle_num_configs(4, g->nb);
    if (ncfg <= 0) return ORACLE_E_INVALID;
    __int128 *ae = (__int128 *)malloc(sizeof(__int128) * (size_t)ncfg);
    __int128 *ao = (__int128 *)malloc(sizeof(__int128) * (size_t)ncfg);
    int sc = 0, rc = ORACLE_E_NOMEM;
    if (ae && ao)
        rc = count_4pcf_impl(g, xyz, 1, nthreads, s4 ? 1 : 0, even, odd, NULL, w, ae, ao, &sc);
    if (!rc)
        for (int64_t c = 0; c < ncfg; c++) { /* one rounding of each exact sum */
            even_w[c] = ldexp((double)ae[c], -sc);
            odd_w[c] = ldexp((double)ao[c], -sc);
        }
    if (!rc && scale_out) *scale_out = sc;
    free(ae);
    free(ao);
    return rc;
}

/* oracle.h - plain CPU reference for the graph-based 3-point / 4-point correlation counts.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the CPU-baseline leg of
 * the benchmark load this library.  The product library (libgtc) never includes, links or calls it,
 * and this code includes nothing from the product library.
 *
 * What it computes follows GRAMSCI v2, "Fast Graph-based Higher-Order Clustering Statistics on the
 * GPU" (arXiv 2607.06604):
 *   - the neighbour graph of §II.1, Eq.(1): for each point, every other point within r_max, as a
 *     list sorted by point index, with a radial-bin byte per edge;
 *   - the hub-and-spoke triangle enumeration of §II.2 with the two-pointer merge-walk of §III.1;
 *   - the tetrahedron (4-clique) enumeration of §II.2 with the three-pointer walk of §III.1.1,
 *     Eq.(2);
 *   - the parity split of §III.2: the sign of the signed volume Eq.(3), zero for degenerate
 *     tetrahedra;
 *   - configurations as sorted side-length bins in lexicographic order (§V.1, Fig. 8 key).
 *
 * Readings where the pages leave a step open (each also listed with its reason in the design notes):
 *   - neighbours: distinct points i != j with e_0 <= d^2 < e_nb (half-open, like every bin);
 *     d^2 is the exact integer squared distance of integer grid coordinates.
 *   - bin(i,j) = the b with e_b <= d^2 < e_{b+1}.
 *   - every triangle / tetrahedron is counted once (vertex labels i < j < k, i < j1 < j2 < j3).
 *   - a 3pCF configuration is the nondecreasing triple of its three edge bins; a 4pCF
 *     configuration is the nondecreasing 6-tuple of its six edge bins.  Ranks number these tuples
 *     in nested-loop (lexicographic) order starting at 0.
 *   - weighted 3pCF: per triangle p = fl(fl(w1*w2)*w3) with w1 <= w2 <= w3 (fp64, no fused
 *     multiply-add).  Each p is scaled to q = rint(p * 2^s), the q are summed exactly and the sum is
 *     rounded once to fp64 and scaled back by 2^-s.  s = 57 - e where M = fl(fl(a*a)*a) for
 *     a = max|w| over all weights and M = f * 2^e with f in [0.5, 1) (s = 0 if M == 0); then
 *     |q| < 2^57, and q is exact whenever p's last bit is >= 2^-s (always so for w in [0.5, 1.5)).
 *   - parity orientation: the four vertices are ordered by key(v) = sum over the other three of
 *     d^2(u, v), ascending; with v0..v3 in that order, V = det[x1-x0; x2-x0; x3-x0] (rows), which
 *     is (r01 x r02) . r03 of Eq.(3).  The odd channel gets +1 if V > 0, -1 if V < 0, and 0 if
 *     V == 0 or any two keys are equal (no label-free chirality).
 *
 * Conventions: coordinates are int32 [n][3] in [0, 2^20); edges are int64 [nb+1], strictly
 * increasing with e_0 >= 0.  All functions return 0 on success and a negative code on bad input.
 */
#ifndef GTC_ORACLE_H
#define GTC_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_MAX_BINS 255
#define ORACLE_MAX_BINS_4PCF 16
#define ORACLE_E_INVALID (-1)
#define ORACLE_E_NOMEM (-2)

typedef struct oracle_graph_s oracle_graph;

/* Neighbour graph in the caller's labels: full symmetric adjacency, rows sorted ascending. */
int oracle_build_graph(int64_t n, const int32_t *xyz, int32_t nbins, const int64_t *edges_sq,
                       int32_t nthreads, oracle_graph **out);
/* The same graph with each row cut to the neighbours above its own label (j > i): half the
 * memory.  The 3pCF, 4pCF and 2pCF counts below read only such entries, so they give the same
 * results on it; an export returns the forward rows. */
int oracle_build_graph_forward(int64_t n, const int32_t *xyz, int32_t nbins,
                               const int64_t *edges_sq, int32_t nthreads, oracle_graph **out);
void oracle_graph_free(oracle_graph *g);
int64_t oracle_graph_n(const oracle_graph *g);
int64_t oracle_graph_nnz(const oracle_graph *g);   /* entries: 2E, or E for a forward graph */
/* Copy out the adjacency: row_ptr [n+1], col [nnz], bin [nnz]. */
int oracle_graph_export(const oracle_graph *g, int64_t *row_ptr, int32_t *col, uint8_t *bin);

/* Number of configurations: C(nb+2, 3) for order 3, C(nb+5, 6) for order 4. */
int64_t oracle_num_configs(int32_t order, int32_t nbins);

/* 3pCF.  counts [n_cfg] (overwritten).  If w != NULL, weighted [n_cfg] receives the weighted sums
 * and *scale_out the exponent s.  Only hubs i (smallest label of the triangle) with
 * i % hub_stride == 0 are enumerated (hub_stride = 1: all).  *walks_out (may be NULL) receives the
 * number of hub-spoke merge-walks done (spokes j > i of enumerated hubs). */
int oracle_count_3pcf(const oracle_graph *g, const double *w, int64_t hub_stride,
                      int32_t nthreads, uint64_t *counts, double *weighted, int32_t *scale_out,
                      uint64_t *walks_out);

/* As oracle_count_3pcf for the hubs i with i % hub_stride == hub_offset (0 <= hub_offset <
 * hub_stride).  The counts of the hub_stride offsets add up to those of all hubs (weighted
 * sums are rounded per call, so only the exact sums add up). */
int oracle_count_3pcf_part(const oracle_graph *g, const double *w, int64_t hub_stride,
                           int64_t hub_offset, int32_t nthreads, uint64_t *counts,
                           double *weighted, int32_t *scale_out, uint64_t *walks_out);

/* The same weighted sums before the final rounding: exact sum of q per configuration as
 * two's-complement 128-bit integers, little-endian (lo word first), [n_cfg][2]. */
int oracle_count_3pcf_exact(const oracle_graph *g, const double *w, int64_t hub_stride,
                            int32_t nthreads, uint64_t *counts, int64_t *sum_q128,
                            int32_t *scale_out);

/* 3pCF of the triangles whose smallest label is one of hubs[0..nh) (distinct labels in [0, n)),
 * straight from the coordinates with no graph: for each hub h, the points j > h within the bin
 * range, and every pair of them within the bin range of each other.  counts / weighted as in
 * oracle_count_3pcf, with the scale s from max|w| over all n weights, so that the sums of any set
 * of hubs add up to the sums of all hubs.  O(nh * (n + m^2)) for m forward neighbours per hub. */
int oracle_count_3pcf_hubs(int64_t n, const int32_t *xyz, int32_t nbins, const int64_t *edges_sq,
                           const double *w, const int32_t *hubs, int64_t nh, int32_t nthreads,
                           uint64_t *counts, double *weighted, int32_t *scale_out);

/* Parity 4pCF (nbins <= ORACLE_MAX_BINS_4PCF).  even, odd [n_cfg] (overwritten). */
int oracle_count_4pcf_parity(const oracle_graph *g, const int32_t *xyz, int64_t hub_stride,
                             int32_t nthreads, uint64_t *even, int64_t *odd,
                             uint64_t *cliques_out);

/* S4 configurations of the 4pCF: a tetrahedron's six edge bins in the edge order (01, 02, 03, 12,
 * 13, 23) of its vertices, up to the 24 relabellings of the vertices (the configuration of
 * Eq. (4)); the canonical tuple is the lexicographically smallest relabelling, and configurations
 * are numbered by their canonical tuples in lexicographic order.  nbins <= ORACLE_MAX_BINS_4PCF.
 *   oracle_num_configs_s4: the number of configurations (0 for bad nbins).
 *   oracle_config_bins_s4: the canonical tuples, bins [n_cfg][6].
 *   oracle_config_realizable_s4: mask [n_cfg], 1 where the configuration's bin centres (the
 *     midpoint in r of [sqrt(e_b), sqrt(e_b+1))) are the edge lengths of a tetrahedron of positive
 *     volume: a positive Cayley-Menger determinant, every face a proper triangle (§V.2).
 *   oracle_count_4pcf_parity_s4: as oracle_count_4pcf_parity, binned by S4 configuration. */
int64_t oracle_num_configs_s4(int32_t nbins);
int oracle_config_bins_s4(int32_t nbins, int32_t *bins);
int oracle_config_realizable_s4(int32_t nbins, const int64_t *edges_sq, uint8_t *mask);
int oracle_count_4pcf_parity_s4(const oracle_graph *g, const int32_t *xyz, int64_t hub_stride,
                                int32_t nthreads, uint64_t *even, int64_t *odd,
                                uint64_t *cliques_out);

/* Weighted parity 4pCF: as oracle_count_4pcf_parity (s4 = 0) or _s4 (s4 != 0), all hubs, and in
 * addition even_w / odd_w [n_cfg]: the sums over tetrahedra of p = fl(fl(fl(w1*w2)*w3)*w4), the
 * four weights ascending (no fused multiply-add), and of sign(V) * p.  Each p is scaled to
 * q = rint(p * 2^s), the q are summed exactly and each sum is rounded once; s = 57 - e for
 * M = fl(fl(fl(a*a)*a)*a) = f * 2^e, a = max|w|. */
int oracle_count_4pcf_weighted(const oracle_graph *g, const int32_t *xyz, const double *w,
                               int32_t s4, int32_t nthreads, uint64_t *even, int64_t *odd,
                               double *even_w, double *odd_w, int32_t *scale_out);

/* 2pCF: pairs of the graph per bin, each once: counts [nbins]; with w, weighted [nbins] receives
 * the sums of w_i w_j, each product p = fl(w_i * w_j) scaled to q = rint(p * 2^s), summed exactly
 * and rounded once (s = 57 - e for M = fl(a * a) = f * 2^e, f in [0.5, 1), a = max|w|; s = 0 if
 * M == 0); *scale_out (may be NULL) receives s.  With data weights summing to +1 and random weights
 * to -1 the weighted sums are the Landy-Szalay numerator DD - 2DR + RR (§II.1). */
int oracle_count_2pcf(const oracle_graph *g, const double *w, uint64_t *counts, double *weighted,
                      int32_t *scale_out);

/* Disconnected 4pCF, Eq. (4), per S4 configuration from the binned 2pCF xi [nbins]:
 * disc[c] = xi(b01) xi(b23) + xi(b02) xi(b13) + xi(b03) xi(b12) of the canonical tuple. */
int oracle_disconnected_4pcf_s4(int32_t nbins, const double *xi, double *disc);

/* Number of forward neighbours of each point (neighbours with a larger label). */
int oracle_forward_degrees(const oracle_graph *g, int32_t *deg_out);

#ifdef __cplusplus
}
#endif
#endif

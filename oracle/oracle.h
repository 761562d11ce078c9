/*
 * Brute-force DBSCAN oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * This is the plain, slow CPU reference that the GPU library is checked
 * against.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it; the library never calls it and has no fallback to
 * it.  It shares no code, header, constant or helper with the GPU path.
 *
 * What it computes follows the definitions in Wang et al., "Design and
 * optimization of DBSCAN Algorithm based on CUDA", Sec. II (epsilon-
 * neighbourhood, core point, reachability, cluster) and the serial
 * three-step outline there (neighbourhoods, core points with their
 * neighbourhoods, merge of reachable cores), with the distance compared
 * against eps^2 as in Sec. IV-A.  Readings where the paper is silent:
 *   - a point is in its own neighbourhood (distance 0);
 *   - core iff |N(i)| >= min_pts; neighbour iff d2 <= eps2 (inclusive);
 *   - d2 is the fp32 sum over k ascending of fl(fl(x_k - y_k)^2), every
 *     operation rounded separately (no fused multiply-add), gradual
 *     underflow kept; eps2 = fl32(eps * eps);
 *   - clusters are the connected components of the graph on core points
 *     with an edge between cores within eps (merge only through cores);
 *   - a non-core point with a core neighbour joins the cluster of its
 *     lowest-index core neighbour; all other points are noise (-1);
 *   - a cluster's label is the smallest point index among its members
 *     (cores and the border points assigned to it).
 *
 * Parity status: every entry point below is pinned by CPU tests against
 * hand-worked cases, exact rational arithmetic, an independent BFS
 * DBSCAN, scipy/scikit-learn routines and invariants.
 */
#ifndef ORACLE_DBSCAN_H
#define ORACLE_DBSCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORACLE_OK = 0,
  ORACLE_BAD_ARG = -1,     /* n<0, d<1, eps NaN/inf/negative, min_pts<1, NULL with n>0 */
  ORACLE_NONFINITE = -2,   /* a coordinate is NaN or +-inf */
  ORACLE_NO_MEMORY = -4,
  ORACLE_FTZ_SET = -7      /* host FPU flushes denormals: results would differ */
};

/* Which distance decides "within eps":
 *   ORACLE_FORM_DIRECT    sum_k fl(fl(x_k - y_k)^2), k ascending (above);
 *   ORACLE_FORM_EXPANDED  the hoisted-norm form of Wang et al. Sec. IV-B2,
 *     dist = T + P - sum_k (2 x_k) y_k with T = |x|^2, P = |y|^2 (each a
 *     sum of rounded squares, k ascending), the products summed in k
 *     order, then T + P, then the subtraction, every step rounded.  It
 *     rounds differently from the direct form (and can even be negative),
 *     so near the radius its decisions may differ. */
enum { ORACLE_FORM_DIRECT = 0, ORACLE_FORM_EXPANDED = 1 };

/* fp32 squared distance, k ascending, each operation rounded. */
float oracle_d2(const float* a, const float* b, int32_t d);

/* fp32 squared norm (squares and sum rounded, k ascending) and the
 * hoisted-norm distance (from given norms, or computing them). */
float oracle_sq_norm(const float* a, int32_t d);
float oracle_d2_expanded_from_norms(const float* a, const float* b, int32_t d,
                                    float ta, float pb);
float oracle_d2_expanded(const float* a, const float* b, int32_t d);

/* fl32(eps * eps). */
float oracle_eps2(float eps);

/* Full fit. points: n*d floats row-major.  labels: n int32 (written).
 * counts: n int32 or NULL.  n_threads <= 0 uses the OpenMP default.
 * Returns ORACLE_OK or a negative status; outputs unspecified on error. */
int oracle_fit(const float* points, int64_t n, int32_t d, float eps,
               int32_t min_pts, int32_t* labels, int32_t* counts,
               int32_t n_threads);

/* The same fit with the neighbour test of the given form. */
int oracle_fit_form(const float* points, int64_t n, int32_t d, float eps,
                    int32_t min_pts, int32_t* labels, int32_t* counts,
                    int32_t n_threads, int32_t form);

/* Neighbour counts of the listed rows only (for sampled checks on large
 * sets): counts_out[r] = |N(rows[r])| over all n points. */
int oracle_row_counts(const float* points, int64_t n, int32_t d, float eps,
                      const int64_t* rows, int64_t n_rows, int32_t* counts_out,
                      int32_t n_threads);
int oracle_row_counts_form(const float* points, int64_t n, int32_t d,
                           float eps, const int64_t* rows, int64_t n_rows,
                           int32_t* counts_out, int32_t n_threads,
                           int32_t form);

/* Indices j (ascending) with d2(i, j) <= eps2, at most cap of them written;
 * returns the full neighbour count, or a negative status. */
int64_t oracle_row_neighbours(const float* points, int64_t n, int32_t d,
                              float eps, int64_t i, int64_t* out, int64_t cap);
int64_t oracle_row_neighbours_form(const float* points, int64_t n, int32_t d,
                                   float eps, int64_t i, int64_t* out,
                                   int64_t cap, int32_t form);

/* Contiguous cluster ids: clusters are numbered 0..K-1 in ascending order
 * of their label (their smallest member); noise stays -1.  out: n int32.
 * sizes: n int32 or NULL, sizes[k] = members of cluster k (entries >= K
 * untouched).  Returns K, or a negative status. */
int64_t oracle_relabel(const int32_t* labels, int64_t n, int32_t* out,
                       int32_t* sizes);

/* Sparse epsilon-graph in CSR form: row i holds every j with
 * d2(i, j) <= eps2, itself included, in ascending j.  row_ptr: n+1 int64
 * (written).  *col_idx_out receives a malloc'd int32 array of row_ptr[n]
 * entries (release it with oracle_free); NULL on error.  Returns the
 * number of entries, or a negative status. */
int64_t oracle_graph(const float* points, int64_t n, int32_t d, float eps,
                     int64_t* row_ptr, int32_t** col_idx_out,
                     int32_t n_threads);
int64_t oracle_graph_form(const float* points, int64_t n, int32_t d, float eps,
                          int64_t* row_ptr, int32_t** col_idx_out,
                          int32_t n_threads, int32_t form);
void oracle_free(void* ptr);

/* Wall time of the last oracle_fit on this thread, seconds (steady clock,
 * fit body only). */
double oracle_last_fit_seconds(void);

#ifdef __cplusplus
}
#endif
#endif

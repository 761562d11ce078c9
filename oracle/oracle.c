/*
 * Brute-force DBSCAN oracle -- TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * Plain C11 + OpenMP.  Build without -ffast-math and with
 * -ffp-contract=off so that every subtraction, square and addition of the
 * distance is rounded on its own, in the order written.
 *
 * The fit follows the serial outline of Wang et al., "Design and
 * optimization of DBSCAN Algorithm based on CUDA", Sec. II: first the
 * epsilon-neighbourhood of every point (compared against eps^2, Sec. IV-A),
 * then the core points (at least MinPts points within eps, Sec. II item 2),
 * then the merge of core points reachable from one another (Sec. II item 3
 * and the cluster definition), without ever storing the N x N matrix.
 */
#define _POSIX_C_SOURCE 199309L
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>
#include <xmmintrin.h>

static _Thread_local double g_last_fit_seconds = 0.0;

double oracle_last_fit_seconds(void) { return g_last_fit_seconds; }

static double now_seconds(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

/* MXCSR bit 15 = flush-to-zero, bit 6 = denormals-are-zero. */
static int host_flushes_denormals(void) {
  return (_mm_getcsr() & 0x8040u) != 0u;
}

static int thread_count(int32_t n_threads) {
  return n_threads > 0 ? (int)n_threads : omp_get_max_threads();
}

float oracle_eps2(float eps) {
  float e2 = eps * eps;
  return e2;
}

/* Squared Euclidean distance in fp32, dimensions in ascending order. */
float oracle_d2(const float* a, const float* b, int32_t d) {
  float s = 0.0f;
  for (int32_t k = 0; k < d; ++k) {
    float t = a[k] - b[k];
    float q = t * t;
    s = s + q;
  }
  return s;
}

/* Squared norm in fp32: squares and their sum rounded, k ascending. */
float oracle_sq_norm(const float* a, int32_t d) {
  float s = a[0] * a[0];
  for (int32_t k = 1; k < d; ++k) {
    float q = a[k] * a[k];
    s = s + q;
  }
  return s;
}

/* The hoisted-norm form of Wang et al. Sec. IV-B2: with T = |a|^2 and
 * P = |b|^2 computed once per point, and the doubled coordinates 2 a_k
 * (exact), dist = T + P - (2a_0 b_0 + 2a_1 b_1 + ...).  Every product and
 * every sum is rounded on its own, the products summed in k order, then
 * (T + P) and finally the subtraction. */
float oracle_d2_expanded_from_norms(const float* a, const float* b, int32_t d,
                                    float ta, float pb) {
  float inner = (2.0f * a[0]) * b[0];
  for (int32_t k = 1; k < d; ++k) {
    float q = (2.0f * a[k]) * b[k];
    inner = inner + q;
  }
  float s = ta + pb;
  return s - inner;
}

float oracle_d2_expanded(const float* a, const float* b, int32_t d) {
  return oracle_d2_expanded_from_norms(a, b, d, oracle_sq_norm(a, d),
                                       oracle_sq_norm(b, d));
}

/* Neighbour test of points i and j under the chosen form; `norms` holds
 * every point's oracle_sq_norm for the hoisted-norm form. */
static int within(int32_t form, const float* p, int32_t d, const float* norms,
                  int64_t i, int64_t j, float eps2) {
  const float* a = p + i * (int64_t)d;
  const float* b = p + j * (int64_t)d;
  if (form == ORACLE_FORM_EXPANDED)
    return oracle_d2_expanded_from_norms(a, b, d, norms[i], norms[j]) <= eps2;
  return oracle_d2(a, b, d) <= eps2;
}

/* The per-point norms the hoisted-norm form needs (NULL otherwise, or on
 * allocation failure with *oom set). */
static float* form_norms(int32_t form, const float* p, int64_t n, int32_t d,
                         int nt, int* oom) {
  *oom = 0;
  if (form != ORACLE_FORM_EXPANDED || n == 0) return NULL;
  float* norms = (float*)malloc((size_t)n * sizeof(float));
  if (!norms) {
    *oom = 1;
    return NULL;
  }
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int64_t i = 0; i < n; ++i) norms[i] = oracle_sq_norm(p + i * (int64_t)d, d);
  return norms;
}

static int check_form(int32_t form) {
  return (form == ORACLE_FORM_DIRECT || form == ORACLE_FORM_EXPANDED) ? ORACLE_OK
                                                                       : ORACLE_BAD_ARG;
}

static int check_args(const float* p, int64_t n, int32_t d, float eps,
                      int32_t min_pts) {
  if (n < 0 || n > (int64_t)INT32_MAX || d < 1 || min_pts < 1) return ORACLE_BAD_ARG;
  if (!(eps >= 0.0f) || isinf(eps)) return ORACLE_BAD_ARG;
  if (n > 0 && p == NULL) return ORACLE_BAD_ARG;
  return ORACLE_OK;
}

static int check_finite(const float* p, int64_t n, int32_t d) {
  const int64_t total = n * (int64_t)d;
  for (int64_t k = 0; k < total; ++k)
    if (!isfinite(p[k])) return ORACLE_NONFINITE;
  return ORACLE_OK;
}

/* ---- union-find (serial) ---------------------------------------------- */

static int32_t uf_find(int32_t* parent, int32_t x) {
  while (parent[x] != x) {
    parent[x] = parent[parent[x]]; /* path halving */
    x = parent[x];
  }
  return x;
}

/* The larger root is hung under the smaller one. */
static void uf_union(int32_t* parent, int32_t a, int32_t b) {
  int32_t ra = uf_find(parent, a);
  int32_t rb = uf_find(parent, b);
  if (ra == rb) return;
  if (ra < rb) parent[rb] = ra;
  else parent[ra] = rb;
}

typedef struct {
  int32_t* ij; /* pairs, 2 ints each */
  int64_t len, cap;
} edge_buf;

static int edge_push(edge_buf* e, int32_t i, int32_t j) {
  if (e->len == e->cap) {
    int64_t nc = e->cap ? 2 * e->cap : 1024;
    int32_t* q = (int32_t*)realloc(e->ij, (size_t)nc * 2 * sizeof(int32_t));
    if (!q) return ORACLE_NO_MEMORY;
    e->ij = q;
    e->cap = nc;
  }
  e->ij[2 * e->len] = i;
  e->ij[2 * e->len + 1] = j;
  e->len++;
  return ORACLE_OK;
}

int oracle_fit(const float* p, int64_t n, int32_t d, float eps,
               int32_t min_pts, int32_t* labels, int32_t* counts_out,
               int32_t n_threads) {
  return oracle_fit_form(p, n, d, eps, min_pts, labels, counts_out, n_threads,
                         ORACLE_FORM_DIRECT);
}

int oracle_fit_form(const float* p, int64_t n, int32_t d, float eps,
                    int32_t min_pts, int32_t* labels, int32_t* counts_out,
                    int32_t n_threads, int32_t form) {
  int st = check_args(p, n, d, eps, min_pts);
  if (st == ORACLE_OK) st = check_form(form);
  if (st != ORACLE_OK) return st;
  if (n > 0 && labels == NULL) return ORACLE_BAD_ARG;
  if (host_flushes_denormals()) return ORACLE_FTZ_SET;
  st = check_finite(p, n, d);
  if (st != ORACLE_OK) return st;
  if (n == 0) {
    g_last_fit_seconds = 0.0;
    return ORACLE_OK;
  }
  const int nt = thread_count(n_threads);
  const double t0 = now_seconds();
  const float eps2 = oracle_eps2(eps);

  int32_t* count = (int32_t*)malloc((size_t)n * sizeof(int32_t));
  uint8_t* core = (uint8_t*)malloc((size_t)n);
  int32_t* parent = (int32_t*)malloc((size_t)n * sizeof(int32_t));
  int32_t* bmin = (int32_t*)malloc((size_t)n * sizeof(int32_t));
  int32_t* first = (int32_t*)malloc((size_t)n * sizeof(int32_t));
  int norms_oom = 0;
  float* norms = form_norms(form, p, n, d, nt, &norms_oom);
  if (!count || !core || !parent || !bmin || !first || norms_oom) {
    free(count); free(core); free(parent); free(bmin); free(first); free(norms);
    return ORACLE_NO_MEMORY;
  }

  /* 1. neighbour count of every point, itself included. */
#pragma omp parallel for schedule(dynamic, 64) num_threads(nt)
  for (int64_t i = 0; i < n; ++i) {
    int64_t c = 0;
    for (int64_t j = 0; j < n; ++j)
      if (within(form, p, d, norms, i, j, eps2)) ++c;
    count[i] = (int32_t)c;
  }

  /* 2. core points. */
  for (int64_t i = 0; i < n; ++i) {
    core[i] = (uint8_t)(count[i] >= min_pts);
    parent[i] = (int32_t)i;
    bmin[i] = -1;
    first[i] = -1;
  }

  /* 3. merge: union every pair of cores within eps.  Pairs (i, j>i) are
   *    found in parallel one block of rows at a time, then united serially. */
  const int64_t block = 4096;
  int oom = 0;
  for (int64_t b0 = 0; b0 < n && !oom; b0 += block) {
    const int64_t b1 = (b0 + block < n) ? b0 + block : n;
    edge_buf* bufs = (edge_buf*)calloc((size_t)nt, sizeof(edge_buf));
    if (!bufs) { oom = 1; break; }
#pragma omp parallel num_threads(nt)
    {
      edge_buf* mine = &bufs[omp_get_thread_num()];
#pragma omp for schedule(dynamic, 8)
      for (int64_t i = b0; i < b1; ++i) {
        if (!core[i]) continue;
        for (int64_t j = i + 1; j < n; ++j) {
          if (!core[j]) continue;
          if (within(form, p, d, norms, i, j, eps2))
            if (edge_push(mine, (int32_t)i, (int32_t)j) != ORACLE_OK) {
#pragma omp atomic write
              oom = 1;
            }
        }
      }
    }
    for (int t = 0; t < nt; ++t) {
      for (int64_t e = 0; e < bufs[t].len; ++e)
        uf_union(parent, bufs[t].ij[2 * e], bufs[t].ij[2 * e + 1]);
      free(bufs[t].ij);
    }
    free(bufs);
  }
  if (oom) {
    free(count); free(core); free(parent); free(bmin); free(first); free(norms);
    return ORACLE_NO_MEMORY;
  }

  /* 4. border points: the lowest-index core neighbour, scanning cores in
   *    ascending index and stopping at the first one within eps. */
#pragma omp parallel for schedule(dynamic, 64) num_threads(nt)
  for (int64_t i = 0; i < n; ++i) {
    if (core[i]) continue;
    for (int64_t c = 0; c < n; ++c) {
      if (core[c] && within(form, p, d, norms, i, c, eps2)) {
        bmin[i] = (int32_t)c;
        break;
      }
    }
  }

  /* 5. labels: visiting points in ascending index, the first member seen
   *    of each cluster is its smallest index, which becomes the label. */
  for (int64_t i = 0; i < n; ++i) {
    int32_t r;
    if (core[i]) r = uf_find(parent, (int32_t)i);
    else if (bmin[i] >= 0) r = uf_find(parent, bmin[i]);
    else { labels[i] = -1; continue; }
    if (first[r] < 0) first[r] = (int32_t)i;
    labels[i] = first[r];
  }

  if (counts_out) memcpy(counts_out, count, (size_t)n * sizeof(int32_t));
  g_last_fit_seconds = now_seconds() - t0;
  free(count); free(core); free(parent); free(bmin); free(first); free(norms);
  return ORACLE_OK;
}

int oracle_row_counts(const float* p, int64_t n, int32_t d, float eps,
                      const int64_t* rows, int64_t n_rows, int32_t* out,
                      int32_t n_threads) {
  return oracle_row_counts_form(p, n, d, eps, rows, n_rows, out, n_threads,
                                ORACLE_FORM_DIRECT);
}

int oracle_row_counts_form(const float* p, int64_t n, int32_t d, float eps,
                           const int64_t* rows, int64_t n_rows, int32_t* out,
                           int32_t n_threads, int32_t form) {
  int st = check_args(p, n, d, eps, 1);
  if (st == ORACLE_OK) st = check_form(form);
  if (st != ORACLE_OK) return st;
  if (n_rows < 0 || (n_rows > 0 && (rows == NULL || out == NULL))) return ORACLE_BAD_ARG;
  if (host_flushes_denormals()) return ORACLE_FTZ_SET;
  st = check_finite(p, n, d);
  if (st != ORACLE_OK) return st;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= n) return ORACLE_BAD_ARG;
  const float eps2 = oracle_eps2(eps);
  const int nt = thread_count(n_threads);
  int oom = 0;
  float* norms = form_norms(form, p, n, d, nt, &oom);
  if (oom) return ORACLE_NO_MEMORY;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t c = 0;
    for (int64_t j = 0; j < n; ++j)
      if (within(form, p, d, norms, rows[r], j, eps2)) ++c;
    out[r] = (int32_t)c;
  }
  free(norms);
  return ORACLE_OK;
}

int64_t oracle_row_neighbours(const float* p, int64_t n, int32_t d, float eps,
                              int64_t i, int64_t* out, int64_t cap) {
  return oracle_row_neighbours_form(p, n, d, eps, i, out, cap,
                                    ORACLE_FORM_DIRECT);
}

int64_t oracle_row_neighbours_form(const float* p, int64_t n, int32_t d,
                                   float eps, int64_t i, int64_t* out,
                                   int64_t cap, int32_t form) {
  int st = check_args(p, n, d, eps, 1);
  if (st == ORACLE_OK) st = check_form(form);
  if (st != ORACLE_OK) return st;
  if (i < 0 || i >= n || cap < 0 || (cap > 0 && out == NULL)) return ORACLE_BAD_ARG;
  if (host_flushes_denormals()) return ORACLE_FTZ_SET;
  const float eps2 = oracle_eps2(eps);
  int oom = 0;
  float* norms = form_norms(form, p, n, d, 1, &oom);
  if (oom) return ORACLE_NO_MEMORY;
  int64_t c = 0;
  for (int64_t j = 0; j < n; ++j) {
    if (within(form, p, d, norms, i, j, eps2)) {
      if (c < cap) out[c] = j;
      ++c;
    }
  }
  free(norms);
  return c;
}

/* Number the clusters in ascending order of their label: a point whose
 * label is its own index is the smallest member of its cluster; visiting
 * points in ascending index meets those heads in ascending label order. */
int64_t oracle_relabel(const int32_t* labels, int64_t n, int32_t* out,
                       int32_t* sizes) {
  if (n < 0 || (n > 0 && (labels == NULL || out == NULL))) return ORACLE_BAD_ARG;
  int32_t* id = (int32_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
  if (!id) return ORACLE_NO_MEMORY;
  int64_t k = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t l = labels[i];
    if (l < -1 || l >= n || (l >= 0 && labels[l] != l)) { free(id); return ORACLE_BAD_ARG; }
    if (l == i) id[i] = (int32_t)k++;
  }
  for (int64_t c = 0; sizes && c < k; ++c) sizes[c] = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t l = labels[i];
    out[i] = l < 0 ? -1 : id[l];
    if (l >= 0 && sizes) sizes[id[l]]++;
  }
  free(id);
  return k;
}

/* Sparse epsilon-graph.  Row i lists every j with d2(i, j) <= eps2,
 * itself included, in ascending j: the per-point neighbourhoods that Wang
 * et al. Sec. IV-B keep as rows of their N x N cluster matrix, stored
 * without the zeros.  Each row is found by a plain scan over all points,
 * rows in parallel, each into its own list; the lists are then laid out
 * one after another. */
int64_t oracle_graph(const float* p, int64_t n, int32_t d, float eps,
                     int64_t* row_ptr, int32_t** col_idx_out,
                     int32_t n_threads) {
  return oracle_graph_form(p, n, d, eps, row_ptr, col_idx_out, n_threads,
                           ORACLE_FORM_DIRECT);
}

int64_t oracle_graph_form(const float* p, int64_t n, int32_t d, float eps,
                          int64_t* row_ptr, int32_t** col_idx_out,
                          int32_t n_threads, int32_t form) {
  int st = check_args(p, n, d, eps, 1);
  if (st == ORACLE_OK) st = check_form(form);
  if (st != ORACLE_OK) return st;
  if (row_ptr == NULL || col_idx_out == NULL) return ORACLE_BAD_ARG;
  *col_idx_out = NULL;
  if (host_flushes_denormals()) return ORACLE_FTZ_SET;
  st = check_finite(p, n, d);
  if (st != ORACLE_OK) return st;
  row_ptr[0] = 0;
  if (n == 0) return 0;
  const float eps2 = oracle_eps2(eps);
  const int nt = thread_count(n_threads);
  int norms_oom = 0;
  float* norms = form_norms(form, p, n, d, nt, &norms_oom);
  int32_t** rows = (int32_t**)calloc((size_t)n, sizeof(int32_t*));
  int64_t* len = (int64_t*)calloc((size_t)n, sizeof(int64_t));
  int oom = (rows == NULL || len == NULL || norms_oom);
  if (!oom) {
#pragma omp parallel num_threads(nt)
    {
      int32_t* tmp = (int32_t*)malloc((size_t)n * sizeof(int32_t));
      if (tmp == NULL) {
#pragma omp atomic write
        oom = 1;
      }
#pragma omp for schedule(dynamic, 64)
      for (int64_t i = 0; i < n; ++i) {
        if (tmp == NULL) continue;
        int64_t c = 0;
        for (int64_t j = 0; j < n; ++j)
          if (within(form, p, d, norms, i, j, eps2)) tmp[c++] = (int32_t)j;
        rows[i] = (int32_t*)malloc((size_t)c * sizeof(int32_t));
        if (rows[i] == NULL) {
#pragma omp atomic write
          oom = 1;
          continue;
        }
        memcpy(rows[i], tmp, (size_t)c * sizeof(int32_t));
        len[i] = c;
      }
      free(tmp);
    }
  }
  int32_t* col = NULL;
  if (!oom) {
    for (int64_t i = 0; i < n; ++i) row_ptr[i + 1] = row_ptr[i] + len[i];
    col = (int32_t*)malloc((size_t)row_ptr[n] * sizeof(int32_t));
    if (col == NULL) oom = 1;
  }
  if (!oom)
    for (int64_t i = 0; i < n; ++i)
      memcpy(col + row_ptr[i], rows[i], (size_t)len[i] * sizeof(int32_t));
  for (int64_t i = 0; rows && i < n; ++i) free(rows[i]);
  free(rows);
  free(len);
  free(norms);
  if (oom) {
    free(col);
    return ORACLE_NO_MEMORY;
  }
  *col_idx_out = col;
  return row_ptr[n];
}

void oracle_free(void* ptr) { free(ptr); }

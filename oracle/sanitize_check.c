/*
 * Case runner for a sanitizer build of the oracle -- TEST INFRASTRUCTURE
 * ONLY.  tests/test_oracle_sanitized.py compiles this file together with
 * oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer (gcc, CPU
 * only), runs it on a file of cases and compares what it writes with the
 * regular oracle build.  It adds no arithmetic of its own: every value it
 * writes comes from an oracle entry point.
 *
 *   sanitize_check <cases.bin> <results.bin>
 *
 * cases.bin is a sequence of records, little-endian:
 *   int32 op, int32 form, int64 n, int32 d, float eps, int32 min_pts,
 *   int32 reserved, then n*d float32 points (row-major).
 * For each record results.bin receives, by op:
 *   1 fit:        int64 status; if 0: n int32 labels, n int32 counts,
 *                 int64 K, n int32 contiguous ids, K int32 sizes
 *   2 graph:      int64 nnz (or a negative status); if >= 0: n+1 int64
 *                 row offsets, nnz int32 columns
 *   3 row counts: int64 status; if 0: n int32 counts (rows 0..n-1)
 *   4 neighbours: for i = 0 .. min(n, 8)-1: int64 count (or status),
 *                 then min(count, 4) int64 indices (a buffer of 4: the
 *                 truncating path)
 *   5 distances:  int32 bits of oracle_eps2(eps); for i = 1 .. n-1: int32
 *                 bits of d2(p0, pi) and of the hoisted-norm d2(p0, pi)
 * Exit status 0 when every record was read; sanitizer reports abort.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static int put(FILE* f, const void* p, size_t bytes) {
  return bytes == 0 || fwrite(p, 1, bytes, f) == bytes;
}

static void put_i64(FILE* f, int64_t v) { put(f, &v, sizeof v); }

static void* alloc_or_die(size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(3);
  }
  return p;
}

static void run_fit(FILE* out, const float* pts, int64_t n, int32_t d,
                    float eps, int32_t m, int32_t form) {
  int32_t* labels = alloc_or_die((size_t)n * sizeof(int32_t));
  int32_t* counts = alloc_or_die((size_t)n * sizeof(int32_t));
  const int st = oracle_fit_form(pts, n, d, eps, m, labels, counts, 2, form);
  put_i64(out, st);
  if (st == ORACLE_OK) {
    put(out, labels, (size_t)n * sizeof(int32_t));
    put(out, counts, (size_t)n * sizeof(int32_t));
    int32_t* ids = alloc_or_die((size_t)n * sizeof(int32_t));
    int32_t* sizes = alloc_or_die((size_t)n * sizeof(int32_t));
    const int64_t k = oracle_relabel(labels, n, ids, sizes);
    put_i64(out, k);
    if (k >= 0) {
      put(out, ids, (size_t)n * sizeof(int32_t));
      put(out, sizes, (size_t)k * sizeof(int32_t));
    }
    free(ids);
    free(sizes);
  }
  free(labels);
  free(counts);
}

static void run_graph(FILE* out, const float* pts, int64_t n, int32_t d,
                      float eps, int32_t form) {
  int64_t* row_ptr = alloc_or_die((size_t)(n + 1) * sizeof(int64_t));
  int32_t* col = NULL;
  const int64_t nnz = oracle_graph_form(pts, n, d, eps, row_ptr, &col, 2, form);
  put_i64(out, nnz);
  if (nnz >= 0) {
    put(out, row_ptr, (size_t)(n + 1) * sizeof(int64_t));
    put(out, col, (size_t)nnz * sizeof(int32_t));
  }
  oracle_free(col);
  free(row_ptr);
}

static void run_rows(FILE* out, const float* pts, int64_t n, int32_t d,
                     float eps, int32_t form) {
  int64_t* rows = alloc_or_die((size_t)n * sizeof(int64_t));
  int32_t* cnt = alloc_or_die((size_t)n * sizeof(int32_t));
  for (int64_t i = 0; i < n; ++i) rows[i] = i;
  const int st = oracle_row_counts_form(pts, n, d, eps, rows, n, cnt, 2, form);
  put_i64(out, st);
  if (st == ORACLE_OK) put(out, cnt, (size_t)n * sizeof(int32_t));
  free(rows);
  free(cnt);
}

static void run_neighbours(FILE* out, const float* pts, int64_t n, int32_t d,
                           float eps, int32_t form) {
  int64_t buf[4];
  for (int64_t i = 0; i < n && i < 8; ++i) {
    const int64_t c =
        oracle_row_neighbours_form(pts, n, d, eps, i, buf, 4, form);
    put_i64(out, c);
    if (c > 0) put(out, buf, (size_t)(c < 4 ? c : 4) * sizeof(int64_t));
  }
}

static void run_distances(FILE* out, const float* pts, int64_t n, int32_t d,
                          float eps) {
  const float e2 = oracle_eps2(eps);
  put(out, &e2, sizeof e2);
  for (int64_t i = 1; i < n; ++i) {
    const float a = oracle_d2(pts, pts + i * d, d);
    const float b = oracle_d2_expanded(pts, pts + i * d, d);
    put(out, &a, sizeof a);
    put(out, &b, sizeof b);
  }
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s cases.bin results.bin\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  FILE* out = fopen(argv[2], "wb");
  if (!in || !out) {
    fprintf(stderr, "cannot open the case or result file\n");
    return 2;
  }
  for (;;) {
    int32_t op, form, d, m, reserved;
    int64_t n;
    float eps;
    if (fread(&op, sizeof op, 1, in) != 1) break;
    if (fread(&form, sizeof form, 1, in) != 1 || fread(&n, sizeof n, 1, in) != 1 ||
        fread(&d, sizeof d, 1, in) != 1 || fread(&eps, sizeof eps, 1, in) != 1 ||
        fread(&m, sizeof m, 1, in) != 1 ||
        fread(&reserved, sizeof reserved, 1, in) != 1 || n < 0 || d < 1) {
      fprintf(stderr, "truncated or malformed case header\n");
      return 2;
    }
    const size_t count = (size_t)n * (size_t)d;
    float* pts = alloc_or_die(count * sizeof(float));
    if (count && fread(pts, sizeof(float), count, in) != count) {
      fprintf(stderr, "truncated case points\n");
      return 2;
    }
    switch (op) {
      case 1: run_fit(out, pts, n, d, eps, m, form); break;
      case 2: run_graph(out, pts, n, d, eps, form); break;
      case 3: run_rows(out, pts, n, d, eps, form); break;
      case 4: run_neighbours(out, pts, n, d, eps, form); break;
      case 5: run_distances(out, pts, n, d, eps); break;
      default:
        fprintf(stderr, "unknown op %d\n", op);
        return 2;
    }
    free(pts);
  }
  fclose(in);
  return fclose(out) == 0 ? 0 : 2;
}

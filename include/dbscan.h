/*
 * dbscan.h -- exact all-pairs DBSCAN on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  No exception, C++ type or torch type crosses it; every argument
 * is a plain pointer (host or device, as stated) or a size.
 *
 * What a fit computes (Wang et al., "Design and optimization of DBSCAN
 * Algorithm based on CUDA", Sec. II: epsilon-neighbourhood, core point,
 * reachability and the two-part cluster definition; Sec. IV-A: compare the
 * squared distance with eps^2), with these fixed readings:
 *   - d2(i,j) = sum over k = 0..d-1, in that order, of fl(fl(x_ik - x_jk)^2),
 *     each operation an IEEE binary32 round-to-nearest-even step (no fused
 *     multiply-add, subnormals kept); eps2 = fl(eps * eps);
 *   - N(i) = { j : d2(i,j) <= eps2 }, i itself included; count[i] = |N(i)|;
 *   - i is a core point iff count[i] >= min_pts;
 *   - clusters are the connected components of the graph whose vertices are
 *     the core points, with an edge between two cores within eps;
 *   - a non-core point with at least one core neighbour (a border point)
 *     joins the cluster of its lowest-index core neighbour;
 *   - every other point is noise, label -1;
 *   - a cluster's label is the smallest point index among its members
 *     (its cores and the border points it received).
 * The result is unique, so labels and counts are bit-for-bit reproducible
 * whatever the launch order on the GPU.
 *
 * Points are row-major fp32: point i occupies points[i*d .. i*d+d-1].
 * 0 <= n <= 2^31-1, 1 <= d <= DBSCAN_MAX_D, eps finite and >= 0,
 * min_pts >= 1.  n = 0 is a successful no-op.
 */
#ifndef DBSCAN_MI355X_H
#define DBSCAN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DBSCAN_ABI_VERSION 2
#define DBSCAN_MAX_D 64

/* Status codes: 0 on success, negative on failure.  On any failure the
 * contents of labels / counts are unspecified.  Argument errors are
 * reported before any device work is enqueued. */
typedef enum dbscan_status {
  DBSCAN_OK = 0,
  DBSCAN_ERR_INVALID_ARG = -1, /* n<0 or n>2^31-1, d<1 or d>DBSCAN_MAX_D,
                                  eps NaN/inf/negative, min_pts<1, a NULL
                                  pointer where n>0, unknown flag bits */
  DBSCAN_ERR_NONFINITE = -2,   /* a coordinate is NaN or +-inf */
  DBSCAN_ERR_NO_DEVICE = -3,   /* no HIP device, or the current device is
                                  not gfx950 */
  DBSCAN_ERR_OOM = -4,         /* dbscan_fit and dbscan_fit_counts only:
                                  device allocation failed */
  DBSCAN_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than
                                  dbscan_workspace_bytes(n, d), or misaligned */
  DBSCAN_ERR_HIP = -6,         /* any other HIP runtime error */
  DBSCAN_ERR_CAPACITY = -7,    /* dbscan_graph_device only: the caller's
                                  col_idx buffer is smaller than the graph
                                  (the call reports the size needed) */
  DBSCAN_ERR_TOO_LARGE = -8    /* dbscan_fit_device_noalloc only:
                                  dbscan_workspace_bytes(n, d) exceeds
                                  DBSCAN_NOALLOC_SCRATCH_BYTES */
} dbscan_status;

/* Merge strategies a fit may take (reported in dbscan_info.merge_mode). */
#define DBSCAN_MERGE_NONE 0  /* n == 0 */
#define DBSCAN_MERGE_EDGES 1 /* the count pass recorded every neighbour pair
                                (i<j) in the workspace's edge area, and the
                                merge walked that list: no distance is
                                evaluated twice */
#define DBSCAN_MERGE_TILES 2 /* the edge area was absent or too small: the
                                merge re-evaluated distances in a second tile
                                pass over (all points) x (core points) */

/* Flag bits for dbscan_fit_device_ex. */
#define DBSCAN_FLAG_TIME_PHASES 0x1u  /* fill the ms_* fields of dbscan_info
                                         from HIP events on the stream */
#define DBSCAN_FLAG_FORCE_TILE_MERGE 0x2u /* ignore the edge area and take the
                                             tile merge (for testing) */
#define DBSCAN_FLAG_PRUNE_TILES 0x4u /* exact tile pruning: sort the points
                                        along a space-filling curve, bound
                                        each block of the count pass by its
                                        box and skip block pairs whose fp32
                                        box gap already exceeds eps^2 (a
                                        lower bound of every distance
                                        between them, in the same rounded
                                        arithmetic); results are identical,
                                        far fewer distances are evaluated
                                        when d is small */
#define DBSCAN_FLAG_REVERSE_SCHEDULE 0x10u /* for testing: walk the count
                                             pass's work items, the recorded
                                             pairs and the tile merge's
                                             blocks in reverse order; the
                                             results must not change */
#define DBSCAN_FLAG_SHUFFLE_SCHEDULE 0x40u /* for testing: walk them in a
                                             fixed shuffled order instead,
                                             chosen by the seed in bits
                                             16..31 of the flags (allowed
                                             only with this flag; not with
                                             the reverse flag); the results
                                             must not change */
#define DBSCAN_FLAG_SCREEN 0x8u /* decide most pairs of the count pass with
                                   the hoisted-norm form |y|^2 - 2 x.y
                                   (Wang et al. Sec. IV-B2) evaluated with
                                   fused multiply-adds, against per-point
                                   thresholds that bracket the exact
                                   decision by a proven rounding-error
                                   bound; pairs inside the bracket are
                                   decided with the exact distance, so the
                                   results are identical to the exact pass
                                   and about d instead of 3d operations are
                                   spent per pair */
#define DBSCAN_FLAG_EXPANDED 0x20u /* decide "within eps" with the
                                      hoisted-norm distance of Wang et al.
                                      Sec. IV-B2 itself instead of the
                                      direct one: dist = T + P - sum_k
                                      (2 x_k) y_k, T = |x|^2 and P = |y|^2
                                      each summed from rounded squares in
                                      k order, the products summed in k
                                      order, then T + P, then the
                                      subtraction, every step a binary32
                                      operation.  It rounds differently
                                      (the error grows with the norms, and
                                      the value can be negative), so
                                      results near the radius may differ
                                      from the default form.  Implies
                                      DBSCAN_FLAG_SCREEN (the screen then
                                      brackets this form); not combined
                                      with DBSCAN_FLAG_PRUNE_TILES, whose
                                      bound is for the direct form
                                      (DBSCAN_ERR_INVALID_ARG) */

/* What a fit did; filled by dbscan_fit_device_ex when info != NULL. */
typedef struct dbscan_info {
  int64_t n_core;        /* number of core points */
  int64_t n_edges;       /* neighbour pairs i<j found by the count pass (0
                            when no edge area was given) */
  int64_t edge_capacity; /* pairs the edge area can hold */
  int64_t pass1_pairs;   /* ordered pairs (i,j) decided by the count pass,
                            including padding: n_pad^2 */
  int64_t pass2_pairs;   /* distances evaluated by a tile merge (0 for the
                            edge merge) */
  int64_t tiles_total;   /* block pairs (I <= J) of the count pass */
  int64_t tiles_kept;    /* block pairs evaluated: all of them, or those
                            left by DBSCAN_FLAG_PRUNE_TILES */
  int32_t merge_mode;    /* DBSCAN_MERGE_* */
  int32_t timed;         /* 1 if the ms_* fields below were measured */
  float ms_layout;       /* ingest, padding, non-finite check, init */
  float ms_count;        /* neighbour-count pass */
  float ms_core;         /* core flags (+ core compaction for a tile merge) */
  float ms_merge;        /* union-find merge and border assignment */
  float ms_label;        /* root compression and canonical labels */
  float ms_total;        /* first to last kernel of the fit */
  int32_t hip_error;     /* hipError_t of the failing HIP call, 0 if none */
  int32_t reserved;
} dbscan_info;

/* Minimum workspace (bytes) for dbscan_fit_device with n points of
 * dimension d; 0 if n or d is out of range. */
size_t dbscan_workspace_bytes(int64_t n, int32_t d);

/* Workspace (bytes) that also holds an edge area for max_edges neighbour
 * pairs: dbscan_workspace_bytes(n, d) + 8 * max_edges, rounded up. */
size_t dbscan_workspace_bytes_with_edges(int64_t n, int32_t d,
                                         int64_t max_edges);

/* Fit from device memory, stream-ordered.
 *   d_points   device, n*d fp32, row-major; read only; caller-owned.
 *   d_labels   device, n int32; written; caller-owned.
 *   d_counts   device, n int32 neighbour counts (self included), or NULL.
 *   d_workspace, workspace_bytes  device scratch owned by the caller, at
 *              least dbscan_workspace_bytes(n, d), 256-byte aligned.  Bytes
 *              beyond that minimum become the edge area (8 bytes per pair);
 *              when every neighbour pair fits there the merge reuses them,
 *              otherwise it re-evaluates distances (same result, slower).
 *   hip_stream hipStream_t passed as void*; NULL = the default stream.
 * All kernels run on hip_stream.  The call synchronises that stream once,
 * after the last kernel, so the returned status is final (the choice
 * between the edge merge and the tile merge is taken on the device).  It
 * is not capturable into a HIP graph (that synchronisation, and a
 * device-to-host copy of a 64-byte status block into host memory).  Calls
 * on different streams with different workspaces may run concurrently; two
 * calls must not share a workspace at the same time.  The library keeps no
 * state between calls. */
int dbscan_fit_device(const float* d_points, int64_t n, int32_t d, float eps,
                      int32_t min_pts, int32_t* d_labels, int32_t* d_counts,
                      void* d_workspace, size_t workspace_bytes,
                      void* hip_stream);

/* As dbscan_fit_device, with flag bits (DBSCAN_FLAG_*) and an optional host
 * dbscan_info to fill (NULL allowed). */
int dbscan_fit_device_ex(const float* d_points, int64_t n, int32_t d,
                         float eps, int32_t min_pts, int32_t* d_labels,
                         int32_t* d_counts, void* d_workspace,
                         size_t workspace_bytes, void* hip_stream,
                         uint32_t flags, dbscan_info* info);

/* Fit from host memory: allocates device memory (points, labels, counts,
 * workspace with an edge area sized from free device memory), copies in,
 * fits on a stream of its own, copies out and frees everything before
 * returning.  Blocking.
 *   points  host, n*d fp32, row-major; read only; caller-owned.
 *   labels  host, n int32; written; caller-owned.
 * The problem is the one Wang et al. Sec. II states (points, eps and MinPts
 * in; clusters and noise out); the arguments are those of the contract
 * dbscan_fit(points[N x d], N, d, eps, minPts) -> labels. */
int dbscan_fit(const float* points, int64_t n, int32_t d, float eps,
               int32_t min_pts, int32_t* labels);

/* As dbscan_fit, and also copies out the neighbour counts (self included):
 * counts is host, n int32, caller-owned, or NULL (then exactly
 * dbscan_fit). */
int dbscan_fit_counts(const float* points, int64_t n, int32_t d, float eps,
                      int32_t min_pts, int32_t* labels, int32_t* counts);

/* Device scratch the no-allocation entry point works in, per GPU. */
#define DBSCAN_NOALLOC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same fit as dbscan_fit_device (same results, same arguments minus the
 * workspace), worked in a fixed scratch array of
 * DBSCAN_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends; the call itself allocates nothing (no
 * hipMalloc, no hipFree, no allocating library routine).  Inputs whose
 * dbscan_workspace_bytes(n, d) exceeds that size are refused with
 * DBSCAN_ERR_TOO_LARGE before any device work; the scratch beyond that
 * minimum serves as the edge area, so the merge reuses the count pass's
 * pairs when they fit.  Every call on one GPU shares that GPU's scratch,
 * which keeps the last call's contents (a fit clears what it needs
 * cleared): calls that overlap in time on one GPU, from any stream or
 * thread, race and must be serialised by the caller.  Synchronises
 * hip_stream once before returning, as dbscan_fit_device does. */
int dbscan_fit_device_noalloc(const float* d_points, int64_t n, int32_t d,
                              float eps, int32_t min_pts, int32_t* d_labels,
                              int32_t* d_counts, void* hip_stream);

/* Contiguous cluster ids from the labels of a fit: clusters are numbered
 * 0..K-1 in ascending order of their label (their smallest member, so the
 * numbering is as deterministic as the labels); noise stays -1.  A
 * scan-based renumbering, as the Times-C summary (Sec. 3.1) computes class
 * offsets.
 *   d_labels  device, n int32 labels from dbscan_fit*; read only.
 *   d_ids     device, n int32; written.
 *   d_sizes   device, n int32 or NULL; sizes[k] = members of cluster k for
 *             k < K (entries >= K untouched).
 *   n_clusters host, K on return (may be NULL).
 *   d_workspace at least dbscan_relabel_workspace_bytes(n), 256-aligned.
 * Labels that are not smallest-member labels (l < -1, l >= n, or
 * labels[l] != l) give DBSCAN_ERR_INVALID_ARG, detected on the device.
 * Synchronises hip_stream before returning. */
size_t dbscan_relabel_workspace_bytes(int64_t n);
int dbscan_relabel_device(const int32_t* d_labels, int64_t n, int32_t* d_ids,
                          int32_t* d_sizes, int64_t* n_clusters,
                          void* d_workspace, size_t workspace_bytes,
                          void* hip_stream);

/* Sparse epsilon-graph in CSR form: row i holds every j with
 * d2(i,j) <= eps2, i itself included, in ascending j, with d2 and eps2
 * exactly as for a fit.  These are the per-point neighbour lists that Wang
 * et al. Sec. IV-B keep as the rows of an N x N cluster matrix ("primitive
 * clusters"), stored here without the zeros; the row lengths are the
 * neighbour counts of a fit.
 *   d_points   device, n*d fp32, row-major; read only.
 *   d_row_ptr  device, n+1 int64; written whenever the count pass ran
 *              (also on DBSCAN_ERR_CAPACITY and DBSCAN_ERR_WORKSPACE):
 *              row_ptr[0] = 0, row_ptr[i+1] - row_ptr[i] = count[i],
 *              row_ptr[n] = nnz.
 *   d_col_idx  device, col_capacity int32; on success entries
 *              row_ptr[i] .. row_ptr[i+1]-1 hold row i.  May be NULL when
 *              col_capacity is 0 (a size query).
 *   nnz_out    host int64, or NULL: nnz, whenever the count pass ran.
 *   d_workspace, workspace_bytes  caller-owned device scratch, 256-byte
 *              aligned, at least dbscan_graph_workspace_bytes(n, d, pairs)
 *              for the number of neighbour pairs i<j, (nnz - n) / 2.
 *   flags      DBSCAN_FLAG_PRUNE_TILES, DBSCAN_FLAG_SCREEN,
 *              DBSCAN_FLAG_EXPANDED and DBSCAN_FLAG_TIME_PHASES; for
 *              this call ms_core times the row offsets, ms_merge the
 *              scatter of the pairs and ms_label the row sort.
 *   info       optional; n_edges = neighbour pairs i<j, edge_capacity =
 *              pairs the workspace holds, tiles as for a fit.
 * Returns DBSCAN_ERR_CAPACITY if nnz > col_capacity, then
 * DBSCAN_ERR_WORKSPACE if the pairs do not fit the workspace: a second call
 * with the sizes reported succeeds.  One distance pass per call.  Synchronises hip_stream (twice)
 * before returning; not capturable into a HIP graph. */
size_t dbscan_graph_workspace_bytes(int64_t n, int32_t d, int64_t max_pairs);
int dbscan_graph_device(const float* d_points, int64_t n, int32_t d, float eps,
                        int64_t* d_row_ptr, int32_t* d_col_idx,
                        int64_t col_capacity, int64_t* nnz_out,
                        void* d_workspace, size_t workspace_bytes,
                        void* hip_stream, uint32_t flags, dbscan_info* info);

/* Static, never-NULL description of a status code. */
const char* dbscan_status_string(int status);

/* DBSCAN_ABI_VERSION of the loaded library. */
int dbscan_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DBSCAN_MI355X_H */

// Internal declarations shared by the library's translation units.
// Nothing here is part of the C ABI (include/dbscan.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dbk {

// Rows per work item of the tile passes (a multiple of the 64-lane wave;
// the count pass uses fewer when that would leave too few work items).
constexpr int kRowsPerItem = 1024;
// Edge records staged in LDS per wave before a flush to the edge area; at
// least the 512 pairs of the (up to) 8 column groups staged per check.
constexpr int kEdgeStage = 512;
constexpr int kThreads = 256;  // 4 waves of 64 lanes per workgroup
constexpr int kMaxGrid = 1 << 20;

// Device-side status block at the start of the workspace.
struct Status {
  unsigned int nonfinite;          // set to 1 if any input coordinate is NaN/inf
  unsigned int n_core;             // number of core points
  unsigned long long n_edges;      // edge slots reserved by the count pass
  unsigned int n_core_list;        // entries written by the core compaction
  unsigned int graph_bad;           // a graph slot fell outside its row
  unsigned long long n_tiles;      // block pairs kept by the tile pruning
  unsigned long long ymax_bits;    // largest squared norm (fp64 bits), screen
  unsigned int screen_unsafe;      // a norm too large for the screen bound
  unsigned int long_rows;          // graph rows listed for the work-group sort
  unsigned int pad[4];
};
static_assert(sizeof(Status) == 64, "status block is 64 bytes");

// True when the fit merges by the tile pass: no edge area was offered, or
// the count pass found more neighbour pairs than it holds.  Decided on the
// device from the status block, so a fit needs no host round trip before
// its merge.
__device__ __forceinline__ bool tile_merge_needed(const Status* st,
                                                  bool want_edges,
                                                  unsigned long long edge_cap) {
  return !want_edges || st->n_edges > edge_cap;
}

// Row stride of the internal point layout: d padded with zeros to the
// compiled dimension D, then to a multiple of 4 floats (16-byte rows) when
// D > 2 so each row is one aligned scalar/vector load.
constexpr int row_stride(int D) { return D <= 2 ? D : ((D + 3) & ~3); }

// The compiled dimensions; a fit with dimension d runs the smallest D >= d
// (extra coordinates are 0 on both sides, which adds exact zeros to the sum).
constexpr int kDims[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64};
int pick_dim(int d);  // smallest compiled D >= d, or 0

// Row stride of the screen's row table: -2x (D floats), then the two
// thresholds, padded to a multiple of 4 floats.
constexpr int screen_stride(int D) { return (D + 2 + 3) & ~3; }

// Column points per lane of the count pass (P) for width D; its blocks hold
// T = 256 * P points (4 waves of 64 lanes).
constexpr int lane_points(int D) {
  return D <= 2 ? 16 : D <= 4 ? 8 : D <= 8 ? 4 : D <= 16 ? 2 : 1;
}
constexpr int block_points(int D) { return 256 * lane_points(D); }
// Point counts are padded to a multiple of this for width D: the count
// pass's block of T points (4096 down to 256), and at least 1024, the block
// of the core-flag pass, of the tile merge's row items and of the scans.
// Padding rows are evaluated like real ones (their NaN never matches), so
// a finer multiple is less wasted work: at 200,000 points of width 8 the
// pass decides 0.7% padding pairs instead of 4.9% with a fixed 4096.
constexpr int64_t pad_multiple(int D) {
  return block_points(D) > 1024 ? block_points(D) : 1024;
}
// Most block pairs a pruning tile list holds (beyond: no pruning).
constexpr int64_t kTileListCap = (int64_t)1 << 24;

struct Layout {
  int64_t n, n_pad;
  int d, D, stride;
  // neighbours decided with the hoisted-norm form T + P - sum 2 x_k y_k
  // (always screened, never pruned) instead of the direct distance
  bool expanded;
  // carved from the workspace
  Status* status;
  float* pts;          // [n_pad][stride], padded rows are NaN
  unsigned* count;     // [n_pad]
  unsigned char* core; // [n_pad]
  int* parent;         // [n_pad] union-find forest over core points
  int* bmin;           // [n_pad] lowest core neighbour of a non-core point
  int* cmin;           // [n_pad] smallest member per root
  int* core_list;      // [n_pad] compacted core indices (tile merge)
  float* core_pts;     // [n_pad][stride] their coordinates (tile merge)
  unsigned* block_sums;// [n_pad / 1024 + 1] compaction scan
  // tile pruning (used only when asked for)
  unsigned* bbox;      // [12] order-encoded min/max of up to 6 key coordinates
  unsigned* keys_in;   // [n_pad] key sort: the other key buffer
  unsigned* keys_out;  // [n_pad] sort keys (in ascending order once sorted)
  int* idx_in;         // [n_pad] key sort: the other index buffer
  int* perm;           // [n_pad] sorted position -> original index
  float* sorted_pts;   // [n_pad][stride] points in sorted order
  float* boxes;        // [nb][2][stride] block bounding boxes
  float* boxes64;      // [n_pad/64][2][stride] boxes of 64-point row groups
  float* boxes_w;      // [n_pad/(64P)][2][stride] boxes of a wave's columns
  float* pca;          // [7*stride + 1] sort-key directions of wide points
  uint2* tiles;        // kept block pairs
  unsigned long long tile_cap;
  float* srow;         // [n_pad][screen_stride] screen row table
  float* ncol;         // [n_pad] fp32 squared norm of each point (screen)
  float* nexp;         // [n_pad] squared norm as the hoisted-norm form
                       //         takes it: rounded squares summed in k order
  unsigned* sort_hist;  // key sort: digit totals, then per-tile counts
  uint2* edges;        // edge area (may be empty)
  unsigned long long edge_cap;
  size_t bytes_min;    // minimum workspace
};

// Extra regions of a graph export, carved after the fit's layout.
struct GraphLayout {
  unsigned* cursor;              // [n] next free slot of each row
  unsigned long long* row_sums;  // [n / 1024 + 1] row-offset scan
  void* alt;                     // second sort buffer (overlays the pairs)
};

size_t layout_min_bytes(int64_t n, int d);
bool carve(Layout& L, void* ws, size_t ws_bytes);

// The order in which a launch walks its work: a test mode whose results
// must not change.  Work item `step` of `count` is item
// (mul * step + add) mod count: mul = 1 walks in order, mul = -1 (add =
// count - 1) in reverse, other multipliers (below 2^14, coprime with
// count) a fixed shuffle.
struct Walk {
  uint32_t seed;  // 0: in order; 1: reverse; otherwise a shuffle
};
struct WalkArgs {
  int64_t mul, add;
};
WalkArgs walk_args(Walk w, int64_t count);

// ---- launchers (each enqueues on `s` and returns hipGetLastError) -------
hipError_t launch_prepare(const Layout& L, const float* in, hipStream_t s);
hipError_t launch_count(const Layout& L, float eps2, bool edges, bool pruned,
                        bool screen, Walk walk, hipStream_t s,
                        int64_t* pairs);
// The screened count pass runs on the matrix cores for these widths
// (launch_count_mfma); its thresholds are then widened for the matrix
// unit's arithmetic.
constexpr bool screen_on_matrix_cores(int D) { return D >= 16; }
hipError_t launch_count_mfma(const Layout& L, float eps2, bool edges,
                             bool pruned, Walk walk, hipStream_t s,
                             int64_t* pairs);
hipError_t launch_screen(const Layout& L, const float* pts, float eps2,
                         hipStream_t s);
size_t prune_sort_bytes(int64_t n_pad);
hipError_t launch_prune(const Layout& L, int T, float eps2, hipStream_t s);
hipError_t launch_core(const Layout& L, int min_pts, int* counts_out,
                       hipStream_t s);
// The merge is chosen on the device (tile_merge_needed): one launch links
// the recorded pairs or, when they overflowed, compacts the core points;
// the tile merge after it exits at once unless it is needed.  want_edges:
// an edge area was offered; spread: take the pairs in a strided chunk
// order (for the spatially grouped pairs of a pruned pass).
hipError_t launch_merge_edges(const Layout& L, bool want_edges, Walk walk,
                              bool spread, hipStream_t s);
hipError_t launch_merge_tiles(const Layout& L, float eps2, bool want_edges,
                              Walk walk, hipStream_t s);
hipError_t launch_label(const Layout& L, int* labels, hipStream_t s);
hipError_t launch_row_offsets(const Layout& L, const GraphLayout& G,
                              int64_t* row_ptr, int* col_idx,
                              unsigned long long col_cap, hipStream_t s);
hipError_t launch_graph_scatter(const Layout& L, const GraphLayout& G,
                                unsigned long long n_pairs,
                                const int64_t* row_ptr, int* col_idx,
                                hipStream_t s);
hipError_t launch_graph_sort(const Layout& L, const GraphLayout& G,
                             const int64_t* row_ptr, int* col_idx, int64_t nnz,
                             hipStream_t s);

}  // namespace dbk

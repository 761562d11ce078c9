// Cluster merge and border assignment.
//
// Merge criterion (Wang et al., Sec. II items 2-3 and the cluster
// definition): two core points within eps are directly reachable from each
// other, so they end in one cluster; reachability runs only through core
// points.  Clusters are therefore the connected components of the graph of
// core points with edges between cores within eps.  The paper's merge
// kernel (Sec. IV-C) retries clusters against one target per launch; here
// every core-core edge is linked at once in a lock-free union-find (larger
// root hung under the smaller root with atomicCAS, path halving), which
// makes the final roots the smallest core index of each component whatever
// the order of the links.
//
// A non-core point within eps of at least one core point joins the cluster
// of its lowest-index core neighbour (atomicMin over its core neighbours).
//
// Two ways to find those pairs:
//   k_merge_edges  walks the neighbour pairs the count pass recorded;
//   k_merge_tiles  re-evaluates distances in a second tile pass of all
//                  points (rows) against the sorted core points (columns),
//                  used when no edge area was given or it overflowed.
#include <climits>

#include "device.h"
#include "internal.h"

namespace dbk {

// One launch for what precedes the tile merge or replaces it, chosen on
// the device from the status block (the host never waits for it):
//   - the pairs fit the edge area: link them (grid-stride over the pairs);
//   - they overflowed it, or no edge area was offered: compact the core
//     points for the tile merge that follows (each block of 1024 points
//     writes its cores in index order at the offset k_scan_totals gave
//     it);
//   - no core point: nothing to do.
__global__ __launch_bounds__(256) void k_merge_edges(
    const uint2* __restrict__ edges, unsigned long long edge_cap,
    bool want_edges, const unsigned char* __restrict__ core, int* parent,
    int* __restrict__ bmin, const Status* __restrict__ st, WalkArgs walk,
    const float* __restrict__ pts, int S, int64_t n_pad,
    const unsigned* __restrict__ sums, int* __restrict__ core_list,
    float* __restrict__ core_pts, bool spread) {
  if (st->n_core == 0) return;
  if (tile_merge_needed(st, want_edges, edge_cap)) {
    __shared__ unsigned sh[4];
    for (int64_t blk = blockIdx.x; blk < n_pad / 1024; blk += gridDim.x) {
      const int64_t base = blk * 1024 + threadIdx.x * 4;
      const unsigned f4 = *reinterpret_cast<const unsigned*>(core + base);
      unsigned f[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = (f4 >> (8 * q)) & 0xffu;
      unsigned tot;
      unsigned pos = sums[blk] +
                     block_excl_scan(f[0] + f[1] + f[2] + f[3], sh, &tot);
      for (int q = 0; q < 4; ++q) {
        if (f[q]) {
          const int64_t i = base + q;
          core_list[pos] = (int)i;
          for (int k = 0; k < S; ++k)
            core_pts[(int64_t)pos * S + k] = pts[i * S + k];
          ++pos;
        }
      }
    }
    return;
  }
  const unsigned long long ne = st->n_edges;
  // (a test mode walks the pairs in another order: results must not
  // change)
  walk_refit((int64_t)ne, walk.mul, walk.add);
  // With spread, wave-sized chunks of pairs are taken in a strided order
  // (chunk c' = 16381 c mod chunks, or the next multiplier coprime with
  // the chunk count).  The pairs of a pruned pass arrive grouped by space,
  // so consecutive chunks mostly link points of one cluster and contend
  // for its root; spread, concurrent chunks come from the whole set.
  // Pruned fits: 1M x 3 merge and labels 1.24 -> 0.96 ms, 262k x 64
  // 7.27 -> 6.66 ms; the unpruned order (neighbouring chunks sharing cache
  // lines) keeps its own: the 262k x 64 merge went 2.45 -> 2.82 ms spread.
  constexpr int kChunk = 64;
  const int64_t chunks = (int64_t)((ne + kChunk - 1) / kChunk);
  int64_t cmul = spread ? 16381 : 1, cadd = 0;
  walk_refit(chunks, cmul, cadd);
  const unsigned long long span = (unsigned long long)chunks * kChunk;
  for (unsigned long long k = blockIdx.x * (unsigned long long)blockDim.x +
                              threadIdx.x;
       k < span; k += (unsigned long long)gridDim.x * blockDim.x) {
    const unsigned long long k2 =
        (unsigned long long)walk_item((int64_t)(k / kChunk), chunks, cmul, cadd) *
            kChunk + k % kChunk;
    if (k2 >= ne) continue;
    const unsigned long long e =
        (unsigned long long)walk_item((int64_t)k2, (int64_t)ne, walk.mul, walk.add);
    const uint2 ij = edges[e];
    const int i = (int)ij.x, j = (int)ij.y;
    // a non-core point's parent is -1 (set with the core flags), so the two
    // parent loads that start a union also tell which ends are cores
    const int pi = uf_load(parent + i), pj = uf_load(parent + j);
    if (pi >= 0 && pj >= 0)
      uf_union(parent, i, j, pi, pj);
    else if (pi >= 0)
      atomicMin(bmin + j, i);
    else if (pj >= 0)
      atomicMin(bmin + i, j);
  }
}

// Enough work-groups to fill every CU at full occupancy (256 CUs x 8 of
// 256 threads); the pair count is only known on the device.
constexpr unsigned kMergeGrid = 2048;

hipError_t launch_merge_edges(const Layout& L, bool want_edges, Walk walk,
                              bool spread, hipStream_t s) {
  const unsigned long long e_cap = want_edges ? L.edge_cap : 0ull;
  unsigned long long g = (e_cap + 255) / 256;
  const unsigned long long nblk = (unsigned long long)L.n_pad / 1024;
  if (g < nblk) g = nblk;
  if (g > kMergeGrid) g = kMergeGrid;
  k_merge_edges<<<(unsigned)g, 256, 0, s>>>(
      L.edges, e_cap, want_edges, L.core, L.parent, L.bmin, L.status,
      walk_args(walk, (int64_t)(e_cap < 2 ? 2 : e_cap)), L.pts, L.stride,
      L.n_pad, L.block_sums, L.core_list, L.core_pts, spread);
  return hipGetLastError();
}

typedef const unsigned char __attribute__((address_space(4)))* const_u8_ptr;

// EXPANDED: pairs are decided with the hoisted-norm form, from the norm
// table nexp (indexed by original point).
// Work items are (rows-row block) x (T-core column block) pairs, walked
// grid-stride; the number of column blocks follows from the core count,
// read on the device.  Exits at once unless the fit merges by tiles.
template <int D, bool EXPANDED, int PP = lane_points(D)>
__global__ __launch_bounds__(kThreads) void k_merge_tiles(
    const float* __restrict__ pts, const float* __restrict__ core_pts,
    const int* __restrict__ core_list, const unsigned char* __restrict__ core,
    int64_t row_blocks, int rows, float eps2, int* parent,
    int* __restrict__ bmin, const float* __restrict__ nexp,
    const Status* __restrict__ st, bool want_edges,
    unsigned long long edge_cap, WalkArgs walk_r, WalkArgs walk_c) {
  constexpr int P = PP;
  constexpr int T = 256 * P;
  constexpr int S = row_stride(D);
  const int64_t n_core = st->n_core_list;
  if (n_core == 0 || !tile_merge_needed(st, want_edges, edge_cap)) return;
  const int64_t col_blocks = (n_core + T - 1) / T;
  const int64_t items = row_blocks * col_blocks;
  walk_refit(col_blocks, walk_c.mul, walk_c.add);
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    // (a test mode walks the blocks in another order: results must not
    // change)
    const int64_t rs = item / col_blocks, cs = item - rs * col_blocks;
    const int64_t rblk = walk_item(rs, row_blocks, walk_r.mul, walk_r.add);
    const int64_t cblk = walk_item(cs, col_blocks, walk_c.mul, walk_c.add);
    const int64_t row0 = rblk * rows;
    const int64_t colw = cblk * T + (int64_t)wave * 64 * P;
    float xc[P][D];
    int cidx[P];
    float pc[EXPANDED ? P : 1];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      // columns past the cores are NaN (never a neighbour); their list
      // entries and coordinates were not written and are not read
      const int64_t c = colw + p * 64 + lane;
      const bool real = c < n_core;
      cidx[p] = real ? core_list[c] : INT_MAX;
#pragma unroll
      for (int k = 0; k < D; ++k)
        xc[p][k] = real ? core_pts[c * S + k] : __builtin_nanf("");
      if (EXPANDED) pc[p] = real ? nexp[cidx[p]] : 0.f;
    }
    for (int rb = 0; rb < rows; rb += 64) {
      int rowmin = INT_MAX;  // lane l: lowest core neighbour of row rb+l
      for (int l = 0; l < 64; ++l) {
        const int64_t row = row0 + rb + l;
        const const_float_ptr rp = (const_float_ptr)(pts + row * S);
        float xr[D];
#pragma unroll
        for (int k = 0; k < D; ++k) xr[k] = rp[k];
        const bool row_core = ((const_u8_ptr)core)[row] != 0;
        const float tr = EXPANDED ? ((const_float_ptr)nexp)[row] : 0.f;
        int best = INT_MAX;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const bool nb = (EXPANDED ? expanded_d2<D>(xr, xc[p], tr, pc[p])
                                    : dist2<D>(xr, xc[p])) <= eps2;
          const uint64_t m = ballot(nb);
          if (m) {
            if (row_core) {
              if (nb) uf_union(parent, (int)row, cidx[p]);
            } else if (best == INT_MAX) {
              // columns ascend with p and lane: the first hit is the lowest
              best = __builtin_amdgcn_readlane(cidx[p], (int)__builtin_ctzll(m));
            }
          }
        }
        rowmin = write_lane(rowmin, best, l);
      }
      if (rowmin != INT_MAX) atomicMin(bmin + row0 + rb + lane, rowmin);
    }
  }
}

// Rows per work item, halved from 1,024 (down to 64) while the plan would
// give fewer than 4,096 items (every point a core), and one column point
// per lane when even that is under 512 items: small sets would otherwise
// run a handful of long work-groups (2,000 points at d = 2: 4 items, the
// merge 4.1 ms).
template <int D, int P>
static hipError_t launch_merge_tiles_p(const Layout& L, float eps2,
                                       bool want_edges, Walk walk,
                                       hipStream_t s) {
  constexpr int T = 256 * P;
  int rows = kRowsPerItem;
  while (rows > 64 && (L.n_pad / rows) * (L.n_pad / T) < 4096) rows >>= 1;
  const int64_t row_blocks = L.n_pad / rows;
  // sized for the most items (every point a core); the excess exits
  const int64_t most = row_blocks * (L.n_pad / T);
  const unsigned grid = (unsigned)(most < 4096 ? most : 4096);
  const WalkArgs wr = walk_args(walk, row_blocks);
  const WalkArgs wc = walk_args(walk, L.n_pad / T < 2 ? 2 : L.n_pad / T);
  if (L.expanded)
    k_merge_tiles<D, true, P><<<grid, kThreads, 0, s>>>(
        L.pts, L.core_pts, L.core_list, L.core, row_blocks, rows, eps2,
        L.parent, L.bmin, L.nexp, L.status, want_edges, L.edge_cap, wr, wc);
  else
    k_merge_tiles<D, false, P><<<grid, kThreads, 0, s>>>(
        L.pts, L.core_pts, L.core_list, L.core, row_blocks, rows, eps2,
        L.parent, L.bmin, nullptr, L.status, want_edges, L.edge_cap, wr, wc);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_merge_tiles_d(const Layout& L, float eps2,
                                       bool want_edges, Walk walk,
                                       hipStream_t s) {
  constexpr int T = 256 * lane_points(D);
  if (lane_points(D) > 1 && (L.n_pad / 64) * (L.n_pad / T) < 512)
    return launch_merge_tiles_p<D, 1>(L, eps2, want_edges, walk, s);
  return launch_merge_tiles_p<D, lane_points(D)>(L, eps2, want_edges, walk, s);
}

hipError_t launch_merge_tiles(const Layout& L, float eps2, bool want_edges,
                              Walk walk, hipStream_t s) {
  switch (L.D) {
#define DBK_CASE(DD) \
  case DD: return launch_merge_tiles_d<DD>(L, eps2, want_edges, walk, s);
    DBK_CASE(1) DBK_CASE(2) DBK_CASE(3) DBK_CASE(4) DBK_CASE(6) DBK_CASE(8)
    DBK_CASE(12) DBK_CASE(16) DBK_CASE(24) DBK_CASE(32) DBK_CASE(48)
    DBK_CASE(64)
#undef DBK_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dbk

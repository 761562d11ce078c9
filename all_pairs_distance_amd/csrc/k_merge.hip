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

__global__ void k_merge_edges(const uint2* __restrict__ edges,
                              unsigned long long ne,
                              const unsigned char* __restrict__ core,
                              int* parent, int* __restrict__ bmin,
                              WalkArgs walk) {
  for (unsigned long long k = blockIdx.x * (unsigned long long)blockDim.x +
                              threadIdx.x;
       k < ne; k += (unsigned long long)gridDim.x * blockDim.x) {
    // (a test mode walks the pairs in another order: results must not
    // change)
    const unsigned long long e =
        (unsigned long long)walk_item((int64_t)k, (int64_t)ne, walk.mul, walk.add);
    const uint2 ij = edges[e];
    const int i = (int)ij.x, j = (int)ij.y;
    const bool ci = core[i] != 0, cj = core[j] != 0;
    if (ci && cj)
      uf_union(parent, i, j);
    else if (ci)
      atomicMin(bmin + j, i);
    else if (cj)
      atomicMin(bmin + i, j);
  }
}

hipError_t launch_merge_edges(const Layout& L, unsigned long long n_edges,
                              Walk walk, hipStream_t s) {
  if (n_edges == 0) return hipSuccess;
  unsigned long long g = (n_edges + 255) / 256;
  if (g > (unsigned long long)kMaxGrid) g = kMaxGrid;
  k_merge_edges<<<(unsigned)g, 256, 0, s>>>(L.edges, n_edges, L.core,
                                            L.parent, L.bmin,
                                            walk_args(walk, (int64_t)n_edges));
  return hipGetLastError();
}

typedef const unsigned char __attribute__((address_space(4)))* const_u8_ptr;

// EXPANDED: pairs are decided with the hoisted-norm form, from the norm
// table nexp (indexed by original point).
template <int D, bool EXPANDED>
__global__ __launch_bounds__(kThreads) void k_merge_tiles(
    const float* __restrict__ pts, const float* __restrict__ core_pts,
    const int* __restrict__ core_list, const unsigned char* __restrict__ core,
    int64_t row_blocks, int64_t col_blocks, float eps2, int* parent,
    int* __restrict__ bmin, const float* __restrict__ nexp, int64_t n_core,
    WalkArgs walk_r, WalkArgs walk_c) {
  constexpr int P = lane_points(D);
  constexpr int T = 256 * P;
  constexpr int S = row_stride(D);
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  for (int64_t rs = blockIdx.y; rs < row_blocks; rs += gridDim.y)
  for (int64_t cs = blockIdx.x; cs < col_blocks; cs += gridDim.x) {
    // (a test mode walks the blocks in another order: results must not
    // change)
    const int64_t rblk = walk_item(rs, row_blocks, walk_r.mul, walk_r.add);
    const int64_t cblk = walk_item(cs, col_blocks, walk_c.mul, walk_c.add);
    const int64_t row0 = rblk * kRowsPerItem;
    const int64_t colw = cblk * T + (int64_t)wave * 64 * P;
    float xc[P][D];
    int cidx[P];
    float pc[EXPANDED ? P : 1];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int64_t c = colw + p * 64 + lane;
      cidx[p] = core_list[c];
#pragma unroll
      for (int k = 0; k < D; ++k) xc[p][k] = core_pts[c * S + k];
      // columns past the cores have NaN coordinates and never match (their
      // core_list entries are not written): no norm is read for them
      if (EXPANDED) pc[p] = c < n_core ? nexp[cidx[p]] : 0.f;
    }
    for (int rb = 0; rb < kRowsPerItem; rb += 64) {
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

template <int D>
static hipError_t launch_merge_tiles_d(const Layout& L, float eps2,
                                       int64_t n_core, Walk walk,
                                       hipStream_t s, int64_t* pairs) {
  constexpr int T = 256 * lane_points(D);
  const int64_t nc_pad = (n_core + T - 1) / T * T;
  const int64_t col_blocks = nc_pad / T;
  const int64_t row_blocks = L.n_pad / kRowsPerItem;
  if (row_blocks == 0 || col_blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)(col_blocks < 4096 ? col_blocks : 4096),
                  (unsigned)(row_blocks < 4096 ? row_blocks : 4096));
  if (L.expanded)
    k_merge_tiles<D, true><<<grid, kThreads, 0, s>>>(
        L.pts, L.core_pts, L.core_list, L.core, row_blocks, col_blocks, eps2,
        L.parent, L.bmin, L.nexp, n_core, walk_args(walk, row_blocks),
        walk_args(walk, col_blocks));
  else
    k_merge_tiles<D, false><<<grid, kThreads, 0, s>>>(
        L.pts, L.core_pts, L.core_list, L.core, row_blocks, col_blocks, eps2,
        L.parent, L.bmin, nullptr, n_core, walk_args(walk, row_blocks),
        walk_args(walk, col_blocks));
  if (pairs) *pairs = L.n_pad * nc_pad;
  return hipGetLastError();
}

hipError_t launch_merge_tiles(const Layout& L, float eps2, int64_t n_core,
                              Walk walk, hipStream_t s, int64_t* pairs) {
  switch (L.D) {
    case 1: return launch_merge_tiles_d<1>(L, eps2, n_core, walk, s, pairs);
    case 2: return launch_merge_tiles_d<2>(L, eps2, n_core, walk, s, pairs);
    case 3: return launch_merge_tiles_d<3>(L, eps2, n_core, walk, s, pairs);
    case 4: return launch_merge_tiles_d<4>(L, eps2, n_core, walk, s, pairs);
    case 6: return launch_merge_tiles_d<6>(L, eps2, n_core, walk, s, pairs);
    case 8: return launch_merge_tiles_d<8>(L, eps2, n_core, walk, s, pairs);
    case 12: return launch_merge_tiles_d<12>(L, eps2, n_core, walk, s, pairs);
    case 16: return launch_merge_tiles_d<16>(L, eps2, n_core, walk, s, pairs);
    case 24: return launch_merge_tiles_d<24>(L, eps2, n_core, walk, s, pairs);
    case 32: return launch_merge_tiles_d<32>(L, eps2, n_core, walk, s, pairs);
    case 48: return launch_merge_tiles_d<48>(L, eps2, n_core, walk, s, pairs);
    case 64: return launch_merge_tiles_d<64>(L, eps2, n_core, walk, s, pairs);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dbk

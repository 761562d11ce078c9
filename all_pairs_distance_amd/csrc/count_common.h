// Helpers shared by the count kernels (k_count.hip, k_count_mfma.hip):
// the tile enumeration, the edge sink and the wave's LDS edge stage.
#pragma once

#include <cmath>

#include "device.h"
#include "internal.h"

namespace dbk {

// Upper-triangle tile t (row-major over I <= J of nb x nb blocks) -> (I, J).
__device__ __forceinline__ void tile_coords(int64_t t, int64_t nb, int64_t& I,
                                            int64_t& J) {
  const double b = 2.0 * (double)nb + 1.0;
  int64_t i = (int64_t)((b - sqrt(b * b - 8.0 * (double)t)) * 0.5);
  if (i < 0) i = 0;
  if (i > nb - 1) i = nb - 1;
  while (i > 0 && i * nb - i * (i - 1) / 2 > t) --i;
  while (i + 1 < nb && (i + 1) * nb - (i + 1) * i / 2 <= t) ++i;
  I = i;
  J = i + (t - (i * nb - i * (i - 1) / 2));
}

// The same triangle in an order that keeps a cache's worth of blocks
// together: super-tiles of kSuperTile x kSuperTile tiles, row-major over
// the triangle of super-tiles, each walked row-major (the diagonal
// super-tiles over their own triangle).  A full super-row s holds
// K(K+1)/2 + K (nb - (s+1) K) tiles, so the first tile of super-row s is
// s K(K+1)/2 + K (s nb - K s(s+1)/2), and a binary search finds the
// super-row.  (A bijection onto the triangle for every nb.)
constexpr int64_t kSuperTile = 16;
__host__ __device__ __forceinline__ int64_t super_row_start(int64_t s, int64_t nb) {
  const int64_t K = kSuperTile;
  return s * (K * (K + 1) / 2) + K * (s * nb - K * s * (s + 1) / 2);
}
__host__ __device__ __forceinline__ void tile_coords_blocked(int64_t t,
                                                             int64_t nb,
                                                             int64_t& I,
                                                             int64_t& J) {
  const int64_t K = kSuperTile;
  int64_t lo = 0, hi = (nb + K - 1) / K - 1;   // last s with start(s) <= t
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (super_row_start(mid, nb) <= t) lo = mid;
    else hi = mid - 1;
  }
  const int64_t s = lo;
  int64_t u = t - super_row_start(s, nb);
  const int64_t r = nb - s * K < K ? nb - s * K : K;   // rows of super-row s
  const int64_t diag = r * (r + 1) / 2;
  if (u < diag) {
    int64_t a = 0;
    while (u >= r - a) {
      u -= r - a;
      ++a;
    }
    I = s * K + a;
    J = I + u;
  } else {
    u -= diag;
    const int64_t m = u / (r * K);               // full super-tiles before
    const int64_t SJ = s + 1 + m;
    const int64_t v = u - m * r * K;
    const int64_t c = nb - SJ * K < K ? nb - SJ * K : K;
    I = s * K + v / c;
    J = SJ * K + v % c;
  }
}

// Work-group b runs on XCD b mod 8 (the hardware deals work-groups to the
// eight XCDs in turn, and each XCD has its own L2): step b takes the
// (b div 8)-th item of XCD b mod 8's contiguous eighth of the items.  A
// bijection on [0, items) for any item count.
__host__ __device__ __forceinline__ int64_t xcd_item(int64_t step, int64_t items) {
  const int64_t q = items >> 3, r = items & 7, x = step & 7, j = step >> 3;
  return x * q + (x < r ? x : r) + j;
}

// Unpruned passes from this many block rows on (where the points outgrow
// an XCD's 4 MB L2) walk the tiles in the blocked order, an eighth per
// XCD.  1M x 3: the count kernel's fetches from the fabric 3.26 -> 0.29 GB
// per launch, its writes 2.04 -> 1.68 GB, time unchanged (the kernel is
// VALU-bound), the merge of its pairs 0.74 -> 0.67 ms.  Smaller sets keep
// the row-major order: their merge was 9-14% slower on the pairs of the
// blocked order (they arrive in another order), for no time in the count.
constexpr int64_t kBlockedTileRows = 256;

struct EdgeSink {
  uint2* edges;
  unsigned long long cap;
  unsigned long long* counter;
};

// Order this wave's LDS accesses around a hand-over between lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Copy the wave's staged edges to the edge area (one atomic per flush).
// Slots past the capacity are dropped; the host sees the overflow because
// the counter then exceeds the capacity.
__device__ __forceinline__ void flush_edges(uint2* stage, unsigned fill,
                                            const EdgeSink& sink) {
  wave_lds_sync();
  unsigned long long base = 0;
  if (lane_id() == 0) base = atomicAdd(sink.counter, (unsigned long long)fill);
  base = uniform_u64(base);
  for (unsigned k = lane_id(); k < fill; k += 64) {
    const unsigned long long dst = base + k;
    if (dst < sink.cap) sink.edges[dst] = stage[k];
  }
  wave_lds_sync();
}

// Stage captured pairs: lane l contributes one pair per set bit b of its
// `bits`, pair_of(b) (a uint2 of output indices), and the pairs are packed
// by a prefix sum over the lanes instead of one ballot scan per column
// group.  When the pairs outnumber the stage they reserve their slots in
// the edge area and are written there directly.
template <typename PairOf>
__device__ __forceinline__ void stage_pairs(unsigned bits, PairOf pair_of,
                                            uint2* stage, unsigned& fill,
                                            const EdgeSink& sink) {
  const unsigned n_e = (unsigned)__builtin_popcount(bits);
  const unsigned incl = wave_incl_sum(n_e);
  const unsigned total = (unsigned)__builtin_amdgcn_readlane((int)incl, 63);
  if (total == 0) return;
  if (fill + total > (unsigned)kEdgeStage) {
    if (fill) flush_edges(stage, fill, sink);
    fill = 0;
  }
  if (total <= (unsigned)kEdgeStage) {
    unsigned pos = fill + incl - n_e;
    for (unsigned w = bits; w != 0; w &= w - 1)
      stage[pos++] = pair_of(__builtin_ctz(w));
    fill += total;
  } else {
    unsigned long long base = 0;
    if (lane_id() == 0) base = atomicAdd(sink.counter, (unsigned long long)total);
    base = uniform_u64(base) + (incl - n_e);
    for (unsigned w = bits; w != 0; w &= w - 1) {
      if (base < sink.cap) sink.edges[base] = pair_of(__builtin_ctz(w));
      ++base;
    }
  }
}

// Threshold for wave_boxes_apart.  Let G be the ascending-k fp32 sum of
// the S squared gaps q_k and W their tree sum (at most 7 additions per
// term), T the exact sum of the q_k.  Both sums of non-negative terms lie
// within a relative g_m = m u / (1 - m u) of T: G >= (1 - g_{S-1}) T and
// W <= (1 + g_7) T, so W > eps2 (1 + g_8) / (1 - g_S) proves G > eps2.
// Every pair's fp32 distance is at least G (boxes_apart), so the boxes
// hold no neighbours.  The bound is rounded up to fp32.
inline float box_gap_threshold(float eps2, int S) {
  const double u = 0x1p-24;
  const auto g = [u](double m) { return m * u / (1.0 - m * u); };
  const double t = (double)eps2 * (1.0 + g(8.0)) / (1.0 - g((double)S)) *
                   (1.0 + 0x1p-50);
  float f = (float)t;
  if ((double)f < t) f = nextafterf(f, __builtin_inff());
  return f;
}

// Work items of a count launch: the upper triangle of nb x nb blocks of T
// points, each tile cut into chunks of `rows` rows.  A whole block of T
// rows per item loads each column block once per tile (a pruned launch
// keeps only some tiles and splits them into items of up to kRowsPerItem
// rows for parallelism); fewer rows, down to one wave's 64, while the full
// triangle would give under 32768 items (16 per resident work-group slot
// at 8 per CU), which keeps the launch's tail short: 200k x 8 points with
// 19,306 whole-tile items ran 2.5% slower than with 38,612 half-tile ones.
struct CountPlan {
  int64_t nb, items;
  int rows, chunks_log2;
  unsigned grid;
};

inline CountPlan plan_count(int64_t n_pad, int T, bool pruned) {
  CountPlan c;
  c.nb = n_pad / T;
  const int64_t tiles = c.nb * (c.nb + 1) / 2;
  c.rows = pruned && kRowsPerItem < T ? kRowsPerItem : T;
  while (c.rows > 64 && tiles * (T / c.rows) < 32768) c.rows >>= 1;
  const int chunks = T / c.rows;  // both powers of two
  c.chunks_log2 = 0;
  while ((1 << c.chunks_log2) < chunks) ++c.chunks_log2;
  c.items = tiles * chunks;
  const int64_t max_grid = pruned ? 16384 : kMaxGrid;
  c.grid = (unsigned)(c.items < max_grid ? c.items : max_grid);
  return c;
}

}  // namespace dbk

// Neighbour-count pass: count[i] = |{ j : d2(i,j) <= eps2 }| over all
// ordered pairs, never storing the N x N relation.
//
// The relation is cut into square blocks of T = 256*P points and only the
// upper triangle of block pairs (I <= J) is visited.  Because the fp32
// distance is bitwise symmetric (fl(a-b) = -fl(b-a), equal squares), one
// evaluation decides both (i,j) and (j,i): off-diagonal tiles credit the
// row point and the column point, diagonal tiles credit only the row
// point (every ordered pair of the block is evaluated there, the point
// itself included).  This is the distance-matrix step of Wang et al.,
// Sec. IV-A / IV-B1 (distance fused with the eps^2 comparison and the
// count, nothing written per pair), restructured for a 64-lane wave:
//   - each wave holds P column points per lane in VGPRs (the paper keeps
//     the goal point in registers, Sec. IV-A3);
//   - row points are wave-uniform and read with scalar loads, so the
//     distance is one VALU op per step with an SGPR operand;
//   - the comparison becomes a 64-bit ballot: its popcount (scalar unit) is
//     the row point's count over 64 columns, and each lane adds its own bit
//     for the column point (the symmetric update of the Sammon-mapping
//     page's "modified approach").
// Optionally every neighbour pair i<j is appended to an edge area so the
// merge never evaluates a distance again.
#include "device.h"
#include "internal.h"

namespace dbk {

// Minimum waves per SIMD the register allocator is asked to allow (1 = no
// constraint), chosen per width by measurement: the narrow widths fit 8
// waves (<= 64 VGPRs) and run faster there; the wide ones would spill.  The
// screen keeps one more value per column point (its norm) and its own
// masks, so it is given more registers.
constexpr int count_waves(int D, bool edges, bool screen) {
  return screen ? (D <= 2 ? 4 : D <= 4 ? 5 : D <= 16 ? 6 : 1)
                : (D <= 2 ? 5 : D <= 16 ? 8 : 1);
}

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

// Stage the pairs (row_out, col_out) of mask m, where row and col0 + lane
// are the positions in the tile; on a diagonal tile only the pairs with
// col > row (each unordered pair once, never (i,i)).  The caller has made
// room for every set bit.
template <bool DIAG>
__device__ __forceinline__ void stage_edges(uint64_t m, int64_t row,
                                            int64_t col0, int row_out,
                                            int col_out, uint2* stage,
                                            unsigned& fill) {
  if (DIAG) {
    const int64_t first = row - col0 + 1;
    if (first >= 64) return;
    if (first > 0) m &= ~0ull << first;
  }
  if (m == 0) return;
  if ((m >> lane_id()) & 1ull)
    stage[fill + bits_below(m)] = make_uint2((unsigned)row_out, (unsigned)col_out);
  fill += (unsigned)__popcll(m);
}

// One work item: `rows` consecutive row points against this wave's 64*P
// column points.
// With PRUNED, pts is the sorted copy and perm maps a sorted position to
// the original index: counts and captured pairs go to original indices.
//
// With SCREEN, most pairs are decided without the exact distance: a screen
// value v = |y|^2 - 2 x.y (fused multiply-adds from the column's norm,
// with the row pre-scaled by -2) is compared with two per-row thresholds
// that bracket the exact decision by a proven error bound (k_screen.hip).
// v <= lo: certainly a neighbour; v > hi: certainly not; in between the
// row's exact distances are evaluated on a rare, wave-uniform path, so the
// result is bit-identical to the exact pass.
template <int D, int P, bool DIAG, bool EDGES, bool PRUNED, bool SCREEN>
__device__ __forceinline__ void count_item(const float* __restrict__ pts,
                                           int64_t row0, int rows,
                                           int64_t colw, float eps2,
                                           unsigned* __restrict__ count,
                                           uint2* stage, unsigned& fill,
                                           const EdgeSink& sink,
                                           const int* __restrict__ perm,
                                           const float* __restrict__ boxes64,
                                           const float* __restrict__ boxes_w,
                                           const float* __restrict__ srow,
                                           const float* __restrict__ ncol) {
  constexpr int S = row_stride(D);
  constexpr int SR = screen_stride(D);
  const int lane = lane_id();
  float xc[P][D];
  float ny[SCREEN ? P : 1];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const float* cp = pts + (colw + p * 64 + lane) * S;
#pragma unroll
    for (int k = 0; k < D; ++k) xc[p][k] = cp[k];
    if (SCREEN) ny[p] = ncol[colw + p * 64 + lane];
  }
  // wait for the column loads here, once: otherwise a wait for each group
  // is re-issued on every row of the loops below
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int k = 0; k < D; ++k) asm volatile("" : "+v"(xc[p][k]));
    if (SCREEN) asm volatile("" : "+v"(ny[p]));
  }
  unsigned lc[P];
#pragma unroll
  for (int p = 0; p < P; ++p) lc[p] = 0;

  for (int rb = 0; rb < rows; rb += 64) {
    // pruned: skip 64 rows whose box is provably farther than eps from
    // every column point of this wave (no neighbour among them); only for
    // narrow points, where the test is a few scalar loads and the boxes
    // are tight
    if (PRUNED && D <= 16 &&
        boxes_apart<S>((const_float_ptr)(boxes64 + ((row0 + rb) >> 6) * 2 * S),
                       (const_float_ptr)(boxes_w + (colw / (64 * P)) * 2 * S),
                       eps2))
      continue;
    int rowv = 0;  // lane l: count of row rb+l over these columns
    // row addresses advance by a constant per row (the screen's exact path
    // recomputes its point address instead of carrying a second pointer)
    const float* next = SCREEN ? srow + (row0 + rb) * SR : pts + (row0 + rb) * S;
#pragma unroll 2
    for (int l = 0; l < 64; ++l) {
      const int64_t row = row0 + rb + l;
      const float* cur = next;
      next += SCREEN ? SR : S;
      // one value per column group: the exact distance, or the screen value
      float val[P];
      float lo = 0.f, thr = eps2;
      if (SCREEN) {
        // wave-uniform address: read through the constant address space so
        // the row lands in SGPRs via scalar loads
        const const_float_ptr sp = (const_float_ptr)cur;
        float a[D];
#pragma unroll
        for (int k = 0; k < D; ++k) a[k] = sp[k];
        lo = sp[D];
        thr = sp[D + 1];
#pragma unroll
        for (int p = 0; p < P; ++p) {
          float v = ny[p];
#pragma unroll
          for (int k = 0; k < D; ++k) v = __builtin_fmaf(a[k], xc[p][k], v);
          val[p] = v;
        }
      } else {
        const const_float_ptr rp = (const_float_ptr)cur;
        float xr[D];
#pragma unroll
        for (int k = 0; k < D; ++k) xr[k] = rp[k];
#pragma unroll
        for (int p = 0; p < P; ++p) val[p] = dist2<D>(xr, xc[p]);
      }
      // Most rows have no neighbour among these 64*P columns: one compare
      // of the lane's smallest value settles that for all P groups (min
      // returns the other operand for a NaN, so padding never hides a
      // real column), and only rows with a candidate pay for the masks,
      // the counters and the captured pairs, on one wave-uniform branch.
      float vmin = val[0];
#pragma unroll
      for (int p = 1; p < P; ++p) vmin = __builtin_fminf(vmin, val[p]);
      unsigned acc = 0;
      uint64_t m[P];
      if (ballot(vmin <= thr)) {
        if (SCREEN) {
          uint64_t amb = 0;
#pragma unroll
          for (int p = 0; p < P; ++p) {
            m[p] = ballot(val[p] <= lo);
            amb |= ballot(val[p] <= thr) & ~m[p];
          }
          if (amb) {
            // some pair of this row lies inside the bound: decide the
            // row's pairs with the exact distance
            const const_float_ptr rp = (const_float_ptr)(pts + row * S);
            float xr[D];
#pragma unroll
            for (int k = 0; k < D; ++k) xr[k] = rp[k];
#pragma unroll
            for (int p = 0; p < P; ++p)
              m[p] = ballot(dist2<D>(xr, xc[p]) <= eps2);
          }
        } else {
#pragma unroll
          for (int p = 0; p < P; ++p) m[p] = ballot(val[p] <= eps2);
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
          acc += (unsigned)__popcll(m[p]);
          if (!DIAG) lc[p] = add_lane_bit(lc[p], m[p]);
        }
        if (EDGES && acc != 0) {
          int lane_col = (int)(colw + lane);
          // recomputed here, on the rare path, instead of P live registers
          asm volatile("" : "+v"(lane_col));
          const int row_out = PRUNED ? ((const_int_ptr)perm)[row] : (int)row;
          // at most 8 column groups (512 pairs) staged per capacity check
#pragma unroll
          for (int g = 0; g < P; g += 8) {
            constexpr int G = P < 8 ? P : 8;
            unsigned want = 0;
#pragma unroll
            for (int p = g; p < g + G; ++p) want += (unsigned)__popcll(m[p]);
            if (fill + want > (unsigned)kEdgeStage) {
              flush_edges(stage, fill, sink);
              fill = 0;
            }
#pragma unroll
            for (int p = g; p < g + G; ++p) {
              const int col = lane_col + p * 64;
              stage_edges<DIAG>(m[p], row, colw + p * 64, row_out,
                                PRUNED ? perm[col] : col, stage, fill);
            }
          }
        }
      }
      rowv = write_lane(rowv, (int)acc, l);
    }
    if (rowv) {
      const int64_t r = row0 + rb + lane;
      atomicAdd(count + (PRUNED ? perm[r] : r), (unsigned)rowv);
    }
  }
  if (!DIAG) {
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (lc[p]) {
        const int64_t c = colw + p * 64 + lane;
        atomicAdd(count + (PRUNED ? perm[c] : c), lc[p]);
      }
  }
}

template <int D, bool EDGES, bool PRUNED, bool SCREEN>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(count_waves(D, EDGES, SCREEN), 8))) void k_count(
    const float* __restrict__ pts, int64_t nb, int chunks_log2, int rows,
    int64_t items, float eps2, unsigned* __restrict__ count,
    uint2* __restrict__ edges, unsigned long long cap,
    unsigned long long* __restrict__ counter,
    const uint2* __restrict__ tiles, const unsigned long long* n_tiles,
    unsigned long long tile_cap, const int* __restrict__ perm,
    const float* __restrict__ boxes64, const float* __restrict__ boxes_w,
    const float* __restrict__ srow, const float* __restrict__ ncol,
    int reverse) {
  constexpr int P = lane_points(D);
  constexpr int T = 256 * P;
  __shared__ uint2 stage_all[EDGES ? 4 * kEdgeStage : 1];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  uint2* stage = stage_all + (EDGES ? wave * kEdgeStage : 0);
  unsigned fill = 0;
  const EdgeSink sink{edges, cap, counter};
  // pruned: walk the kept block pairs (written by the previous kernel);
  // if the list overflowed, every block pair of the sorted points
  bool from_list = false;
  if (PRUNED) {
    const unsigned long long kept = *n_tiles;
    if (kept <= tile_cap) {
      items = (int64_t)kept << chunks_log2;
      from_list = true;
    }
  }
  for (int64_t step = blockIdx.x; step < items; step += gridDim.x) {
    // (a test mode walks the items in reverse: results must not change)
    const int64_t item = reverse ? items - 1 - step : step;
    const int64_t tile = item >> chunks_log2;
    const int c = (int)(item & ((1 << chunks_log2) - 1));
    int64_t I, J;
    if (PRUNED && from_list) {
      const uint2 tl = tiles[tile];
      I = tl.x;
      J = tl.y;
    } else {
      tile_coords(tile, nb, I, J);
    }
    const int64_t row0 = I * T + (int64_t)c * rows;
    const int64_t colw = J * T + (int64_t)wave * 64 * P;
    if (I == J)
      count_item<D, P, true, EDGES, PRUNED, SCREEN>(
          pts, row0, rows, colw, eps2, count, stage, fill, sink, perm, boxes64,
          boxes_w, srow, ncol);
    else
      count_item<D, P, false, EDGES, PRUNED, SCREEN>(
          pts, row0, rows, colw, eps2, count, stage, fill, sink, perm, boxes64,
          boxes_w, srow, ncol);
  }
  if (EDGES && fill) flush_edges(stage, fill, sink);
}

// ---- the screen on the matrix cores (widths 16 and up) ---------------------
// Same decisions as the screened pass above, with the screen value
//   v = n_y + sum_k (-2 x_k) y_k
// of a 16-row block against the wave's 64*P columns formed by
// v_mfma_f32_16x16x4_f32: the rows (pre-scaled by -2) are the A operand,
// the columns the B operand and the column norms the accumulator's start.
// Lane l supplies A[l%16][k] and B[k][l%16] for dims k of its lane group
// q = l/16 (dims q*D/4 .. q*D/4 + D/4 - 1, one per instruction) and holds
// the results of rows 4q + r (r = 0..3) against column l%16.  Every row
// and column value arrives through vector loads: no scalar load per row.
// The thresholds of this path are widened for the matrix unit's
// unspecified summation order, rounding and subnormal handling
// (k_screen.hip); undecided pairs take the exact distance, per lane.
typedef float mf4 __attribute__((ext_vector_type(4)));

// Sum over each 16-lane row of the wave; every lane gets its row's total.
__device__ __forceinline__ unsigned row16_sum(unsigned v) {
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, true);   // quad_perm 1,0,3,2
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, true);   // quad_perm 2,3,0,1
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, true);  // row_half_mirror
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, true);  // row_mirror
  return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ unsigned wave_incl_sum(unsigned v) {
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);  // row_shr:8
  const unsigned t0 = (unsigned)__builtin_amdgcn_readlane((int)v, 15);
  const unsigned t1 = (unsigned)__builtin_amdgcn_readlane((int)v, 31);
  const unsigned t2 = (unsigned)__builtin_amdgcn_readlane((int)v, 47);
  const int q = lane_id() >> 4;
  return v + (q >= 1 ? t0 : 0u) + (q >= 2 ? t1 : 0u) + (q >= 3 ? t2 : 0u);
}

// The fixed direct distance of one pair, computed by the whole wave: lane k
// forms fl(fl(x_k - y_k)^2), then the squares are added in ascending k.
// The result is the same in every lane.
template <int D>
__device__ __forceinline__ bool wave_exact_within(const float* __restrict__ xp,
                                                  const float* __restrict__ yp,
                                                  float eps2) {
  const int k = lane_id();
  float sq = 0.f;
  if (k < D) {
    const float t = xp[k] - yp[k];
    sq = t * t;
  }
  float d2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sq), 0));
#pragma unroll
  for (int kk = 1; kk < D; ++kk)
    d2 = d2 + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sq), kk));
  return d2 <= eps2;
}

// waves per SIMD the register budget is held to (the widths listed fit
// three without spilling)
constexpr int mfma_waves(int D, bool edges) {
  return D == 24 || D == 32 ? 3 : 2;
}

template <int D, bool EDGES, bool PRUNED>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(mfma_waves(D, EDGES), 8))) void k_count_mfma(
    const float* __restrict__ pts, int64_t nb, int chunks_log2, int rows,
    int64_t items, float eps2, unsigned* __restrict__ count,
    uint2* __restrict__ edges, unsigned long long cap,
    unsigned long long* __restrict__ counter,
    const uint2* __restrict__ tiles, const unsigned long long* n_tiles,
    unsigned long long tile_cap, const int* __restrict__ perm,
    const float* __restrict__ srow, const float* __restrict__ ncol,
    int reverse) {
  constexpr int P = lane_points(D);
  constexpr int T = 256 * P;
  constexpr int S = row_stride(D);
  constexpr int SR = screen_stride(D);
  constexpr int KQ = D / 4;    // dims per lane group, one per instruction
  constexpr int NG = 4 * P;    // groups of 16 columns per wave
  static_assert(D % 4 == 0 && NG * 16 == 64 * P && NG <= 8, "matrix-core layout");
  // bits 4g + r of a lane's pair mask that belong to row r
  constexpr unsigned kRowBits = NG == 8 ? 0x11111111u : 0x1111u;
  __shared__ uint2 stage_all[EDGES ? 4 * kEdgeStage : 1];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = lane_id();
  const int l16 = lane & 15, q = lane >> 4;
  uint2* stage = stage_all + (EDGES ? wave * kEdgeStage : 0);
  unsigned fill = 0;
  const EdgeSink sink{edges, cap, counter};
  bool from_list = false;
  if (PRUNED) {
    const unsigned long long kept = *n_tiles;
    if (kept <= tile_cap) {
      items = (int64_t)kept << chunks_log2;
      from_list = true;
    }
  }
  for (int64_t step = blockIdx.x; step < items; step += gridDim.x) {
    const int64_t item = reverse ? items - 1 - step : step;
    const int64_t tile = item >> chunks_log2;
    const int c = (int)(item & ((1 << chunks_log2) - 1));
    int64_t I, J;
    if (PRUNED && from_list) {
      const uint2 tl = tiles[tile];
      I = tl.x;
      J = tl.y;
    } else {
      tile_coords(tile, nb, I, J);
    }
    const bool diag = I == J;
    const int64_t row0 = I * T + (int64_t)c * rows;
    const int64_t colw = J * T + (int64_t)wave * 64 * P;
    // this lane's column of each group: coordinates of its lane group's
    // dims (B operand), norm, counter
    float bq[NG][KQ];
    float ny[NG];
    unsigned lc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int64_t col = colw + g * 16 + l16;
      const float* cp = pts + col * S + q * KQ;
#pragma unroll
      for (int k = 0; k < KQ; ++k) bq[g][k] = cp[k];
      ny[g] = ncol[col];
      lc[g] = 0;
    }
    unsigned rowv = 0;  // lane l: count of row (64-row window) + l
    // the A operand and the thresholds of the next 16-row block are
    // requested while the current block is on the matrix cores
    float a_next[KQ];
    float2 th_next[4];
    {
      const float* ap = srow + (row0 + l16) * SR + q * KQ;
#pragma unroll
      for (int k = 0; k < KQ; ++k) a_next[k] = ap[k];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        th_next[r] = *(const float2*)(srow + (row0 + 4 * q + r) * SR + D);
    }
    for (int rb = 0; rb < rows; rb += 16) {
      if ((rb & 63) == 0 && rb > 0) {
        if (rowv) {
          const int64_t i = row0 + rb - 64 + lane;
          atomicAdd(count + (PRUNED ? perm[i] : i), rowv);
        }
        rowv = 0;
      }
      const int64_t rbase = row0 + rb;
      // A operand: row rbase + l16, dims of lane group q; thresholds (lo,
      // hi) of this lane's rows rbase + 4q + r
      float a[KQ];
      float2 th[4];
#pragma unroll
      for (int k = 0; k < KQ; ++k) a[k] = a_next[k];
#pragma unroll
      for (int r = 0; r < 4; ++r) th[r] = th_next[r];
      if (rb + 16 < rows) {
        const float* ap = srow + (rbase + 16 + l16) * SR + q * KQ;
#pragma unroll
        for (int k = 0; k < KQ; ++k) a_next[k] = ap[k];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          th_next[r] = *(const float2*)(srow + (rbase + 16 + 4 * q + r) * SR + D);
      }
      mf4 acc[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) acc[g] = mf4{ny[g], ny[g], ny[g], ny[g]};
#pragma unroll
      for (int k = 0; k < KQ; ++k)
#pragma unroll
        for (int g = 0; g < NG; ++g)
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k], bq[g][k], acc[g],
                                                        0, 0, 0);
      // any candidate neighbour in the block?  (min skips NaN padding)
      float tmin = acc[0][0] - th[0].y;
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          tmin = __builtin_fminf(tmin, acc[g][r] - th[r].y);
      if (!ballot(tmin <= 0.f)) continue;
      // per lane: bit 4g+r of `sure` / `maybe` for pair (row 4q+r, col g)
      unsigned sure = 0, maybe = 0;
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sure |= (acc[g][r] <= th[r].x ? 1u : 0u) << (4 * g + r);
          maybe |= (acc[g][r] <= th[r].y ? 1u : 0u) << (4 * g + r);
        }
      unsigned flag = sure;
      unsigned amb = maybe & ~sure;
      uint64_t pend = ballot(amb != 0);
      if (__popcll(pend) > 8) {
        // many undecided pairs (the screen is off for this set, or the
        // radius is at a scale the screen cannot resolve): per lane
        for (unsigned w = amb; w != 0; w &= w - 1) {
          const int b = __builtin_ctz(w);
          const int g = b >> 2, r = b & 3;
          const float* xp = pts + (rbase + 4 * q + r) * S;
          const float* yp = pts + (colw + g * 16 + l16) * S;
          float t0 = xp[0] - yp[0];
          float d2 = t0 * t0;
          for (int k = 1; k < D; ++k) {
            const float t = xp[k] - yp[k];
            const float q2 = t * t;
            d2 = d2 + q2;
          }
          if (d2 <= eps2) flag |= 1u << b;
        }
      } else {
        // a few: one pair at a time across the wave
        while (pend) {
          const int src = (int)__builtin_ctzll(pend);
          const unsigned bits = (unsigned)__builtin_amdgcn_readlane((int)amb, src);
          const int b = __builtin_ctz(bits);
          const int64_t i = rbase + 4 * (src >> 4) + (b & 3);
          const int64_t j = colw + (b >> 2) * 16 + (src & 15);
          const bool in = wave_exact_within<D>(pts + i * S, pts + j * S, eps2);
          if (lane == src) {
            if (in) flag |= 1u << b;
            amb &= amb - 1;
          }
          if ((bits & (bits - 1)) == 0) pend &= pend - 1;
        }
      }
      if (!diag) {
        // the row side only on a diagonal tile, which holds both orders
#pragma unroll
        for (int g = 0; g < NG; ++g)
          lc[g] += (unsigned)__builtin_popcount((flag >> (4 * g)) & 15u);
      }
      // row counts: this lane's pairs of rows 4q + r, 8 bits per r, summed
      // over the 16 lanes of the group, then added by the lane of rowv
      // that holds the row (rows rbase - (rb % 64) + lane)
      {
        unsigned pk = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pk |= (unsigned)__builtin_popcount(flag & (kRowBits << r)) << (8 * r);
        pk = row16_sum(pk);
        const unsigned got = (unsigned)__builtin_amdgcn_ds_bpermute(
            (16 * ((lane & 15) >> 2)) << 2, (int)pk);
        if ((lane >> 4) == ((rb >> 4) & 3)) rowv += (got >> (8 * (lane & 3))) & 255u;
      }
      if (EDGES) {
        unsigned e = flag;
        if (diag) {
          // pairs with column > row (in block order) only: each unordered
          // pair once, never (i, i)
          unsigned keep = 0;
#pragma unroll
          for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              keep |= (colw + g * 16 + l16 > rbase + 4 * q + r ? 1u : 0u)
                      << (4 * g + r);
          e &= keep;
        }
        const unsigned n_e = (unsigned)__builtin_popcount(e);
        const unsigned incl = wave_incl_sum(n_e);
        const unsigned total = (unsigned)__builtin_amdgcn_readlane((int)incl, 63);
        if (total) {
          if (fill + total > (unsigned)kEdgeStage) {
            if (fill) flush_edges(stage, fill, sink);
            fill = 0;
          }
          if (total <= (unsigned)kEdgeStage) {
            unsigned pos = fill + incl - n_e;
            for (unsigned w = e; w != 0; w &= w - 1) {
              const int b = __builtin_ctz(w);
              const int64_t i = rbase + 4 * q + (b & 3);
              const int64_t j = colw + (b >> 2) * 16 + l16;
              stage[pos++] = make_uint2((unsigned)(PRUNED ? perm[i] : i),
                                        (unsigned)(PRUNED ? perm[j] : j));
            }
            fill += total;
          } else {
            // more than the stage holds: reserve the slots and write them
            unsigned long long base = 0;
            if (lane == 0)
              base = atomicAdd(sink.counter, (unsigned long long)total);
            base = uniform_u64(base) + (incl - n_e);
            for (unsigned w = e; w != 0; w &= w - 1) {
              const int b = __builtin_ctz(w);
              const int64_t i = rbase + 4 * q + (b & 3);
              const int64_t j = colw + (b >> 2) * 16 + l16;
              if (base < sink.cap)
                sink.edges[base] = make_uint2((unsigned)(PRUNED ? perm[i] : i),
                                              (unsigned)(PRUNED ? perm[j] : j));
              ++base;
            }
          }
        }
      }
    }
    if (rowv) {
      const int64_t i = row0 + rows - 64 + lane;
      atomicAdd(count + (PRUNED ? perm[i] : i), rowv);
    }
    if (!diag) {
      // column counters: sum the four lane groups of each column
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        unsigned t = lc[g];
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        if (q == 0 && t) {
          const int64_t j = colw + g * 16 + l16;
          atomicAdd(count + (PRUNED ? perm[j] : j), t);
        }
      }
    }
  }
  if (EDGES && fill) flush_edges(stage, fill, sink);
}

template <int D>
static hipError_t launch_count_mfma_d(const Layout& L, float eps2, bool edges,
                                      bool pruned, bool reverse, hipStream_t s,
                                      int64_t* pairs) {
  constexpr int P = lane_points(D);
  constexpr int T = 256 * P;
  const int64_t nb = L.n_pad / T;
  const int64_t tiles = nb * (nb + 1) / 2;
  int rows = pruned && kRowsPerItem < T ? kRowsPerItem : T;
  while (rows > 64 && tiles * (T / rows) < 4096) rows >>= 1;
  const int chunks = T / rows;
  int chunks_log2 = 0;
  while ((1 << chunks_log2) < chunks) ++chunks_log2;
  const int64_t items = tiles * chunks;
  const int64_t max_grid = pruned ? 16384 : kMaxGrid;
  const unsigned grid = (unsigned)(items < max_grid ? items : max_grid);
  const float* pts = pruned ? L.sorted_pts : L.pts;
#define DBK_MFMA_ARGS                                                        \
  pts, nb, chunks_log2, rows, items, eps2, L.count,                          \
      edges ? L.edges : nullptr, edges ? L.edge_cap : 0ull,                  \
      &L.status->n_edges, L.tiles, &L.status->n_tiles, L.tile_cap, L.perm,   \
      L.srow, L.ncol, reverse ? 1 : 0
  if (edges && pruned)
    k_count_mfma<D, true, true><<<grid, kThreads, 0, s>>>(DBK_MFMA_ARGS);
  else if (edges)
    k_count_mfma<D, true, false><<<grid, kThreads, 0, s>>>(DBK_MFMA_ARGS);
  else if (pruned)
    k_count_mfma<D, false, true><<<grid, kThreads, 0, s>>>(DBK_MFMA_ARGS);
  else
    k_count_mfma<D, false, false><<<grid, kThreads, 0, s>>>(DBK_MFMA_ARGS);
#undef DBK_MFMA_ARGS
  if (pairs) *pairs = L.n_pad * L.n_pad;
  return hipGetLastError();
}

template <int D>
static hipError_t launch_count_d(const Layout& L, float eps2, bool edges,
                                 bool pruned, bool screen, bool reverse,
                                 hipStream_t s, int64_t* pairs) {
  constexpr int P = lane_points(D);
  constexpr int T = 256 * P;
  const int64_t nb = L.n_pad / T;
  const int64_t tiles = nb * (nb + 1) / 2;
  // rows per work item: a whole block of T rows, so each column block is
  // loaded once per tile (a pruned launch keeps only some tiles and splits
  // them into items of up to kRowsPerItem rows for parallelism); fewer,
  // down to one wave's 64, while the full triangle would give under 4096
  // work items
  int rows = pruned && kRowsPerItem < T ? kRowsPerItem : T;
  while (rows > 64 && tiles * (T / rows) < 4096) rows >>= 1;
  const int chunks = T / rows;  // both powers of two
  int chunks_log2 = 0;
  while ((1 << chunks_log2) < chunks) ++chunks_log2;
  const int64_t items = tiles * chunks;
  const int64_t max_grid = pruned ? 16384 : kMaxGrid;
  const unsigned grid = (unsigned)(items < max_grid ? items : max_grid);
  const float* pts = pruned ? L.sorted_pts : L.pts;
  const unsigned long long* n_tiles = &L.status->n_tiles;
#define DBK_COUNT_ARGS                                                      \
  pts, nb, chunks_log2, rows, items, eps2, L.count,                         \
      edges ? L.edges : nullptr, edges ? L.edge_cap : 0ull,                 \
      &L.status->n_edges, L.tiles, n_tiles, L.tile_cap, L.perm, L.boxes64,  \
      L.boxes_w, L.srow, L.ncol, reverse ? 1 : 0
#define DBK_LAUNCH(E, PR, SC) \
  k_count<D, E, PR, SC><<<grid, kThreads, 0, s>>>(DBK_COUNT_ARGS)
  if (screen) {
    if (edges && pruned) DBK_LAUNCH(true, true, true);
    else if (edges) DBK_LAUNCH(true, false, true);
    else if (pruned) DBK_LAUNCH(false, true, true);
    else DBK_LAUNCH(false, false, true);
  } else {
    if (edges && pruned) DBK_LAUNCH(true, true, false);
    else if (edges) DBK_LAUNCH(true, false, false);
    else if (pruned) DBK_LAUNCH(false, true, false);
    else DBK_LAUNCH(false, false, false);
  }
#undef DBK_LAUNCH
#undef DBK_COUNT_ARGS
  if (pairs) *pairs = L.n_pad * L.n_pad;
  return hipGetLastError();
}

bool screen_on_matrix_cores(int D) { return D >= 16; }

hipError_t launch_count(const Layout& L, float eps2, bool edges, bool pruned,
                        bool screen, bool reverse, hipStream_t s,
                        int64_t* pairs) {
  if (screen && screen_on_matrix_cores(L.D)) {
    switch (L.D) {
      case 16: return launch_count_mfma_d<16>(L, eps2, edges, pruned, reverse, s, pairs);
      case 24: return launch_count_mfma_d<24>(L, eps2, edges, pruned, reverse, s, pairs);
      case 32: return launch_count_mfma_d<32>(L, eps2, edges, pruned, reverse, s, pairs);
      case 48: return launch_count_mfma_d<48>(L, eps2, edges, pruned, reverse, s, pairs);
      case 64: return launch_count_mfma_d<64>(L, eps2, edges, pruned, reverse, s, pairs);
      default: return hipErrorInvalidValue;
    }
  }
  switch (L.D) {
#define DBK_CASE(DD)                                                        \
  case DD:                                                                  \
    return launch_count_d<DD>(L, eps2, edges, pruned, screen, reverse, s,   \
                              pairs);
    DBK_CASE(1) DBK_CASE(2) DBK_CASE(3) DBK_CASE(4) DBK_CASE(6) DBK_CASE(8)
    DBK_CASE(12) DBK_CASE(16) DBK_CASE(24) DBK_CASE(32) DBK_CASE(48)
    DBK_CASE(64)
#undef DBK_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dbk

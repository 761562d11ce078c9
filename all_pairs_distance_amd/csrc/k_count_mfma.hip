// Screened neighbour-count pass on the matrix cores (widths 16 to 64).
//
// Same work items, tiles, counts and captured pairs as the count pass in
// k_count.hip, and the same decisions as its screened mode; only the
// screen value is formed differently (see below), with the widened
// thresholds of k_screen.hip.
#include "count_common.h"
#include "device.h"
#include "internal.h"

namespace dbk {

// The screen value
//   v = n_y + sum_k (-2 x_k) y_k
// of a 16-row block against the wave's 64*P columns formed by
// v_mfma_f32_16x16x4_f32: the rows (pre-scaled by -2) are the A operand,
// the columns the B operand; the column norms are added to the products.
// Lane l supplies A[l%16][k] and B[k][l%16] for dims k of its lane group
// q = l/16 (dims q*D/4 .. q*D/4 + D/4 - 1, one per instruction) and holds
// the results of rows 4q + r (r = 0..3) against column l%16.  Rows come
// through LDS (64 at a time, copied straight from memory into LDS and
// shared by the work-group's four waves), columns through vector loads:
// no scalar load per row.
// The thresholds of this path are widened for the matrix unit's
// unspecified summation order, rounding and subnormal handling
// (k_screen.hip).  Undecided pairs take the exact distance (or the exact
// hoisted-norm form): one pair at a time across the wave when a block
// has a few, per lane when it has many.
typedef float mf4 __attribute__((ext_vector_type(4)));

// Sum over each 16-lane row of the wave; every lane gets its row's total.
__device__ __forceinline__ unsigned row16_sum(unsigned v) {
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, true);   // quad_perm 1,0,3,2
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, true);   // quad_perm 2,3,0,1
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, true);  // row_half_mirror
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, true);  // row_mirror
  return v;
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

// The hoisted-norm form of one pair, by the whole wave: lane k forms the
// rounded product (2 x_k) y_k, the products are added in ascending k from
// the lanes in turn, then (tx + ty) minus that sum.  Same value in every
// lane.
template <int D>
__device__ __forceinline__ bool wave_expanded_within(
    const float* __restrict__ xp, const float* __restrict__ yp, float tx,
    float ty, float eps2) {
  const int k = lane_id();
  float pr = 0.f;
  if (k < D) pr = (2.f * xp[k]) * yp[k];
  float inner = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pr), 0));
#pragma unroll
  for (int kk = 1; kk < D; ++kk)
    inner = inner + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pr), kk));
  const float s = tx + ty;
  return s - inner <= eps2;
}

// Copy n4 16-byte words from global memory (src) to LDS (dst) with the
// work-group's 256 threads, straight into LDS (no registers): word
// t + 256 j of the copy is lane t % 64 of wave t / 64's j-th load, which
// writes its 16 bytes at the wave's LDS base + 16 * lane.  Completion is
// awaited by the caller (vmcnt, then a barrier).
__device__ __forceinline__ void stage_to_lds(const float* __restrict__ src,
                                             float* dst, int n4) {
  const int w = (int)(threadIdx.x >> 6), lane = lane_id();
  for (int j = 0; j * 256 < n4; ++j) {
    const int base = j * 256 + w * 64;
    if (base + lane < n4)
      __builtin_amdgcn_global_load_lds(
          (const void*)(src + (int64_t)(base + lane) * 4),
          (__attribute__((address_space(3))) void*)(dst + base * 4), 16, 0, 0);
  }
}

// waves per SIMD the register budget is held to: three from width 24
constexpr int mfma_waves(int D, bool edges) {
  return D >= 24 ? 3 : 2;
}

// (s, m) = (2 s + [v <= lo], 2 m + [v <= hi]) per lane: two compares, then
// two adds with the compare masks as carry-in; the second compare and the
// s_nop give the first mask's read its two wait states, the s_nop and the
// first add the second's.
__device__ __forceinline__ void shift_in_le2(unsigned& s, unsigned& m, float v,
                                             float lo, float hi) {
  uint64_t t;
  asm("v_cmp_le_f32_e32 vcc, %3, %4\n\t"
      "v_cmp_le_f32_e64 %2, %3, %5\n\t"
      "s_nop 0\n\t"
      "v_addc_co_u32_e32 %0, vcc, %0, %0, vcc\n\t"
      "v_addc_co_u32_e64 %1, %2, %1, %1, %2"
      : "+v"(s), "+v"(m), "=&s"(t)
      : "v"(v), "v"(lo), "v"(hi)
      : "vcc");
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
    const float* __restrict__ boxes64, const float* __restrict__ boxes_w,
    float box_thr, const float* __restrict__ srow,
    const float* __restrict__ ncol, const float* __restrict__ nexp,
    WalkArgs walk, const unsigned* __restrict__ nonfinite) {
  constexpr int P = lane_points(D);
  constexpr int T = 256 * P;
  constexpr int S = row_stride(D);
  constexpr int SR = screen_stride(D);
  constexpr int KQ = D / 4;    // dims per lane group, one per instruction
  constexpr int NG = 4 * P;    // groups of 16 columns per wave
  static_assert(D % 4 == 0 && NG * 16 == 64 * P && NG <= 8, "matrix-core layout");
  // rows (-2x, lo, hi) reach the waves through LDS, 64 at a time, double
  // buffered and shared by the work-group's four waves (same rows,
  // different columns)
  constexpr int kChunk4 = 16 * SR;   // 16-byte words per 64 rows
  __shared__ __attribute__((aligned(16))) float rows_lds[2 * 64 * SR];
  // bits 4g + r of a lane's pair mask that belong to row r
  constexpr unsigned kRowBits = NG == 8 ? 0x11111111u : 0x1111u;
  __shared__ uint2 stage_all[EDGES ? 4 * kEdgeStage : 1];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = lane_id();
  const int l16 = lane & 15, q = lane >> 4;
  uint2* stage = stage_all + (EDGES ? wave * kEdgeStage : 0);
  unsigned fill = 0;
  const EdgeSink sink{edges, cap, counter};
  // a non-finite input coordinate fails the fit: skip the pass
  if (*nonfinite) return;
  bool from_list = false;
  if (PRUNED) {
    const unsigned long long kept = *n_tiles;
    if (kept <= tile_cap) {
      items = (int64_t)kept << chunks_log2;
      from_list = true;
      walk_refit(items, walk.mul, walk.add);
    }
  }
  const bool blocked = !from_list && nb >= kBlockedTileRows;
  for (int64_t step = blockIdx.x; step < items; step += gridDim.x) {
    const int64_t item = walk_item(
        blocked ? xcd_item(step, items) : step, items, walk.mul, walk.add);
    const int64_t tile = item >> chunks_log2;
    const int c = (int)(item & ((1 << chunks_log2) - 1));
    int64_t I, J;
    if (PRUNED && from_list) {
      const uint2 tl = tiles[tile];
      I = tl.x;
      J = tl.y;
    } else {
      if (blocked) tile_coords_blocked(tile, nb, I, J);
      else tile_coords(tile, nb, I, J);
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
    // every wave is done with the previous item's rows before the first
    // chunk of this one lands
    __syncthreads();
    stage_to_lds(srow + row0 * SR, rows_lds, kChunk4);
    bool chunk_apart = false;
    for (int rb = 0; rb < rows; rb += 16) {
      if ((rb & 63) == 0) {
        if (rb > 0) {
          if (rowv) {
            const int64_t i = row0 + rb - 64 + lane;
            atomicAdd(count + (PRUNED ? perm[i] : i), rowv);
          }
          rowv = 0;
        }
        // this chunk has landed (and every wave is done with the buffer
        // the next chunk goes to); start the next chunk
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (rb + 64 < rows)
          stage_to_lds(srow + (row0 + rb + 64) * SR,
                       rows_lds + (((rb >> 6) + 1) & 1) * 64 * SR, kChunk4);
        // pruned: these 64 rows' box provably farther than eps from this
        // wave's columns (the barrier above is still every wave's)
        if (PRUNED)
          chunk_apart = wave_boxes_apart<S>(
              boxes64 + ((row0 + rb) >> 6) * 2 * S,
              boxes_w + (colw / (64 * P)) * 2 * S, box_thr);
      }
      if (PRUNED && chunk_apart) continue;
      const int64_t rbase = row0 + rb;
      const float* cur = rows_lds + ((rb >> 6) & 1) * 64 * SR + (rb & 63) * SR;
      // A operand: row rbase + l16, dims of lane group q; thresholds (lo,
      // hi) of this lane's rows rbase + 4q + r
      float a[KQ];
      float2 th[4];
      {
        const float* ap = cur + l16 * SR + q * KQ;
#pragma unroll
        for (int k = 0; k < KQ; ++k) a[k] = ap[k];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          th[r] = *(const float2*)(cur + (4 * q + r) * SR + D);
      }
      mf4 acc[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) acc[g] = mf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KQ; ++k)
#pragma unroll
        for (int g = 0; g < NG; ++g)
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k], bq[g][k], acc[g],
                                                        0, 0, 0);
      // the column norm joins last: one more rounded addition, an order
      // the bound allows (any order of the D + 1 terms); starting the
      // products from zero spares the registers of a replicated norm
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[g][r] = acc[g][r] + ny[g];
      // any candidate neighbour in the block?  The smallest value of each
      // row minus its upper threshold (rounding is monotone, so this is
      // the smallest of the differences; min skips NaN padding).
      float tmin = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = acc[0][r];
#pragma unroll
        for (int g = 1; g < NG; ++g) m = __builtin_fminf(m, acc[g][r]);
        m = m - th[r].y;
        tmin = r == 0 ? m : __builtin_fminf(tmin, m);
      }
      if (!ballot(tmin <= 0.f)) continue;
      // per lane: bit 4g+r of `sure` / `maybe` for pair (row 4q+r, col g)
      // (built from the top bit down: each step doubles the word and adds
      // the compare's lane bit as the carry)
      unsigned sure = 0, maybe = 0;
#pragma unroll
      for (int g = NG - 1; g >= 0; --g)
#pragma unroll
        for (int r = 3; r >= 0; --r)
          shift_in_le2(sure, maybe, acc[g][r], th[r].x, th[r].y);
      unsigned flag = sure;
      unsigned amb = maybe & ~sure;
      uint64_t pend = ballot(amb != 0);
      if (__popcll(pend) > 8) {
        // many undecided pairs (the screen is off for this set, or the
        // radius is at a scale the screen cannot resolve): per lane
        for (unsigned w = amb; w != 0; w &= w - 1) {
          const int b = __builtin_ctz(w);
          const int g = b >> 2, r = b & 3;
          const int64_t i = rbase + 4 * q + r, j = colw + g * 16 + l16;
          const float* xp = pts + i * S;
          const float* yp = pts + j * S;
          float v;
          if (!PRUNED && nexp != nullptr) {
            float inner = (2.f * xp[0]) * yp[0];
            for (int k = 1; k < D; ++k) {
              const float pr = (2.f * xp[k]) * yp[k];
              inner = inner + pr;
            }
            const float s = nexp[i] + nexp[j];
            v = s - inner;
          } else {
            float t0 = xp[0] - yp[0];
            v = t0 * t0;
            for (int k = 1; k < D; ++k) {
              const float t = xp[k] - yp[k];
              const float q2 = t * t;
              v = v + q2;
            }
          }
          if (v <= eps2) flag |= 1u << b;
        }
      } else {
        // a few: one pair at a time across the wave
        while (pend) {
          const int src = (int)__builtin_ctzll(pend);
          const unsigned bits = (unsigned)__builtin_amdgcn_readlane((int)amb, src);
          const int b = __builtin_ctz(bits);
          const int64_t i = rbase + 4 * (src >> 4) + (b & 3);
          const int64_t j = colw + (b >> 2) * 16 + (src & 15);
          const bool in =
              (!PRUNED && nexp != nullptr)
                  ? wave_expanded_within<D>(pts + i * S, pts + j * S,
                                            ((const_float_ptr)nexp)[i],
                                            ((const_float_ptr)nexp)[j], eps2)
                  : wave_exact_within<D>(pts + i * S, pts + j * S, eps2);
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
                                      bool pruned, Walk walk, hipStream_t s,
                                      int64_t* pairs) {
  const CountPlan c = plan_count(L.n_pad, 256 * lane_points(D), pruned);
  const float* pts = pruned ? L.sorted_pts : L.pts;
  constexpr int S = row_stride(D);
#define DBK_MFMA_ARGS                                                        \
  pts, c.nb, c.chunks_log2, c.rows, c.items, eps2, L.count,                  \
      edges ? L.edges : nullptr, edges ? L.edge_cap : 0ull,                  \
      &L.status->n_edges, L.tiles, &L.status->n_tiles, L.tile_cap, L.perm,   \
      L.boxes64, L.boxes_w, box_gap_threshold(eps2, S), L.srow, L.ncol,      \
      L.expanded ? L.nexp : nullptr, walk_args(walk, c.items), &L.status->nonfinite
  if (edges && pruned)
    k_count_mfma<D, true, true><<<c.grid, kThreads, 0, s>>>(DBK_MFMA_ARGS);
  else if (edges)
    k_count_mfma<D, true, false><<<c.grid, kThreads, 0, s>>>(DBK_MFMA_ARGS);
  else if (pruned)
    k_count_mfma<D, false, true><<<c.grid, kThreads, 0, s>>>(DBK_MFMA_ARGS);
  else
    k_count_mfma<D, false, false><<<c.grid, kThreads, 0, s>>>(DBK_MFMA_ARGS);
#undef DBK_MFMA_ARGS
  if (pairs) *pairs = L.n_pad * L.n_pad;
  return hipGetLastError();
}

hipError_t launch_count_mfma(const Layout& L, float eps2, bool edges,
                             bool pruned, Walk walk, hipStream_t s,
                             int64_t* pairs) {
  switch (L.D) {
    case 16: return launch_count_mfma_d<16>(L, eps2, edges, pruned, walk, s, pairs);
    case 24: return launch_count_mfma_d<24>(L, eps2, edges, pruned, walk, s, pairs);
    case 32: return launch_count_mfma_d<32>(L, eps2, edges, pruned, walk, s, pairs);
    case 48: return launch_count_mfma_d<48>(L, eps2, edges, pruned, walk, s, pairs);
    case 64: return launch_count_mfma_d<64>(L, eps2, edges, pruned, walk, s, pairs);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dbk

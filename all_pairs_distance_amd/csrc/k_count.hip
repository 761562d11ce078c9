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
//     page's "modified approach"); with 16 column points per lane (d <= 2)
//     each lane builds its own pattern of the row's pairs from signs, and
//     the row counts are summed through LDS.
// Optionally every neighbour pair i<j is appended to an edge area so the
// merge never evaluates a distance again.
#include "count_common.h"
#include "device.h"
#include "internal.h"

namespace dbk {

// Minimum waves per SIMD the register allocator is asked to allow (1 = no
// constraint), chosen per width by measurement: the narrow widths fit 8
// waves (<= 64 VGPRs) and run faster there; widths 48 and 64 fit 6 (80
// VGPRs; at 64, 48 bytes of spills in the per-item setup, none in the row
// loop): 262k x 64 count 102.0 -> 101.5 ms, pruned 19.3 -> 18.2 ms against
// the 5 waves the allocator picks unasked.  The screen keeps one more
// value per column point (its norm) and its own masks, so it is given
// more registers: 5 waves, which its LDS (rows and pair stage, 28.5 KB per
// work-group at width 8) allows anyway; asking for 6 left the allocator
// at 4 (200k x 8 screened count 5.03 -> 4.80 ms with 5), and 7 or more
// spill in the row loop.  Widths up to 2 (16 column points per lane,
// 117-124 VGPRs) take 4 waves: with 5 they spilled 18-25 registers, and
// 4 ran 1% faster on 50k x 2 and 3-7% on sparser 2-d sets.
constexpr int count_waves(int D, bool screen) {
  return screen ? (D <= 2 ? 4 : D <= 16 ? 5 : 1)
                : (D <= 2 ? 4 : D <= 16 ? 8 : D >= 48 ? 6 : 1);
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
  // the mask itself becomes the exec mask of the store (no per-lane test)
  if (__builtin_amdgcn_inverse_ballot_w64(m))
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
// row's exact distances (or, with a norm table, the exact hoisted-norm
// form) are evaluated on a rare, wave-uniform path, so the result is
// bit-identical to the exact pass (or to that form).  Its row records go
// through the wave's LDS area, 64 rows at a time, read back as broadcasts.
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
                                           float box_thr,
                                           const float* __restrict__ srow,
                                           const float* __restrict__ ncol,
                                           const float* __restrict__ nexp,
                                           float* rows_lds, unsigned* rowc,
                                           int64_t n_real) {
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
  // Narrow points (16 groups per lane), where most rows have a pair: the
  // row's pairs become one pattern per lane (bit P-1-p: group p), taken
  // from the signs of val - e2n, e2n the float just above eps2.  val <=
  // eps2 exactly when val - e2n < 0 (a rounded difference has the sign of
  // the exact one and is +0 only for equal operands; subnormals are
  // kept), so a group costs a full-rate subtraction and a bit shift, where
  // a compare and a carry-in add read a mask from scalar registers at half
  // rate.  Padding columns (NaN, sign unspecified) are masked out; padding
  // rows never get here (a NaN row has no candidate).  No float lies above
  // +inf: with eps2 = +inf the pattern comes from ballots.  The row counts
  // go through LDS (a byte per row and lane, summed every 64 rows) and the
  // column counts through 8-bit counters, four to a register, moved into
  // 16-bit counters, two to a register, every 64 rows (at most 64 and
  // 4096 a counter).
  constexpr bool SIGNS = !SCREEN && P >= 16;
  constexpr int NLC = SIGNS ? 1 : P;
  unsigned lc[NLC];
#pragma unroll
  for (int p = 0; p < NLC; ++p) lc[p] = 0;
  unsigned lcw[SIGNS ? P / 2 : 1];  // half h of lcw[k]: pattern bit 2k + h
  unsigned lcb[SIGNS ? P / 4 : 1];  // byte b of lcb[g]: pattern bit 4g + b
  unsigned colvalid = 0;
  bool signs = false;
  float e2n = 0.f;
  if constexpr (SIGNS) {
#pragma unroll
    for (int k = 0; k < P / 2; ++k) lcw[k] = 0u;
#pragma unroll
    for (int p = 0; p < P; ++p)
      colvalid = (colvalid << 1) | (colw + p * 64 + lane < n_real ? 1u : 0u);
    signs = __float_as_uint(eps2) < 0x7f800000u;
    e2n = __uint_as_float(__float_as_uint(eps2) + 1u);
  }

  for (int rb = 0; rb < rows; rb += 64) {
    // pruned: skip 64 rows whose box is provably farther than eps from
    // every column point of this wave (no neighbour among them): for
    // narrow points a few scalar loads in the distance's own order, for
    // wide ones one dimension per lane with a widened threshold
    if (PRUNED) {
      const float* rbox = boxes64 + ((row0 + rb) >> 6) * 2 * S;
      const float* cbox = boxes_w + (colw / (64 * P)) * 2 * S;
      if (D <= 16 ? boxes_apart<S>((const_float_ptr)rbox,
                                   (const_float_ptr)cbox, eps2)
                  : wave_boxes_apart<S>(rbox, cbox, box_thr))
        continue;
    }
    // wide points, pruned: which of the 64 rows are provably farther than
    // eps from every column of this wave (lane l: row rb + l against the
    // wave's column box, in the distance's own rounded order: the bound
    // of boxes_apart with the row as a degenerate box)
    uint64_t far_rows = 0;
    if (PRUNED && !SCREEN && D > 16) {
      const const_float_ptr cb =
          (const_float_ptr)(boxes_w + (colw / (64 * P)) * 2 * S);
      const float4* xp = (const float4*)(pts + (row0 + rb + lane) * S);
      // (the sum starts from +0: adding the first square to it is exact)
      float sg = 0.f;
#pragma unroll 2
      for (int k4 = 0; k4 < S / 4; ++k4) {
        const float4 x4 = xp[k4];
        const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int k = 4 * k4 + r;
          const float lo = cb[k], hi = cb[S + k];
          float g = 0.f;
          if (lo > xs[r]) g = lo - xs[r];
          else if (xs[r] > hi) g = xs[r] - hi;
          sg = sg + g * g;
        }
      }
      far_rows = ballot(sg > eps2);
    }
    int rowv = 0;  // lane l: count of row rb+l over these columns
    if constexpr (SIGNS) {
      uint4* z = reinterpret_cast<uint4*>(rowc) + lane * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) z[k] = make_uint4(0u, 0u, 0u, 0u);
      wave_lds_sync();
#pragma unroll
      for (int g = 0; g < P / 4; ++g) lcb[g] = 0u;
    }
    if (SCREEN) {
      // the 64 rows' records (-2x, lo, hi) go to the wave's LDS area with
      // one coalesced load (lane l: row rb + l); each row is then read
      // back by all lanes from one address (a broadcast)
      const float4* rp = (const float4*)(srow + (row0 + rb + lane) * SR);
      float4* wp = (float4*)(rows_lds + lane * SR);
      wave_lds_sync();
#pragma unroll
      for (int k = 0; k < SR / 4; ++k) wp[k] = rp[k];
      wave_lds_sync();
    }
    // row addresses advance by a constant per row (the screen's exact path
    // recomputes its point address instead of carrying a second pointer)
    const float* next = SCREEN ? rows_lds : pts + (row0 + rb) * S;
    // screened: the next row's coefficients and upper threshold are read
    // while the current row is evaluated (the area has a spare 65th row)
    float a_next[SCREEN ? D : 1], hi_next = 0.f;
    if (SCREEN) {
#pragma unroll
      for (int k = 0; k < D; ++k) a_next[k] = rows_lds[k];
      hi_next = rows_lds[D + 1];
    }
#pragma unroll 2
    for (int l = 0; l < 64; ++l) {
      const int64_t row = row0 + rb + l;
      const float* cur = next;
      next += SCREEN ? SR : S;
      if (PRUNED && !SCREEN && D > 16 && ((far_rows >> l) & 1)) continue;
      // one value per column group: the exact distance, or the screen value
      float val[P];
      float lo = 0.f, thr = eps2;
      if (SCREEN) {
        float a[D];
#pragma unroll
        for (int k = 0; k < D; ++k) a[k] = a_next[k];
        thr = hi_next;
#pragma unroll
        for (int k = 0; k < D; ++k) a_next[k] = next[k];
        hi_next = next[D + 1];
        lo = cur[D];
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
        if constexpr (D <= 3) {
#pragma unroll
          for (int p = 0; p < P; ++p) val[p] = dist2<D>(xr, xc[p]);
        } else {
          // wider points: the P groups interleaved dimension by dimension
          // (each group's sum still in ascending k, so the same bits), which
          // gives the scheduler P independent chains instead of one (200k x
          // 8: 1.8% faster; at width 3 the per-group order is faster)
          float t[P];
#pragma unroll
          for (int p = 0; p < P; ++p) {
            t[p] = xr[0] - xc[p][0];
            val[p] = t[p] * t[p];
          }
#pragma unroll
          for (int k = 1; k < D; ++k) {
#pragma unroll
            for (int p = 0; p < P; ++p) t[p] = xr[k] - xc[p][k];
#pragma unroll
            for (int p = 0; p < P; ++p) t[p] = t[p] * t[p];
#pragma unroll
            for (int p = 0; p < P; ++p) val[p] = val[p] + t[p];
          }
        }
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
      uint64_t m[SIGNS ? 1 : P];
      if (ballot(vmin <= thr)) {
        if constexpr (SIGNS) {
          unsigned pat = 0;
          if (signs) {
#pragma unroll
            for (int p = 0; p < P; ++p)
              pat = __builtin_amdgcn_alignbit(
                  pat, __float_as_uint(val[p] - e2n), 31u);
            pat &= colvalid;
          } else {
#pragma unroll
            for (int p = 0; p < P; ++p)
              pat = shift_in_lane_bit(pat, ballot(val[p] <= eps2));
          }
          reinterpret_cast<unsigned char*>(rowc)[l * 64 + lane] =
              (unsigned char)__builtin_popcount(pat);
          if (!DIAG) {
            // nibble g of the pattern spread to the bytes of a word
#pragma unroll
            for (int g = 0; g < P / 4; ++g)
              lcb[g] += (((pat >> (4 * g)) & 15u) * 0x204081u) & 0x01010101u;
          }
          if (EDGES) {
            int lane_col = (int)(colw + lane);
            asm volatile("" : "+v"(lane_col));
            const int row_out = PRUNED ? ((const_int_ptr)perm)[row] : (int)row;
            if (DIAG) {
              // pairs with column > row only (each unordered pair once)
              const int q = (int)(row - colw) - lane;
              const int p0 = q < 0 ? 0 : (q >> 6) + 1;
              pat = p0 >= P ? 0u : pat & ((2u << (P - 1 - p0)) - 1u);
            }
            stage_pairs(
                pat,
                [&](int b) {
                  const int col = lane_col + (P - 1 - b) * 64;
                  return make_uint2((unsigned)row_out,
                                    (unsigned)(PRUNED ? perm[col] : col));
                },
                stage, fill, sink);
          }
        } else {
          if (SCREEN) {
            uint64_t amb = 0;
#pragma unroll
            for (int p = 0; p < P; ++p) {
              m[p] = ballot(val[p] <= lo);
              amb |= ballot(val[p] <= thr) & ~m[p];
            }
            if (amb) {
              // some pair of this row lies inside the bound: decide the
              // pairs of each group that holds one with the exact distance
              // (or, given its norms, the exact hoisted-norm form); the
              // other groups keep their screened masks
              const const_float_ptr rp = (const_float_ptr)(pts + row * S);
              float xr[D];
#pragma unroll
              for (int k = 0; k < D; ++k) xr[k] = rp[k];
              const float tr = !PRUNED && nexp != nullptr
                                   ? ((const_float_ptr)nexp)[row] : 0.f;
#pragma unroll
              for (int p = 0; p < P; ++p) {
                if ((ballot(val[p] <= thr) & ~m[p]) == 0) continue;
                if (!PRUNED && nexp != nullptr)
                  m[p] = ballot(expanded_d2<D>(xr, xc[p], tr,
                                               nexp[colw + p * 64 + lane]) <=
                                eps2);
                else
                  m[p] = ballot(dist2<D>(xr, xc[p]) <= eps2);
              }
            }
          } else {
#pragma unroll
            for (int p = 0; p < P; ++p) m[p] = ballot(val[p] <= eps2);
          }
#pragma unroll
          for (int p = 0; p < P; ++p) acc += (unsigned)__popcll(m[p]);
          if (!DIAG && P < 16) {
            // Off the diagonal with few groups per lane: only groups with a
            // pair pay for the lane counter and the staging (one wave-uniform
            // test each), and the group's mask is the exec mask of its
            // stores.  One check makes room for the whole row (at most 64 P
            // <= 512 pairs).  200k x 8: count 7.46 -> 7.32 ms; 262k x 64:
            // 104.3 -> 99.3 ms (two registers fewer, five waves per SIMD).
            // (a row without a pair adds 0, and fill never exceeds the
            // stage, so it never flushes here)
            if (EDGES && fill + acc > (unsigned)kEdgeStage) {
              flush_edges(stage, fill, sink);
              fill = 0;
            }
            int lane_col = (int)(colw + lane);
            asm volatile("" : "+v"(lane_col));
            const int row_out =
                PRUNED && EDGES ? ((const_int_ptr)perm)[row] : (int)row;
#pragma unroll
            for (int p = 0; p < P; ++p) {
              if (m[p] == 0) continue;
              // the masks were written by the compares above, many
              // instructions back
              lc[p] = add_lane_bit_far(lc[p], m[p]);
              if (EDGES) {
                if (__builtin_amdgcn_inverse_ballot_w64(m[p])) {
                  const int col = lane_col + p * 64;
                  stage[fill + bits_below(m[p])] = make_uint2(
                      (unsigned)row_out, (unsigned)(PRUNED ? perm[col] : col));
                }
                fill += (unsigned)__popcll(m[p]);
              }
            }
          } else {
#pragma unroll
            for (int p = 0; p < P; ++p)
              if (!DIAG) lc[p] = add_lane_bit(lc[p], m[p]);
            if (EDGES && acc != 0) {
              int lane_col = (int)(colw + lane);
              // recomputed here, on the rare path, instead of P live registers
              asm volatile("" : "+v"(lane_col));
              const int row_out =
                  PRUNED ? ((const_int_ptr)perm)[row] : (int)row;
              if constexpr (P >= 16) {
                // many groups per row (narrow points, dense rows): collect the
                // lane's pairs of all groups (group p's bit at position P-1-p)
                // and pack them with one prefix sum over the lanes
                unsigned pat = 0;
#pragma unroll
                for (int p = 0; p < P; ++p) pat = shift_in_lane_bit(pat, m[p]);
                if (DIAG) {
                  // pairs with column > row only (each unordered pair once,
                  // never (i, i)): the lane's column of group p exceeds the
                  // row for p >= p0
                  const int q = (int)(row - colw) - lane;
                  const int p0 = q < 0 ? 0 : (q >> 6) + 1;
                  pat = p0 >= P ? 0u : pat & ((2u << (P - 1 - p0)) - 1u);
                }
                stage_pairs(
                    pat,
                    [&](int b) {
                      const int col = lane_col + (P - 1 - b) * 64;
                      return make_uint2((unsigned)row_out,
                                        (unsigned)(PRUNED ? perm[col] : col));
                    },
                    stage, fill, sink);
              } else {
                // few groups on a diagonal tile: one ballot scan per group
                // with a pair, at most 8 groups (512 pairs) per capacity check
#pragma unroll
                for (int g = 0; g < P; g += 8) {
                  constexpr int G = P < 8 ? P : 8;
                  unsigned want = 0;
#pragma unroll
                  for (int p = g; p < g + G; ++p)
                    want += (unsigned)__popcll(m[p]);
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
          }
          // lane l of rowv holds row l's count; rows without a candidate
          // leave it at the 0 it started from
          rowv = write_lane(rowv, (int)acc, l);
        }
      }
    }
    if constexpr (SIGNS) {
      wave_lds_sync();
      const uint4* rp = reinterpret_cast<const uint4*>(rowc) + lane * 4;
      unsigned sum = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 w = rp[k];
        sum = __builtin_amdgcn_sad_u8(w.x, 0u, sum);
        sum = __builtin_amdgcn_sad_u8(w.y, 0u, sum);
        sum = __builtin_amdgcn_sad_u8(w.z, 0u, sum);
        sum = __builtin_amdgcn_sad_u8(w.w, 0u, sum);
      }
      rowv = (int)sum;
      wave_lds_sync();
      if (!DIAG) {
        // bytes 0, 1 of lcb[g] to the halves of lcw[2g], bytes 2, 3 to
        // those of lcw[2g+1] (selector 0x0c gives a zero byte)
#pragma unroll
        for (int g = 0; g < P / 4; ++g) {
          lcw[2 * g] += __builtin_amdgcn_perm(0u, lcb[g], 0x0c010c00u);
          lcw[2 * g + 1] += __builtin_amdgcn_perm(0u, lcb[g], 0x0c030c02u);
        }
      }
    }
    if (rowv) {
      const int64_t r = row0 + rb + lane;
      atomicAdd(count + (PRUNED ? perm[r] : r), (unsigned)rowv);
    }
  }
  if (!DIAG) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      unsigned v;
      if constexpr (SIGNS) {
        const int q = P - 1 - p;  // the group's pattern bit
        v = (lcw[q >> 1] >> (16 * (q & 1))) & 0xffffu;
      } else {
        v = lc[p];
      }
      if (v) {
        const int64_t c = colw + p * 64 + lane;
        atomicAdd(count + (PRUNED ? perm[c] : c), v);
      }
    }
  }
}

template <int D, bool EDGES, bool PRUNED, bool SCREEN, int PP = lane_points(D)>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(count_waves(D, SCREEN), 8))) void k_count(
    const float* __restrict__ pts, int64_t nb, int chunks_log2, int rows,
    int64_t items, int64_t n_real, float eps2, unsigned* __restrict__ count,
    uint2* __restrict__ edges, unsigned long long cap,
    unsigned long long* __restrict__ counter,
    const uint2* __restrict__ tiles, const unsigned long long* n_tiles,
    unsigned long long tile_cap, const int* __restrict__ perm,
    const float* __restrict__ boxes64, const float* __restrict__ boxes_w,
    float box_thr, const float* __restrict__ srow,
    const float* __restrict__ ncol, const float* __restrict__ nexp,
    WalkArgs walk, const unsigned* __restrict__ nonfinite) {
  constexpr int P = PP;
  constexpr int T = 256 * P;
  constexpr int SR = screen_stride(D);
  __shared__ uint2 stage_all[EDGES ? 4 * kEdgeStage : 1];
  __shared__ __attribute__((aligned(16))) float rows_all[SCREEN ? 4 * 65 * SR : 1];
  // narrow points: each wave's row counts, a byte per (row, lane)
  constexpr bool ROWC = !SCREEN && P >= 16;
  __shared__ __attribute__((aligned(16)))
  unsigned rowc_all[ROWC ? 4 * 1024 : 1];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  uint2* stage = stage_all + (EDGES ? wave * kEdgeStage : 0);
  float* rows_lds = rows_all + (SCREEN ? wave * 65 * SR : 0);
  unsigned* rowc = rowc_all + (ROWC ? wave * 1024 : 0);
  unsigned fill = 0;
  const EdgeSink sink{edges, cap, counter};
  // a non-finite input coordinate fails the fit: skip the pass
  if (*nonfinite) return;
  // pruned: walk the kept block pairs (written by the previous kernel);
  // if the list overflowed, every block pair of the sorted points
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
    // (a test mode walks the items in another order: results must not
    // change)
    const int64_t item = walk_item(
        blocked ? xcd_item(step, items) : step, items, walk.mul, walk.add);
    const int64_t tile = item >> chunks_log2;
    const int c = (int)(item & ((1 << chunks_log2) - 1));
    int64_t I, J;
    if (PRUNED && from_list) {
      const uint2 tl = tiles[tile];
      I = tl.x;
      J = tl.y;
      if (!SCREEN && D > 16 && I != J) {
        // rows from the block whose first 64-point box is wider (a heuristic:
        // the evaluation is symmetric); far rows are then skipped row by row
        constexpr int S = row_stride(D);
        const float* bi = boxes_w + I * (T / (64 * P)) * 2 * S;
        const float* bj = boxes_w + J * (T / (64 * P)) * 2 * S;
        const int k = lane_id();
        float ei = 0.f, ej = 0.f;
        if (k < S) {
          const float di = bi[S + k] - bi[k], dj = bj[S + k] - bj[k];
          ei = di * di;
          ej = dj * dj;
        }
        if (wave_sum_f32(ej) > wave_sum_f32(ei)) {
          const int64_t t = I;
          I = J;
          J = t;
        }
      }
    } else {
      if (blocked) tile_coords_blocked(tile, nb, I, J);
      else tile_coords(tile, nb, I, J);
    }
    const int64_t row0 = I * T + (int64_t)c * rows;
    const int64_t colw = J * T + (int64_t)wave * 64 * P;
    // Padding points (index >= n; in the sorted order of a pruned pass
    // they sort last) are NaN and never neighbours: a wave whose columns
    // are all padding skips the item, and the rows stop at the first
    // 64-row chunk past n.  At 50,000 points of width 2 (padded to 53,248)
    // this leaves 0.4% padding pairs instead of 11.8%.
    if (colw >= n_real || row0 >= n_real) continue;
    const int64_t left = n_real - row0;
    const int rows_eff = left < rows ? (int)((left + 63) & ~(int64_t)63) : rows;
    if (I == J)
      count_item<D, P, true, EDGES, PRUNED, SCREEN>(
          pts, row0, rows_eff, colw, eps2, count, stage, fill, sink, perm,
          boxes64, boxes_w, box_thr, srow, ncol, nexp, rows_lds, rowc, n_real);
    else
      count_item<D, P, false, EDGES, PRUNED, SCREEN>(
          pts, row0, rows_eff, colw, eps2, count, stage, fill, sink, perm,
          boxes64, boxes_w, box_thr, srow, ncol, nexp, rows_lds, rowc, n_real);
  }
  if (EDGES && fill) flush_edges(stage, fill, sink);
}

// Small sets: with the usual P the whole triangle is a handful of tiles
// and the pass runs on a few work-groups (64 for 2,000 points at d = 2);
// one column point per lane gives more, shorter work items.  Measured:
// 2k x 2 count pass 0.056 -> 0.019 ms; at 50k x 2 (5,824 items) the usual
// P stays faster, so only launches of under 512 items switch.
constexpr int kSmallP = 1;
constexpr int64_t kSmallItems = 512;

template <int D>
static hipError_t launch_count_d(const Layout& L, float eps2, bool edges,
                                 bool pruned, bool screen, Walk walk,
                                 hipStream_t s, int64_t* pairs) {
  const CountPlan c = plan_count(L.n_pad, 256 * lane_points(D), pruned);
  const float* pts = pruned ? L.sorted_pts : L.pts;
  const unsigned long long* n_tiles = &L.status->n_tiles;
#define DBK_COUNT_ARGS                                                      \
  pts, c.nb, c.chunks_log2, c.rows, c.items, L.n, eps2, L.count,            \
      edges ? L.edges : nullptr, edges ? L.edge_cap : 0ull,                 \
      &L.status->n_edges, L.tiles, n_tiles, L.tile_cap, L.perm, L.boxes64,  \
      L.boxes_w, box_gap_threshold(eps2, row_stride(D)), L.srow, L.ncol,    \
      screen && L.expanded ? L.nexp : nullptr,                              \
      walk_args(walk, c.items), &L.status->nonfinite
#define DBK_LAUNCH(E, PR, SC) \
  k_count<D, E, PR, SC><<<c.grid, kThreads, 0, s>>>(DBK_COUNT_ARGS)
  if (screen) {
    // the wider widths screen on the matrix cores instead
    if constexpr (screen_on_matrix_cores(D)) return hipErrorInvalidValue;
    else if (edges && pruned) DBK_LAUNCH(true, true, true);
    else if (edges) DBK_LAUNCH(true, false, true);
    else if (pruned) DBK_LAUNCH(false, true, true);
    else DBK_LAUNCH(false, false, true);
  } else if (!pruned && lane_points(D) > kSmallP && c.items < kSmallItems) {
    const CountPlan cs = plan_count(L.n_pad, 256 * kSmallP, false);
#define DBK_SMALL_ARGS                                                      \
  pts, cs.nb, cs.chunks_log2, cs.rows, cs.items, L.n, eps2, L.count,        \
      edges ? L.edges : nullptr, edges ? L.edge_cap : 0ull,                 \
      &L.status->n_edges, L.tiles, n_tiles, L.tile_cap, L.perm, L.boxes64,  \
      L.boxes_w, 0.f, L.srow, L.ncol, nullptr, walk_args(walk, cs.items),  \
      &L.status->nonfinite
    if (edges)
      k_count<D, true, false, false, kSmallP><<<cs.grid, kThreads, 0, s>>>(
          DBK_SMALL_ARGS);
    else
      k_count<D, false, false, false, kSmallP><<<cs.grid, kThreads, 0, s>>>(
          DBK_SMALL_ARGS);
#undef DBK_SMALL_ARGS
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

hipError_t launch_count(const Layout& L, float eps2, bool edges, bool pruned,
                        bool screen, Walk walk, hipStream_t s,
                        int64_t* pairs) {
  if (screen && screen_on_matrix_cores(L.D))
    return launch_count_mfma(L, eps2, edges, pruned, walk, s, pairs);
  switch (L.D) {
#define DBK_CASE(DD)                                                        \
  case DD:                                                                  \
    return launch_count_d<DD>(L, eps2, edges, pruned, screen, walk, s,      \
                              pairs);
    DBK_CASE(1) DBK_CASE(2) DBK_CASE(3) DBK_CASE(4) DBK_CASE(6) DBK_CASE(8)
    DBK_CASE(12) DBK_CASE(16) DBK_CASE(24) DBK_CASE(32) DBK_CASE(48)
    DBK_CASE(64)
#undef DBK_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dbk

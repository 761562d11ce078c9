// Sparse epsilon-graph export in CSR form.
//
// Row i of the graph lists every j with d2(i, j) <= eps2, i itself
// included, in ascending j: the per-point neighbour lists that Wang et al.
// ("Design and optimization of DBSCAN Algorithm based on CUDA", Sec. IV-B)
// keep as rows of an N x N cluster matrix, here without the zeros.  The
// count pass already gives the row lengths and, with an edge area, every
// neighbour pair i<j once.  From there:
//   1. row_ptr = exclusive prefix sum of the counts (64-bit);
//   2. every row starts with the point itself, then each captured pair
//      (i, j) lands once in row i and once in row j (a cursor per row
//      hands out the slots, in no particular order, to chunks of pairs
//      ranked in LDS);
//   3. every row is sorted in ascending order (below), which makes the
//      result unique.
#include <climits>

#include "device.h"
#include "internal.h"

namespace dbk {

constexpr int kScanItems = 4;                       // counts per thread
constexpr int kScanBlock = kThreads * kScanItems;   // counts per workgroup

static unsigned grid_for_g(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (unsigned)(g < kMaxGrid ? g : kMaxGrid);
}

// Exclusive prefix sum of 64-bit values over a 256-thread block; *total gets
// the block's sum.  sh: 4 words of LDS.
__device__ __forceinline__ unsigned long long block_excl_scan64(
    unsigned long long v, unsigned long long* sh, unsigned long long* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  unsigned long long x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  unsigned long long wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += sh[w];
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return wbase + x - v;
}

// Sum of the counts of each block of kScanBlock rows.
__global__ __launch_bounds__(kThreads) void k_row_block_totals(
    const unsigned* __restrict__ count, int64_t n,
    unsigned long long* __restrict__ sums) {
  __shared__ unsigned long long sh[4];
  const int64_t base = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * kScanItems;
  unsigned long long c = 0;
  for (int q = 0; q < kScanItems; ++q)
    if (base + q < n) c += count[base + q];
  unsigned long long tot;
  block_excl_scan64(c, sh, &tot);
  if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

// Exclusive scan of the block totals in place, by one workgroup.
__global__ __launch_bounds__(kThreads) void k_scan_row_totals(
    unsigned long long* sums, int64_t nblk) {
  __shared__ unsigned long long sh[4];
  unsigned long long carry = 0;
  for (int64_t b0 = 0; b0 < nblk; b0 += kThreads) {
    const int64_t b = b0 + threadIdx.x;
    const unsigned long long v = b < nblk ? sums[b] : 0ull;
    unsigned long long tot;
    const unsigned long long ex = block_excl_scan64(v, sh, &tot);
    if (b < nblk) sums[b] = carry + ex;
    carry += tot;
  }
}

// row_ptr[i] = sum of count[0..i-1]; the thread holding row n-1 also
// writes row_ptr[n].  Every row's first slot gets the point itself and its
// cursor starts after it.  n = 0 only writes row_ptr[0] = 0.
__global__ __launch_bounds__(kThreads) void k_row_offsets(
    const unsigned* __restrict__ count, int64_t n,
    const unsigned long long* __restrict__ sums, int64_t* __restrict__ row_ptr,
    unsigned* __restrict__ cursor, int* __restrict__ col_idx,
    unsigned long long col_cap) {
  __shared__ unsigned long long sh[4];
  const int64_t base = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * kScanItems;
  unsigned c[kScanItems];
  unsigned long long mine = 0;
  for (int q = 0; q < kScanItems; ++q) {
    c[q] = base + q < n ? count[base + q] : 0u;
    mine += c[q];
  }
  unsigned long long tot;
  unsigned long long pos = sums[blockIdx.x] + block_excl_scan64(mine, sh, &tot);
  if (n == 0 && blockIdx.x == 0 && threadIdx.x == 0) row_ptr[0] = 0;
  for (int q = 0; q < kScanItems; ++q) {
    const int64_t i = base + q;
    if (i >= n) break;
    row_ptr[i] = (int64_t)pos;
    // the self slot is written only when the whole graph fits the caller's
    // buffer (the host checks the same bound before the scatter)
    if (col_idx != nullptr && pos < col_cap) col_idx[pos] = (int)i;
    cursor[i] = 1u;
    pos += c[q];
    if (i == n - 1) row_ptr[n] = (int64_t)pos;
  }
}

// Each captured pair (i, j) goes once into row i and once into row j, at a
// slot handed out by that row's cursor.  A work-group takes CH pairs at a
// time and ranks both ends of each pair in an LDS hash table (linear
// probing, at most 2 CH keys in 4 CH slots, so a probe always ends): the
// entries of one index within the chunk get consecutive local ranks, and
// one global atomic per distinct index reserves them all.  A slot beyond
// its row's length (or an index beyond n) would mean the counts and the
// pairs disagree; it is never written and the call reports an internal
// error.
template <int CH>
__global__ __launch_bounds__(kThreads) void k_graph_scatter(
    const uint2* __restrict__ pairs, int64_t m, int64_t n,
    const int64_t* __restrict__ row_ptr, unsigned* __restrict__ cursor,
    int* __restrict__ col_idx, Status* __restrict__ st) {
  constexpr int kSlots = 4 * CH;                  // power of two
  constexpr int kBits = __builtin_ctz(kSlots);
  constexpr int PER = CH / kThreads;              // pairs per thread
  constexpr unsigned kEmpty = 0xffffffffu;
  __shared__ unsigned keys[kSlots];
  __shared__ unsigned cnt[kSlots];
  const int t = threadIdx.x;
  for (int64_t c0 = (int64_t)blockIdx.x * CH; c0 < m;
       c0 += (int64_t)gridDim.x * CH) {
    for (int s = t; s < kSlots; s += kThreads) {
      keys[s] = kEmpty;
      cnt[s] = 0u;
    }
    __syncthreads();
    uint2 p[PER];
    unsigned sx[PER], sy[PER];                    // slot << 16 | local rank
    bool ok[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int64_t e = c0 + q * kThreads + t;
      const bool live = e < m;
      p[q] = live ? pairs[e] : make_uint2(kEmpty, kEmpty);
      ok[q] = live && p[q].x < n && p[q].y < n;
      if (live && !ok[q]) atomicOr(&st->graph_bad, 1u);
      sx[q] = sy[q] = 0u;
      if (!ok[q]) continue;
#pragma unroll
      for (int side = 0; side < 2; ++side) {
        const unsigned key = side ? p[q].y : p[q].x;
        unsigned h = (key * 2654435761u) >> (32 - kBits);
        while (true) {
          const unsigned k = atomicCAS(&keys[h], kEmpty, key);
          if (k == kEmpty || k == key) break;
          h = (h + 1u) & (unsigned)(kSlots - 1);
        }
        const unsigned r = atomicAdd(&cnt[h], 1u);
        (side ? sy[q] : sx[q]) = (h << 16) | r;
      }
    }
    __syncthreads();
    // one reservation per distinct index; the table then holds its base
    for (int s = t; s < kSlots; s += kThreads) {
      const unsigned c = cnt[s];
      if (c != 0u) cnt[s] = atomicAdd(cursor + keys[s], c);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      if (!ok[q]) continue;
      const unsigned a = cnt[sx[q] >> 16] + (sx[q] & 0xffffu);
      const int64_t ri = row_ptr[p[q].x];
      if ((int64_t)a < row_ptr[p[q].x + 1] - ri) col_idx[ri + a] = (int)p[q].y;
      else atomicOr(&st->graph_bad, 1u);
      const unsigned b = cnt[sy[q] >> 16] + (sy[q] & 0xffffu);
      const int64_t rj = row_ptr[p[q].y];
      if ((int64_t)b < row_ptr[p[q].y + 1] - rj) col_idx[rj + b] = (int)p[q].x;
      else atomicOr(&st->graph_bad, 1u);
    }
    __syncthreads();                              // before the table is reset
  }
}

hipError_t launch_row_offsets(const Layout& L, const GraphLayout& G,
                              int64_t* row_ptr, int* col_idx,
                              unsigned long long col_cap, hipStream_t s) {
  const int64_t nblk = (L.n + kScanBlock - 1) / kScanBlock;
  const unsigned grid = (unsigned)(nblk > 0 ? nblk : 1);
  if (nblk > 0) {
    k_row_block_totals<<<grid, kThreads, 0, s>>>(L.count, L.n, G.row_sums);
    k_scan_row_totals<<<1, kThreads, 0, s>>>(G.row_sums, nblk);
  } else {
    k_scan_row_totals<<<1, kThreads, 0, s>>>(G.row_sums, 1);
  }
  k_row_offsets<<<grid, kThreads, 0, s>>>(L.count, L.n, G.row_sums, row_ptr,
                                          G.cursor, col_idx, col_cap);
  return hipGetLastError();
}

hipError_t launch_graph_scatter(const Layout& L, const GraphLayout& G,
                                unsigned long long n_pairs,
                                const int64_t* row_ptr, int* col_idx,
                                hipStream_t s) {
  // 512 pairs per chunk (16 KB of LDS per work-group).  Measured against
  // the earlier scatter (row runs aggregated, one atomic per pair on the
  // column side): 262k x 64 22.5 -> 10.3 ms, 1M x 3 1.31 -> 0.62 ms,
  // 200k x 8 2.06 -> 1.36 ms; chunks of 256, 1024 and 2048 were slower
  // on the three.
  constexpr int kChunk = 512;
  if (n_pairs > 0)
    k_graph_scatter<kChunk>
        <<<grid_for_g((int64_t)n_pairs, kChunk), kThreads, 0, s>>>(
            L.edges, (int64_t)n_pairs, L.n, row_ptr, G.cursor, col_idx,
            L.status);
  return hipGetLastError();
}

// ---- row sort ------------------------------------------------------------
// Each row holds distinct indices in [0, n) in arbitrary order; it is
// sorted in place (the result is back in col_idx).  A bitonic network in
// its direction-free form (every compare-exchange puts the smaller value at
// the smaller position: each level k starts with a "flip" stage pairing
// entry i with i ^ (k-1), then half-cleaners pair i with i ^ j for
// j = k/4 .. 1) over the row padded with INT_MAX to M entries, each thread
// holding E consecutive entries in registers (entry index = thread * E +
// r).  Stages whose partner is in the same thread are plain min / max on
// registers; partners in another lane of the wave come through DPP, the
// LDS crossbar's swizzle or a permute; partners in another wave through
// LDS (laid out [r][thread]) with work-group barriers.  By row length:
//   <= 64     one wave, one entry per lane (M = 64);
//   <= 128, 256, 512, 1024   one wave, 2, 4, 8, 16 per lane;
//   <= 2048, 4096, 8192   one work-group of 4 waves, 8, 16, 32 per
//             thread;
//   longer    the work-group sorts the row's 8192-entry chunks, then merges
//             neighbouring runs, doubling their length per pass, from
//             col_idx to the dead pair area and back (each thread merges an
//             equal share of the output, split by a binary search on the
//             two runs), and copies the row back after an odd number of
//             passes.
// Waves take rows 16 at a time and sort those up to 1024 entries; longer
// ones go on a list (one atomic per batch, into the row cursors, dead once
// the pairs are scattered) for a work-group kernel: the bitmap sort below
// when a bitmap of [0, n) fits its LDS (n up to 491,520), else the
// networks and merges above (262k x 64, rows of 1,000 to 12,600 entries:
// 11.3 ms by networks, 3.7 ms by bitmap).

// LDS of the bitmap sort of long rows: up to 491,520 points
constexpr size_t kBitmapSortBytes = 60 * 1024;
constexpr int kWaveSortMax = 1024;                 // rows sorted by one wave
constexpr int kBlockSortMax = kThreads * 32;       // 8192: by one work-group

__device__ __forceinline__ void cx(int& lo, int& hi) {
  const int a = lo < hi ? lo : hi, b = lo < hi ? hi : lo;
  lo = a;
  hi = b;
}

// The value of lane (lane ^ X) of the wave, X < 64: DPP for the partners
// inside a 16-lane row (quad permutations for 1, 2, 3; half-row mirror for
// 7, row mirror for 15, rotation by 8 for 8), the LDS crossbar's swizzle
// for 4, 16 and 31 (within each 32 lanes, no address operand), a permute
// for 32 and 63.
template <int X>
__device__ __forceinline__ int lane_xor(int v) {
  if constexpr (X == 1) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false);
  else if constexpr (X == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false);
  else if constexpr (X == 3) return __builtin_amdgcn_update_dpp(0, v, 0x1B, 0xf, 0xf, false);
  else if constexpr (X == 7) return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false);
  else if constexpr (X == 8) return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false);
  else if constexpr (X == 15) return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false);
  else if constexpr (X < 32) return __builtin_amdgcn_ds_swizzle(v, (X << 10) | 0x1f);
  else return __shfl_xor(v, X, 64);
}

// Flip stage with the partner in thread t ^ X (X = k/E - 1 < 64): entry r
// pairs with the partner's entry E-1-r.  The thread with bit HB of t clear
// (HB = k / 2E) holds the smaller positions and keeps the minima.
template <int E, int X>
__device__ __forceinline__ void flip_lanes(int (&v)[E], int t) {
  int o[E];
#pragma unroll
  for (int r = 0; r < E; ++r) o[r] = lane_xor<X>(v[E - 1 - r]);
  const bool lower = (t & ((X + 1) >> 1)) == 0;
#pragma unroll
  for (int r = 0; r < E; ++r)
    v[r] = lower ? (o[r] < v[r] ? o[r] : v[r]) : (o[r] > v[r] ? o[r] : v[r]);
}

// Half-cleaner with the partner in thread t ^ X (X a power of two < 64).
template <int E, int X>
__device__ __forceinline__ void half_lanes(int (&v)[E], int t) {
  int o[E];
#pragma unroll
  for (int r = 0; r < E; ++r) o[r] = lane_xor<X>(v[r]);
  const bool lower = (t & X) == 0;
#pragma unroll
  for (int r = 0; r < E; ++r)
    v[r] = lower ? (o[r] < v[r] ? o[r] : v[r]) : (o[r] > v[r] ? o[r] : v[r]);
}

// Flip or half-cleaner with the partner in another wave (X >= 64): through
// LDS, [r][thread].
template <int E, int W>
__device__ __forceinline__ void cross_waves(int (&v)[E], int t, int x,
                                            bool flip, int* lds) {
  constexpr int T = 64 * W;
#pragma unroll
  for (int r = 0; r < E; ++r) lds[r * T + t] = v[r];
  __syncthreads();
  const bool lower = (t & (flip ? (x + 1) >> 1 : x)) == 0;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int o = lds[(flip ? E - 1 - r : r) * T + (t ^ x)];
    v[r] = lower ? (o < v[r] ? o : v[r]) : (o > v[r] ? o : v[r]);
  }
  __syncthreads();
}

// In-thread stages of level K (K <= E): the flip, then the half-cleaners.
template <int E, int K, int J>
__device__ __forceinline__ void thread_half(int (&v)[E]) {
#pragma unroll
  for (int r = 0; r < E; ++r)
    if ((r & J) == 0) cx(v[r], v[r | J]);
  if constexpr (J > 1) thread_half<E, K, J / 2>(v);
}
template <int E, int K>
__device__ __forceinline__ void thread_level(int (&v)[E]) {
  // flip within each block of K registers
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int p = r ^ (K - 1);
    if ((r & (K / 2)) == 0) cx(v[r], v[p]);
  }
  if constexpr (K >= 4) thread_half<E, K, K / 4>(v);
  if constexpr (2 * K <= E) thread_level<E, 2 * K>(v);
}

// Half-cleaners j < E of a level above E (in-thread, partner r ^ J).
template <int E, int J>
__device__ __forceinline__ void thread_cleaners(int (&v)[E]) {
  if constexpr (J >= 1) {
#pragma unroll
    for (int r = 0; r < E; ++r)
      if ((r & J) == 0) cx(v[r], v[r | J]);
    thread_cleaners<E, J / 2>(v);
  }
}

// Half-cleaners across lanes at thread distances JT, JT/2, .., 1.
template <int E, int JT>
__device__ __forceinline__ void lane_cleaners(int (&v)[E], int t) {
  if constexpr (JT >= 1) {
    half_lanes<E, JT>(v, t);
    lane_cleaners<E, JT / 2>(v, t);
  }
}

// Levels k = KT*E .. 64*E of a one-wave network, unrolled at compile time.
template <int E, int KT>
__device__ __forceinline__ void wave_levels(int (&v)[E], int t) {
  flip_lanes<E, KT - 1>(v, t);
  lane_cleaners<E, KT / 4>(v, t);
  thread_cleaners<E, E / 2>(v);
  if constexpr (KT < 64) wave_levels<E, 2 * KT>(v, t);
}

// Bitonic network over M = E * 64 * W entries; thread t (of 64 * W) holds
// entries t*E .. t*E+E-1 in v; ascending on return.  One wave: every stage
// unrolled at compile time; a work-group (32 entries per thread): the
// levels above the thread in a loop, each stage a compile-time variant.
template <int E, int W>
__device__ __forceinline__ void bitonic_regs(int (&v)[E], int* lds) {
  constexpr int T = 64 * W;
  const int t = W == 1 ? lane_id() : (int)threadIdx.x;
  if constexpr (E > 1) thread_level<E, 2>(v);
  if constexpr (W == 1) {
    wave_levels<E, 2>(v, t);
    return;
  }
  for (int kt = 2; kt <= T; kt <<= 1) {   // level k = kt * E
    switch (kt - 1) {                      // the flip: partner thread t ^ (kt-1)
      case 1: flip_lanes<E, 1>(v, t); break;
      case 3: flip_lanes<E, 3>(v, t); break;
      case 7: flip_lanes<E, 7>(v, t); break;
      case 15: flip_lanes<E, 15>(v, t); break;
      case 31: flip_lanes<E, 31>(v, t); break;
      case 63: flip_lanes<E, 63>(v, t); break;
      default: cross_waves<E, W>(v, t, kt - 1, true, lds); break;
    }
    for (int jt = kt >> 2; jt >= 1; jt >>= 1) {  // half-cleaners across threads
      switch (jt) {
        case 1: half_lanes<E, 1>(v, t); break;
        case 2: half_lanes<E, 2>(v, t); break;
        case 4: half_lanes<E, 4>(v, t); break;
        case 8: half_lanes<E, 8>(v, t); break;
        case 16: half_lanes<E, 16>(v, t); break;
        case 32: half_lanes<E, 32>(v, t); break;
        default: cross_waves<E, W>(v, t, jt, false, lds); break;
      }
    }
    thread_cleaners<E, E / 2>(v);
  }
}

// LDS index of row entry i in the staging area: one pad word per 32
// entries, so that thread t reading entry t*E + r (fixed r) and thread t
// writing entry t (coalesced side) both spread over the banks.
__device__ __forceinline__ int stage_at(int i) { return i + (i >> 5); }

template <int W>
__device__ __forceinline__ void group_sync() {
  if (W == 1) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

// Sort row[0 .. len) in place with the E-per-thread network of W waves
// (len <= E * 64 * W).  The row moves between memory and registers through
// the staging area st (E * 64 * W + E * 2 * W ints of LDS), so that the
// global loads and stores are coalesced; the cross-wave stages of the
// network reuse it.
template <int E, int W>
__device__ __forceinline__ void sort_row(int* row, int len, int* st) {
  constexpr int T = 64 * W;
  constexpr int M = E * T;
  const int t = W == 1 ? lane_id() : (int)threadIdx.x;
  int v[E];
  if (E == 1) {
    v[0] = t < len ? row[t] : INT_MAX;
  } else {
    for (int i = t; i < M; i += T) st[stage_at(i)] = i < len ? row[i] : INT_MAX;
    group_sync<W>();
#pragma unroll
    for (int r = 0; r < E; ++r) v[r] = st[stage_at(t * E + r)];
    group_sync<W>();
  }
  bitonic_regs<E, W>(v, st);
  if (E == 1) {
    if (t < len) row[t] = v[0];
  } else {
#pragma unroll
    for (int r = 0; r < E; ++r) st[stage_at(t * E + r)] = v[r];
    group_sync<W>();
    for (int i = t; i < len; i += T) row[i] = st[stage_at(i)];
    group_sync<W>();
  }
}

constexpr int kRowBatch = 16;                      // rows per wave and step
constexpr int kWaveStage = kWaveSortMax + kWaveSortMax / 32;   // ints per wave

__global__ __launch_bounds__(kThreads) void k_sort_rows_wave(
    const int64_t* __restrict__ row_ptr, int64_t n, int* col_idx,
    unsigned* __restrict__ long_list, Status* __restrict__ st) {
  __shared__ int stage_all[4 * kWaveStage];
  int* stage = stage_all + (threadIdx.x >> 6) * kWaveStage;
  const int lane = lane_id();
  const int64_t wave = blockIdx.x * (int64_t)(blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t b0 = wave * kRowBatch; b0 < n; b0 += waves * kRowBatch) {
    const int64_t i = b0 + lane;
    const int64_t len =
        lane < kRowBatch && i < n ? row_ptr[i + 1] - row_ptr[i] : 0;
    // the batch's long rows go on the list, one atomic for the batch
    const uint64_t longm = ballot(len > kWaveSortMax);
    if (longm) {
      unsigned base = 0;
      if (lane == 0) base = atomicAdd(&st->long_rows, (unsigned)__popcll(longm));
      base = (unsigned)__builtin_amdgcn_readfirstlane((int)base);
      if (len > kWaveSortMax) long_list[base + bits_below(longm)] = (unsigned)i;
    }
    uint64_t todo = ballot(len > 1 && len <= kWaveSortMax);
    while (todo) {
      const int l = __builtin_ctzll(todo);
      todo &= todo - 1;
      const int64_t r = b0 + l;
      const int64_t rb = row_ptr[r];
      const int rl = (int)(row_ptr[r + 1] - rb);
      int* row = col_idx + rb;
      if (rl <= 64) sort_row<1, 1>(row, rl, stage);
      else if (rl <= 128) sort_row<2, 1>(row, rl, stage);
      else if (rl <= 256) sort_row<4, 1>(row, rl, stage);
      else if (rl <= 512) sort_row<8, 1>(row, rl, stage);
      else sort_row<16, 1>(row, rl, stage);
    }
  }
}

// Number of entries of run x (length nx) among the first d outputs of the
// merge of x and y (ties cannot occur: the entries are distinct).
__device__ __forceinline__ int merge_split(const int* x, int nx, const int* y,
                                           int ny, int d) {
  int lo = d > ny ? d - ny : 0, hi = d < nx ? d : nx;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;       // take mid from x, d - mid from y
    if (x[mid] < y[d - mid - 1]) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) void k_sort_rows_group(
    const int64_t* __restrict__ row_ptr, int* col_idx, int* alt,
    const unsigned* __restrict__ long_list, const Status* __restrict__ st) {
  __shared__ int lds[kBlockSortMax + kBlockSortMax / 32];
  const unsigned rows = st->long_rows;
  for (unsigned q = blockIdx.x; q < rows; q += gridDim.x) {
    const int64_t i = long_list[q];
    const int64_t b = row_ptr[i];
    const int len = (int)(row_ptr[i + 1] - b);
    int* row = col_idx + b;
    if (len <= 2048) {
      sort_row<8, 4>(row, len, lds);
    } else if (len <= 4096) {
      sort_row<16, 4>(row, len, lds);
    } else {
      for (int c = 0; c < len; c += kBlockSortMax) {
        const int cl = len - c < kBlockSortMax ? len - c : kBlockSortMax;
        sort_row<32, 4>(row + c, cl, lds);
      }
    }
    __syncthreads();
    if (len <= kBlockSortMax) continue;
    int* src = row;
    int* dst = alt + b;
    for (int w = kBlockSortMax; w < len; w <<= 1) {
      // merge runs [s, s + w) and [s + w, s + 2w) for every s
      for (int s0 = 0; s0 < len; s0 += 2 * w) {
        const int nx = len - s0 < w ? len - s0 : w;
        const int rest = len - s0 - nx;
        const int ny = rest < w ? rest : w;
        const int* x = src + s0;
        const int* y = x + nx;
        int* out = dst + s0;
        const int total = nx + ny;
        const int per = (total + (int)blockDim.x - 1) / (int)blockDim.x;
        const int d0 = min((int)threadIdx.x * per, total);
        const int d1 = min(d0 + per, total);
        int ix = merge_split(x, nx, y, ny, d0);
        int iy = d0 - ix;
        for (int d = d0; d < d1; ++d) {
          const bool take_x = iy >= ny || (ix < nx && x[ix] < y[iy]);
          out[d] = take_x ? x[ix++] : y[iy++];
        }
      }
      __syncthreads();
      int* t = src;
      src = dst;
      dst = t;
    }
    if (src != row) {
      for (int t = threadIdx.x; t < len; t += blockDim.x) row[t] = src[t];
      __syncthreads();
    }
  }
}

// Long rows when the point count is small enough for a bitmap of [0, n)
// in LDS (dynamic shared memory, one range of whole 256-word steps per
// wave).  A row holds distinct indices, so setting one bit per entry and
// reading the bitmap back in index order sorts it: each wave counts the
// bits of its range, the ranges' totals give each wave its first output
// slot, and the wave then walks its range 256 words at a time, four
// consecutive words per lane, placing the lane's indices after a prefix
// sum of the lanes' bit counts and clearing the words for the next row.
__global__ __launch_bounds__(kThreads) void k_sort_rows_bitmap(
    const int64_t* __restrict__ row_ptr, int* col_idx,
    const unsigned* __restrict__ long_list, Status* __restrict__ st,
    int64_t n, int wave_words) {
  extern __shared__ uint4 bm4[];
  unsigned* bm = reinterpret_cast<unsigned*>(bm4);
  __shared__ unsigned wave_total[kThreads / 64];
  const int lane = lane_id();
  const int wave = (int)(threadIdx.x >> 6);
  const int total_quads = wave_words * (kThreads / 64) / 4;
  for (int w = threadIdx.x; w < total_quads; w += kThreads)
    bm4[w] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  const unsigned rows = st->long_rows;
  const int q0 = wave * (wave_words / 4);           // the wave's first quad
  for (unsigned q = blockIdx.x; q < rows; q += gridDim.x) {
    const int64_t i = long_list[q];
    const int64_t b = row_ptr[i];
    const int len = (int)(row_ptr[i + 1] - b);
    int* row = col_idx + b;
    // eight loads in flight per thread before their bits are set
    for (int t0 = 0; t0 < len; t0 += 8 * kThreads) {
      unsigned v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int t = t0 + r * kThreads + (int)threadIdx.x;
        v[r] = t < len ? (unsigned)row[t] : 0xffffffffu;
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (t0 + r * kThreads + (int)threadIdx.x >= len) continue;
        if (v[r] < (unsigned long long)n)
          atomicOr(&bm[v[r] >> 5], 1u << (v[r] & 31u));
        else
          atomicOr(&st->graph_bad, 1u);
      }
    }
    __syncthreads();
    unsigned c = 0;
#pragma unroll 4
    for (int k = 0; k < wave_words / 4; k += 64) {
      const uint4 x = bm4[q0 + k + lane];
      c += __popc(x.x) + __popc(x.y) + __popc(x.z) + __popc(x.w);
    }
    c = wave_incl_sum(c);
    if (lane == 63) wave_total[wave] = c;
    __syncthreads();
    unsigned pos = 0;
    for (int w = 0; w < wave; ++w) pos += wave_total[w];
#pragma unroll 2
    for (int k = 0; k < wave_words / 4; k += 64) {
      const int qi = q0 + k + lane;
      const uint4 x = bm4[qi];
      bm4[qi] = make_uint4(0u, 0u, 0u, 0u);
      const unsigned cnt = __popc(x.x) + __popc(x.y) + __popc(x.z) + __popc(x.w);
      const unsigned incl = wave_incl_sum(cnt);
      unsigned o = pos + incl - cnt;
      pos += (unsigned)__builtin_amdgcn_readlane((int)incl, 63);
      const unsigned words[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        unsigned word = words[r];
        const unsigned base = ((unsigned)qi * 4u + (unsigned)r) * 32u;
        // a row of distinct indices fills exactly its len slots
        while (word != 0u) {
          if (o < (unsigned)len) row[o] = (int)(base + (unsigned)__builtin_ctz(word));
          ++o;
          word &= word - 1u;
        }
      }
    }
    __syncthreads();
  }
}

// Rows in ascending order, in place in col_idx.
hipError_t launch_graph_sort(const Layout& L, const GraphLayout& G,
                             const int64_t* row_ptr, int* col_idx, int64_t nnz,
                             hipStream_t s) {
  if (L.n == 0 || nnz == 0) return hipSuccess;
  // one batch of kRowBatch rows per wave at first
  int64_t g = (L.n + 4 * kRowBatch - 1) / (4 * kRowBatch);
  if (g > kMaxGrid) g = kMaxGrid;
  k_sort_rows_wave<<<(unsigned)g, kThreads, 0, s>>>(row_ptr, L.n, col_idx,
                                                    G.cursor, L.status);
  // long rows: by bitmap when [0, n) fits the work-group's LDS, else by
  // the work-group's sorting network and merges
  const int64_t words = (L.n + 31) / 32;
  const int64_t wave_words = (words + 256 * 4 - 1) / (256 * 4) * 256;
  const size_t bitmap_bytes = (size_t)wave_words * 4 * sizeof(unsigned);
  if (bitmap_bytes <= kBitmapSortBytes) {
    // as many work-groups as the LDS lets every CU hold at once (rows are
    // dealt round-robin, so a second partial round would double the time)
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess)
      cus = 256;
    int per_cu = (int)((160u * 1024u) / (bitmap_bytes + 64));
    per_cu = per_cu < 1 ? 1 : per_cu > 8 ? 8 : per_cu;
    k_sort_rows_bitmap<<<(unsigned)(cus * per_cu), kThreads, bitmap_bytes, s>>>(
        row_ptr, col_idx, G.cursor, L.status, L.n, (int)wave_words);
  } else {
    k_sort_rows_group<<<2048, kThreads, 0, s>>>(
        row_ptr, col_idx, reinterpret_cast<int*>(G.alt), G.cursor, L.status);
  }
  return hipGetLastError();
}

}  // namespace dbk

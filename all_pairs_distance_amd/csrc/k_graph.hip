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
//      (i, j) lands once in row i and once in row j (an atomic cursor per
//      row hands out the slots, in no particular order);
//   3. a segmented radix sort (rocPRIM, one segment per row) puts every
//      row in ascending order, which makes the result unique.
#include <rocprim/device/device_segmented_radix_sort.hpp>

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

// Each captured pair (i, j) goes once into row i and once into row j.
// Pairs of one row arrive in runs (the count pass writes them row by row),
// so lanes with the same first index share one atomic: the run's first
// lane reserves the whole run and the others take consecutive slots.  A
// slot beyond its row's length (or an index beyond n) would mean the
// counts and the pairs disagree; it is never written and the call reports
// an internal error.
__global__ __launch_bounds__(kThreads) void k_graph_scatter(
    const uint2* __restrict__ pairs, int64_t m, int64_t n,
    const int64_t* __restrict__ row_ptr, unsigned* __restrict__ cursor,
    int* __restrict__ col_idx, Status* __restrict__ st) {
  const int lane = lane_id();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // whole waves iterate together so the run detection sees all 64 lanes
  const int64_t first = blockIdx.x * (int64_t)blockDim.x + (threadIdx.x & ~63);
  for (int64_t e0 = first; e0 < m; e0 += stride) {
    const int64_t e = e0 + lane;
    const bool live = e < m;
    uint2 p = live ? pairs[e] : make_uint2(0xffffffffu, 0xffffffffu);
    // runs of equal first index among the live lanes
    const unsigned prev = __shfl_up(p.x, 1, 64);
    const bool head = live && (lane == 0 || prev != p.x);
    const uint64_t heads = ballot(head);
    const uint64_t upto = heads & (lane == 63 ? ~0ull : ((2ull << lane) - 1));
    const int start = upto ? 63 - __clzll(upto) : lane;
    const uint64_t after = heads & (lane == 63 ? 0ull : (~0ull << (lane + 1)));
    const uint64_t live_mask = ballot(live);
    const int live_end = 64 - __clzll(live_mask);   // one past the last live lane
    const int next = after ? __ffsll((long long)after) - 1 : live_end;
    unsigned slot0 = 0;
    if (head && p.x < n) slot0 = atomicAdd(cursor + p.x, (unsigned)(next - lane));
    slot0 = __shfl(slot0, start, 64);
    if (live && (p.x >= n || p.y >= n)) {
      atomicOr(&st->graph_bad, 1u);
    } else if (live) {
      const unsigned a = slot0 + (unsigned)(lane - start);
      const int64_t ri = row_ptr[p.x];
      const int64_t li = row_ptr[p.x + 1] - ri;
      if ((int64_t)a < li) col_idx[ri + a] = (int)p.y;
      else atomicOr(&st->graph_bad, 1u);
      const unsigned b = atomicAdd(cursor + p.y, 1u);
      const int64_t rj = row_ptr[p.y];
      const int64_t lj = row_ptr[p.y + 1] - rj;
      if ((int64_t)b < lj) col_idx[rj + b] = (int)p.x;
      else atomicOr(&st->graph_bad, 1u);
    }
  }
}

static unsigned key_bits(int64_t n) {
  unsigned b = 1;
  while (b < 31 && ((int64_t)1 << b) < n) ++b;
  return b;
}

size_t graph_sort_bytes(int64_t n) {
  size_t bytes = 0;
  rocprim::double_buffer<unsigned> keys(nullptr, nullptr);
  const hipError_t e = rocprim::segmented_radix_sort_keys(
      nullptr, bytes, keys, 0u, (unsigned)(n > 0 ? n : 1),
      (const int64_t*)nullptr, (const int64_t*)nullptr, 0u, key_bits(n));
  return e == hipSuccess ? bytes : 0;
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
  if (n_pairs > 0)
    k_graph_scatter<<<grid_for_g((int64_t)n_pairs, kThreads), kThreads, 0, s>>>(
        L.edges, (int64_t)n_pairs, L.n, row_ptr, G.cursor, col_idx, L.status);
  return hipGetLastError();
}

// Rows in ascending order.  The pair area is dead once scattered and serves
// as the sort's second buffer; *in_alt tells whether the sorted rows ended
// there.
hipError_t launch_graph_sort(const Layout& L, const GraphLayout& G,
                             const int64_t* row_ptr, int* col_idx, int64_t nnz,
                             bool* in_alt, hipStream_t s) {
  rocprim::double_buffer<unsigned> keys(reinterpret_cast<unsigned*>(col_idx),
                                        reinterpret_cast<unsigned*>(G.alt));
  size_t bytes = G.sort_bytes;
  const hipError_t e = rocprim::segmented_radix_sort_keys(
      G.sort_tmp, bytes, keys, (unsigned)nnz, (unsigned)L.n, row_ptr,
      row_ptr + 1, 0u, key_bits(L.n), s);
  if (e != hipSuccess) return e;
  *in_alt = keys.current() != reinterpret_cast<unsigned*>(col_idx);
  return hipGetLastError();
}

}  // namespace dbk

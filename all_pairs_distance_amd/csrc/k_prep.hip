// Bandwidth-bound passes around the two distance passes: ingest/layout,
// core flags (+ sorted compaction for the tile merge), root compression
// and canonical labels.  Each is a grid-stride loop over points with
// coalesced loads and stores.
#include <climits>

#include "device.h"
#include "internal.h"

namespace dbk {

static unsigned grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (unsigned)(g < kMaxGrid ? g : kMaxGrid);
}

__global__ void k_zero_status(Status* st) {
  unsigned* w = reinterpret_cast<unsigned*>(st);
  if (threadIdx.x < sizeof(Status) / 4) w[threadIdx.x] = 0u;
}

// Copy the caller's [n][d] points into the padded [n_pad][S] layout: the
// coordinates d..S-1 of a real point are 0 (adding 0 to a sum of squares
// is exact), every coordinate of a padding row is NaN (never a neighbour
// of anything).  Flags any non-finite input coordinate.  The same launch
// initialises the per-point arrays: counts 0, no border or member minimum
// yet (the union-find forest is set up with the core flags).
__global__ void k_layout(const float* __restrict__ in, int64_t n, int d, int S,
                         int64_t total, float* __restrict__ pts,
                         Status* __restrict__ st, int64_t n_pad,
                         unsigned* __restrict__ count, int* __restrict__ bmin,
                         int* __restrict__ cmin) {
  bool bad = false;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  for (int64_t e = t0; e < total; e += stride) {
    const int64_t i = e / S;
    const int k = (int)(e - i * S);
    float v;
    if (i < n) {
      v = k < d ? in[i * d + k] : 0.0f;
      bad |= !__builtin_isfinite(v);
    } else {
      v = __builtin_nanf("");
    }
    pts[e] = v;
  }
  if (bad) st->nonfinite = 1u;
  for (int64_t i = t0; i < n_pad; i += stride) {
    count[i] = 0u;
    bmin[i] = INT_MAX;
    cmin[i] = INT_MAX;
  }
}

hipError_t launch_prepare(const Layout& L, const float* in, hipStream_t s) {
  k_zero_status<<<1, 64, 0, s>>>(L.status);
  const int64_t total = L.n_pad * L.stride;
  k_layout<<<grid_for(total, 256 * 8), 256, 0, s>>>(
      in, L.n, L.d, L.stride, total, L.pts, L.status, L.n_pad, L.count,
      L.bmin, L.cmin);
  return hipGetLastError();
}

// core[i] = count[i] >= min_pts (Wang et al., Sec. II item 2: at least
// MinPts points within eps); copies the counts out if asked.  parent[i]
// becomes -1 for a point that is not core (only cores enter the forest),
// so the edge merge learns both ends' core flags from the two parent
// loads that start a union (four scattered loads per pair become two:
// merges 6-12% faster, a pruned set's 14-25%).  Each
// workgroup takes 1024 consecutive points, four per thread (one 16-byte
// load of counts, one 4-byte store of flags), and writes the number of
// core points among them to sums[block]: no atomics (one same-address
// atomic per wave serialised this pass at 1M points).  k_scan_totals then
// turns the totals into offsets and the core count.  n_pad is a multiple
// of 1024, so every workgroup is full.
__global__ __launch_bounds__(256) void k_core(
    const unsigned* __restrict__ count, int64_t n, int min_pts,
    unsigned char* __restrict__ core, int* __restrict__ parent,
    int* __restrict__ counts_out, bool out_vec, unsigned* __restrict__ sums) {
  __shared__ unsigned sh[4];
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x * 4;
  const uint4 c4 = *reinterpret_cast<const uint4*>(count + base);
  const unsigned c[4] = {c4.x, c4.y, c4.z, c4.w};
  unsigned flags = 0, mine = 0;
  int par[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const unsigned is_core = base + q < n && c[q] >= (unsigned)min_pts;
    flags |= is_core << (8 * q);
    mine += is_core;
    par[q] = is_core ? (int)(base + q) : -1;
  }
  *reinterpret_cast<unsigned*>(core + base) = flags;
  *reinterpret_cast<int4*>(parent + base) = make_int4(par[0], par[1], par[2], par[3]);
  if (counts_out != nullptr) {
    if (out_vec && base + 4 <= n) {
      *reinterpret_cast<int4*>(counts_out + base) =
          make_int4((int)c[0], (int)c[1], (int)c[2], (int)c[3]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (base + q < n) counts_out[base + q] = (int)c[q];
    }
  }
  unsigned tot;
  block_excl_scan(mine, sh, &tot);
  if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

// Exclusive scan of the per-block core totals in place, by one workgroup;
// the total is the number of core points.
__global__ __launch_bounds__(256) void k_scan_totals(unsigned* sums,
                                                     int64_t nblk,
                                                     Status* st) {
  __shared__ unsigned sh[4];
  unsigned carry = 0;
  for (int64_t b0 = 0; b0 < nblk; b0 += 256) {
    const int64_t b = b0 + threadIdx.x;
    const unsigned v = b < nblk ? sums[b] : 0u;
    unsigned tot;
    const unsigned ex = block_excl_scan(v, sh, &tot);
    if (b < nblk) sums[b] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    st->n_core = carry;
    st->n_core_list = carry;
  }
}

hipError_t launch_core(const Layout& L, int min_pts, int* counts_out,
                       hipStream_t s) {
  const int64_t nblk = L.n_pad / 1024;
  const bool out_vec = ((uintptr_t)counts_out & 15u) == 0;
  k_core<<<(unsigned)nblk, 256, 0, s>>>(L.count, L.n, min_pts, L.core,
                                        L.parent, counts_out, out_vec,
                                        L.block_sums);
  k_scan_totals<<<1, 256, 0, s>>>(L.block_sums, nblk, L.status);
  return hipGetLastError();
}

// ---- labels ----------------------------------------------------------------
// Every core point finds its root, which is the smallest core of its
// component (a root is only ever hung under a smaller root).  A border
// point takes the root of its lowest-index core neighbour.  A cluster's
// label is its smallest member: the root itself, unless a border point
// with a smaller index joined it; only such border points touch cmin[]
// (atomicMin), so no atomic is spent on cores.  Roots are kept in bmin[]
// (unused for cores until now) for the label pass.
__global__ void k_finalize(int64_t n, const unsigned char* __restrict__ core,
                           int* __restrict__ parent, int* __restrict__ bmin,
                           int* __restrict__ cmin) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    if (core[i]) {
      bmin[i] = uf_find(parent, (int)i);
    } else {
      const int b = bmin[i];
      if (b == INT_MAX) continue;
      const int r = uf_find(parent, b);
      bmin[i] = r;
      if (i < r) atomicMin(cmin + r, (int)i);
    }
  }
}

__global__ void k_write_labels(int64_t n, const int* __restrict__ bmin,
                               const int* __restrict__ cmin,
                               int* __restrict__ labels) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int r = bmin[i];
    if (r == INT_MAX) {
      labels[i] = -1;
    } else {
      const int c = cmin[r];
      labels[i] = c < r ? c : r;
    }
  }
}

hipError_t launch_label(const Layout& L, int* labels, hipStream_t s) {
  k_finalize<<<grid_for(L.n, 256 * 4), 256, 0, s>>>(L.n, L.core, L.parent,
                                                    L.bmin, L.cmin);
  k_write_labels<<<grid_for(L.n, 256 * 4), 256, 0, s>>>(L.n, L.bmin, L.cmin,
                                                        labels);
  return hipGetLastError();
}

}  // namespace dbk

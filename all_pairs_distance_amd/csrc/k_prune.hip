// Exact tile pruning for the neighbour-count pass (an opt-in mode).
//
// The points are put in a locality-preserving order (a Morton key over the
// first min(d,3) coordinates, or, for points of 16 or more dimensions, over
// six principal directions, sorted), each block of T consecutive sorted
// points gets its bounding box, and a block pair (I, J) is skipped when the
// boxes are provably farther apart than eps in the same fp32 arithmetic the
// distance uses:
//   G_k = fl(lo_J,k - hi_I,k) (or the mirror) when the boxes are apart in
//   dimension k, else 0; Gs = (((fl(G_0^2) + fl(G_1^2)) + fl(G_2^2)) ...)
//   summed in ascending k with every step rounded.
// For x in block I and y in block J, |x_k - y_k| >= the real gap, rounding
// is monotone, so |fl(x_k - y_k)| >= G_k, fl(t^2) >= fl(G_k^2), and each
// rounded partial sum of the true distance is >= the matching partial sum
// of Gs.  Gs > eps2 therefore implies d2(x,y) > eps2 for every pair of the
// two blocks: no neighbour is ever skipped, and counts, captured pairs and
// labels stay bit-identical to the unpruned pass.
//
// This follows the domain partitioning of CUDAScan as described by Wang et
// al., Sec. III (blocks of nearby points handled together), restated as a
// pruning rule on the all-pairs tiles.
#include <climits>

#include "device.h"
#include "internal.h"

namespace dbk {

static unsigned grid_for_p(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (unsigned)(g < kMaxGrid ? g : kMaxGrid);
}

// float <-> order-preserving unsigned
__device__ __forceinline__ unsigned ord_u(float f) {
  unsigned b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float ord_f(unsigned u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Most coordinates a sort key covers.
constexpr int kKeyDims = 6;

// Key sort: 8-bit digits of 32-bit keys.
constexpr int kSortPasses = 4;

// ---- sort key of wide points: principal directions --------------------
// For points of 16 or more dimensions the key covers the coordinates along
// the six leading principal directions of a strided sample of the points,
// plus one bit that sets apart points far off those directions (squared
// residual above the sample's mean): on embedded blobs with uniform noise
// the noise then sorts apart from the blobs and the blobs' blocks stay
// compact.  Only the order depends on it; the box bound decides.
constexpr int kPcaSample = 1024;
constexpr int kPcaIters = 30;

// Sum over the wave by an xor butterfly (partners 32, 16, 8, 4, 2, 1, in
// that order; both partners of a step form the same sum, so every lane
// ends with the same total).  Only the step across the two halves goes
// through the LDS crossbar; 16 is a swizzle within each half, and 8, 4, 2
// and 1 are DPP moves within rows of 16 (4: two half-row moves under
// bank masks).
template <int CTRL>
__device__ __forceinline__ float xor_lane_dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v += __shfl_xor(v, 32);
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401f));
  v += xor_lane_dpp<0x128>(v);  // row_ror:8 (lane ^ 8 within a row)
  {
    // lane ^ 4: banks 0 and 2 read 4 lanes up, banks 1 and 3 4 lanes down
    int t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x104, 0xf, 0x5,
                                        false);
    t = __builtin_amdgcn_update_dpp(t, __float_as_int(v), 0x114, 0xf, 0xa,
                                    false);
    v += __int_as_float(t);
  }
  v += xor_lane_dpp<0x4e>(v);   // quad_perm 2,3,0,1 (lane ^ 2)
  v += xor_lane_dpp<0xb1>(v);   // quad_perm 1,0,3,2 (lane ^ 1)
  return v;
}

// One workgroup of 256 threads.  out: the sample mean [S], then kKeyDims
// orthonormal directions [S each], then the sample's mean squared residual
// off them.
__global__ __launch_bounds__(256) void k_pca(const float* __restrict__ pts,
                                             int64_t n, int S, int d,
                                             float* __restrict__ out) {
  __shared__ float tile[64][65];
  __shared__ float mean[64];
  __shared__ float cov[64][65];
  __shared__ float vs[kKeyDims][64];
  const int tid = threadIdx.x;
  const int64_t m = n < kPcaSample ? n : kPcaSample;
  const int64_t step = n / m;
  // The sample in blocks of 64 points: thread t holds coordinate t % 64
  // of points t / 64 + 4q (q < 16) of a block, and the next block's loads
  // are issued before the current block is summed.
  const int kk = tid & 63, r0 = tid >> 6;
  float buf[16];
  const auto load_block = [&](int64_t s0) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t smp = s0 + r0 + 4 * q;
      buf[q] = (smp < m && kk < d) ? pts[smp * step * S + kk] : 0.f;
    }
  };
  // sample mean
  float msum = 0.f;
  load_block(0);
  for (int64_t s0 = 0; s0 < m; s0 += 64) {
#pragma unroll
    for (int q = 0; q < 16; ++q) tile[r0 + 4 * q][kk] = buf[q];
    __syncthreads();
    if (s0 + 64 < m) load_block(s0 + 64);
    if (tid < 64)
      for (int r = 0; r < 64; ++r) msum += tile[r][tid];
    __syncthreads();
  }
  if (tid < 64) mean[tid] = msum / (float)m;
  __syncthreads();
  // scatter matrix of the centred sample; each thread a 4 x 4 block
  const int k0 = 4 * (tid >> 4), l0 = 4 * (tid & 15);
  float c[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) c[i][j] = 0.f;
  load_block(0);
  for (int64_t s0 = 0; s0 < m; s0 += 64) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t smp = s0 + r0 + 4 * q;
      tile[r0 + 4 * q][kk] = (smp < m && kk < d) ? buf[q] - mean[kk] : 0.f;
    }
    __syncthreads();
    if (s0 + 64 < m) load_block(s0 + 64);
    for (int r = 0; r < 64; ++r) {
      float a[4], b[4];
      for (int i = 0; i < 4; ++i) {
        a[i] = tile[r][k0 + i];
        b[i] = tile[r][l0 + i];
      }
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) c[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) cov[k0 + i][l0 + j] = c[i][j];
  __syncthreads();
  // subspace iteration in wave 0: lane k holds component k of every
  // direction; V <- orth(C V), modified Gram-Schmidt
  if (tid < 64) {
    const int k = tid;
    float v[kKeyDims];
    for (int j = 0; j < kKeyDims; ++j)   // a fixed full-rank start
      v[j] = (k == j ? 4.f : 0.f) + (float)((k * (2 * j + 3) + j) % 7) - 3.f;
    for (int it = 0; it < kPcaIters; ++it) {
      for (int j = 0; j < kKeyDims; ++j) vs[j][k] = v[j];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float w[kKeyDims];
      for (int j = 0; j < kKeyDims; ++j) {
        float acc = 0.f;
        for (int l = 0; l < 64; ++l) acc += cov[k][l] * vs[j][l];
        w[j] = acc;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int j = 0; j < kKeyDims; ++j) {
        for (int i = 0; i < j; ++i) {
          const float dot = wave_sum_f(w[j] * v[i]);
          w[j] -= dot * v[i];
        }
        const float nrm = sqrtf(wave_sum_f(w[j] * w[j]));
        v[j] = nrm > 0.f ? w[j] / nrm : 0.f;
      }
    }
    // mean squared residual = (trace C - sum_j v_j' C v_j) / m
    float cv[kKeyDims];
    for (int j = 0; j < kKeyDims; ++j) vs[j][k] = v[j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float captured = 0.f;
    for (int j = 0; j < kKeyDims; ++j) {
      float acc = 0.f;
      for (int l = 0; l < 64; ++l) acc += cov[k][l] * vs[j][l];
      cv[j] = acc;
      captured += v[j] * cv[j];
    }
    captured = wave_sum_f(captured);
    const float trace = wave_sum_f(cov[k][k]);
    if (k < S) {
      out[k] = mean[k];
      for (int j = 0; j < kKeyDims; ++j) out[(1 + j) * S + k] = k < d ? v[j] : 0.f;
    }
    if (k == 0) out[(1 + kKeyDims) * S] = (trace - captured) / (float)m;
  }
}

// The KD key coordinates of point p: its first KD coordinates, or (with a
// principal-direction table) its coordinates along those directions and
// its squared residual off them.
__device__ __forceinline__ void key_coords(const float* __restrict__ p, int KD,
                                           int d, int S,
                                           const float* __restrict__ pca,
                                           float* y, float* r2) {
  if (pca == nullptr) {
    for (int k = 0; k < KD; ++k) y[k] = p[k];
    *r2 = 0.f;
    return;
  }
  float tot = 0.f;
  for (int j = 0; j < kKeyDims; ++j) y[j] = 0.f;
  for (int k = 0; k < d; ++k) {
    const float c = p[k] - pca[k];
    tot += c * c;
    for (int j = 0; j < kKeyDims; ++j) y[j] += c * pca[(1 + j) * S + k];
  }
  float cap = 0.f;
  for (int j = 0; j < kKeyDims; ++j) cap += y[j] * y[j];
  *r2 = tot - cap;
}

// Global min/max of the first KD coordinates of the real points
// (lohi: KD minima, then KD maxima, order-encoded).  Reduced per wave with
// shuffles, then per workgroup in LDS, so each workgroup issues one atomic
// per bound: one per wave on these 2*KD words serialised the pass.
__global__ __launch_bounds__(256) void k_bbox(
    const float* __restrict__ pts, int64_t n, int S, int KD, int d,
    const float* __restrict__ pca, unsigned* __restrict__ lohi) {
  __shared__ unsigned sh[4][2 * kKeyDims];
  unsigned lo[kKeyDims], hi[kKeyDims];
  for (int k = 0; k < kKeyDims; ++k) {
    lo[k] = ~0u;
    hi[k] = 0u;
  }
  // four points per thread and step, their loads issued together
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i0 < n;
       i0 += 4 * stride) {
    float y[4][kKeyDims], r2;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n) key_coords(pts + i * S, KD, d, S, pca, y[u], &r2);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (i0 + u * stride >= n) break;
      for (int k = 0; k < KD; ++k) {
        const unsigned v = ord_u(y[u][k]);
        lo[k] = v < lo[k] ? v : lo[k];
        hi[k] = v > hi[k] ? v : hi[k];
      }
    }
  }
  const int wave = threadIdx.x >> 6;
  for (int k = 0; k < KD; ++k) {
    unsigned a = lo[k], b = hi[k];
    for (int off = 32; off > 0; off >>= 1) {
      const unsigned oa = __shfl_xor(a, off), ob = __shfl_xor(b, off);
      a = oa < a ? oa : a;
      b = ob > b ? ob : b;
    }
    if (lane_id() == 0) {
      sh[wave][k] = a;
      sh[wave][KD + k] = b;
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 2 * KD) {
    unsigned v = sh[0][t];
    for (int w = 1; w < 4; ++w) {
      const unsigned o = sh[w][t];
      v = t < KD ? (o < v ? o : v) : (o > v ? o : v);
    }
    if (t < KD) atomicMin(lohi + t, v);
    else atomicMax(lohi + t, v);
  }
}

// Also clears the key sort's digit totals (kSortPasses * 256 words).
__global__ void k_bbox_init(unsigned* lohi, int KD, unsigned* totals) {
  if ((int)threadIdx.x < KD) lohi[threadIdx.x] = ~0u;
  else if ((int)threadIdx.x < 2 * KD) lohi[threadIdx.x] = 0u;
  for (int i = threadIdx.x; i < kSortPasses * 256; i += blockDim.x)
    totals[i] = 0u;
}

// Spread the low 10 bits of v to every third bit.
__device__ __forceinline__ unsigned spread3(unsigned v) {
  v &= 0x3ffu;
  v = (v | (v << 16)) & 0x030000ffu;
  v = (v | (v << 8)) & 0x0300f00fu;
  v = (v | (v << 4)) & 0x030c30c3u;
  v = (v | (v << 2)) & 0x09249249u;
  return v;
}
// Spread the low 15 bits of v to every second bit.
__device__ __forceinline__ unsigned spread2(unsigned v) {
  v &= 0x7fffu;
  v = (v | (v << 8)) & 0x00ff00ffu;
  v = (v | (v << 4)) & 0x0f0f0f0fu;
  v = (v | (v << 2)) & 0x33333333u;
  v = (v | (v << 1)) & 0x55555555u;
  return v;
}

// Sort keys: d = 1 sorts by the value itself; otherwise a Morton code over
// the bounding box of the KD key coordinates: 15 bits each for 2, 10 for 3,
// 5 for 6.  Padding rows get the largest key (they sort last, after every
// real point).
__global__ void k_keys(const float* __restrict__ pts, int64_t n, int64_t n_pad,
                       int S, int KD, int d, const float* __restrict__ pca,
                       const unsigned* __restrict__ lohi,
                       unsigned* __restrict__ keys, int* __restrict__ idx) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n_pad;
       i += (int64_t)gridDim.x * blockDim.x) {
    unsigned key = 0xffffffffu;
    if (i < n) {
      if (KD == 1) {
        key = ord_u(pts[i * S]) >> 1;  // order kept, below the padding key
      } else {
        const int bits = 30 / KD;
        const float cells = (float)((1 << bits) - 1);
        float y[kKeyDims], r2;
        key_coords(pts + i * S, KD, d, S, pca, y, &r2);
        unsigned q[kKeyDims];
        for (int k = 0; k < KD; ++k) {
          const float lo = ord_f(lohi[k]), hi = ord_f(lohi[KD + k]);
          const float span = hi - lo;
          float f = span > 0.f ? (y[k] - lo) / span * cells : 0.f;
          f = f < 0.f ? 0.f : (f > cells ? cells : f);
          q[k] = (unsigned)f;
        }
        if (KD == 2) {
          key = spread2(q[0]) | (spread2(q[1]) << 1);
        } else if (KD == 3) {
          key = spread3(q[0]) | (spread3(q[1]) << 1) | (spread3(q[2]) << 2);
        } else {
          // bit b of coordinate k goes to bit KD*b + k
          key = 0;
          for (int b = 0; b < bits; ++b)
            for (int k = 0; k < KD; ++k)
              key |= ((q[k] >> b) & 1u) << (KD * b + k);
          // far off the principal directions: after every point near them
          if (pca != nullptr && r2 > pca[(1 + kKeyDims) * S]) key |= 1u << 31;
        }
      }
    }
    keys[i] = key;
    idx[i] = (int)i;
  }
}

// sorted_pts[s] = pts[perm[s]]
__global__ void k_gather(const float* __restrict__ pts,
                         const int* __restrict__ perm, int64_t total, int S,
                         float* __restrict__ out) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t s = e / S;
    const int k = (int)(e - s * S);
    out[e] = pts[(int64_t)perm[s] * S + k];
  }
}

// Bounding box of each block of T sorted points over all S coordinates;
// padding rows are skipped, an all-padding block gets lo > hi.  Thread t
// takes coordinate t % S of every G-th point of the block from point t / S
// on (G = 256 / S groups), so a group reads whole rows, coalesced; the G
// partial boxes are then combined in LDS.
__global__ __launch_bounds__(256) void k_block_boxes(
    const float* __restrict__ spts, const int* __restrict__ perm, int64_t n,
    int T, int S, float* __restrict__ boxes) {
  __shared__ float part_lo[256], part_hi[256];
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x, G = 256 / S, k = t % S, g = t / S;
  float lo = __builtin_inff(), hi = -__builtin_inff();
  if (g < G) {
    for (int q = g; q < T; q += G) {
      const int64_t s = b * T + q;
      if (perm[s] < n) {
        const float v = spts[s * S + k];
        lo = v < lo ? v : lo;
        hi = v > hi ? v : hi;
      }
    }
  }
  part_lo[t] = lo;
  part_hi[t] = hi;
  __syncthreads();
  if (t < S) {
    for (int j = 1; j < G; ++j) {
      const float l = part_lo[j * S + t], h = part_hi[j * S + t];
      lo = l < lo ? l : lo;
      hi = h > hi ? h : hi;
    }
    boxes[(b * 2) * S + t] = lo;
    boxes[(b * 2 + 1) * S + t] = hi;
  }
}

// Boxes of blocks of F consecutive 64-point groups from the groups' own
// boxes: minima and maxima are exact, so these are the boxes of the points
// themselves (an all-padding group, lo > hi, adds nothing).
__global__ void k_box_union(const float* __restrict__ in, int64_t nb_out,
                            int F, int S, float* __restrict__ out) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
       e < nb_out * S; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = e / S;
    const int k = (int)(e - b * S);
    float lo = __builtin_inff(), hi = -__builtin_inff();
    for (int f = 0; f < F; ++f) {
      const float* src = in + (b * F + f) * 2 * S;
      const float l = src[k], h = src[S + k];
      lo = l < lo ? l : lo;
      hi = h > hi ? h : hi;
    }
    out[(b * 2) * S + k] = lo;
    out[(b * 2 + 1) * S + k] = hi;
  }
}

// ---- key sort ---------------------------------------------------------------
// A least-significant-digit radix sort of the (key, index) pairs: four
// stable passes over 8-bit digits.  A pass cuts the keys into tiles of
// 256 * ITEMS consecutive keys and runs three kernels:
//   k_sort_hist     each tile counts its digits into hist[d * tiles + t];
//   k_sort_offsets  one work-group per digit d rewrites its row of counts
//                   as the output position of tile t's first key of digit
//                   d: the keys of every digit below d, plus the keys of
//                   digit d in the tiles before t;
//   k_sort_scatter  each tile writes its keys, in input order, from there.
// Equal digits keep their input order, so every pass is stable, and after
// the four the keys ascend with equal keys in their input (index) order.
// The digit totals do not depend on the order of the keys: the first
// pass's histogram kernel sums them for all four passes.

// lanes of this wave holding the same digit as this lane, valid lanes only
// (0 for an invalid lane): eight ballots, one per digit bit
__device__ __forceinline__ uint64_t same_digit(unsigned dig, bool valid) {
  uint64_t peers = ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (dig >> b) & 1u;
    const uint64_t ones = ballot(bit);
    peers &= bit ? ones : ~ones;
  }
  return valid ? peers : 0ull;
}

template <int ITEMS, bool TOTALS>
__global__ __launch_bounds__(256) void k_sort_hist(
    const unsigned* __restrict__ keys, int64_t n, int shift, int64_t tiles,
    unsigned* __restrict__ hist, unsigned* __restrict__ totals) {
  constexpr int H = TOTALS ? kSortPasses * 256 : 256;
  __shared__ unsigned h[H];
  for (int i = threadIdx.x; i < H; i += 256) h[i] = 0u;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * 256 * ITEMS;
  unsigned k[ITEMS];
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int64_t g = base + r * 256 + threadIdx.x;
    k[r] = g < n ? keys[g] : 0u;
  }
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    if (base + r * 256 + threadIdx.x >= n) continue;
    if (TOTALS) {
#pragma unroll
      for (int p = 0; p < kSortPasses; ++p)
        atomicAdd(&h[p * 256 + ((k[r] >> (8 * p)) & 255u)], 1u);
    } else {
      atomicAdd(&h[(k[r] >> shift) & 255u], 1u);
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  hist[(int64_t)t * tiles + blockIdx.x] = h[(TOTALS ? shift / 8 * 256 : 0) + t];
  if (TOTALS) {
    for (int i = t; i < H; i += 256)
      if (h[i]) atomicAdd(&totals[i], h[i]);
  }
}

// grid: 256 work-groups, one per digit; totals: this pass's 256 digit counts
__global__ __launch_bounds__(256) void k_sort_offsets(
    const unsigned* __restrict__ totals, int64_t tiles,
    unsigned* __restrict__ hist) {
  __shared__ unsigned sh[4];
  __shared__ unsigned first;
  const int dig = blockIdx.x;
  unsigned all;
  const unsigned below = block_excl_scan(totals[threadIdx.x], sh, &all);
  if ((int)threadIdx.x == dig) first = below;
  __syncthreads();
  unsigned run = first;
  unsigned* row = hist + (int64_t)dig * tiles;
  for (int64_t b = 0; b < tiles; b += 256) {
    const int64_t i = b + threadIdx.x;
    const unsigned v = i < tiles ? row[i] : 0u;
    unsigned sum;
    const unsigned ex = block_excl_scan(v, sh, &sum);
    if (i < tiles) row[i] = run + ex;
    run += sum;
  }
}

// Rounds of 256 keys in input order (thread t: key r*256 + t of the tile):
// a key's place is its digit's running position, plus the keys of that
// digit in lower waves of the round, plus those in lower lanes of its wave.
template <int ITEMS>
__global__ __launch_bounds__(256) void k_sort_scatter(
    const unsigned* __restrict__ kin, const int* __restrict__ vin, int64_t n,
    int shift, int64_t tiles, const unsigned* __restrict__ offs,
    unsigned* __restrict__ kout, int* __restrict__ vout) {
  __shared__ unsigned pos[256];
  __shared__ unsigned wcnt[4][256];
  const int t = threadIdx.x, wave = t >> 6;
  pos[t] = offs[(int64_t)t * tiles + blockIdx.x];
#pragma unroll
  for (int w = 0; w < 4; ++w) wcnt[w][t] = 0u;
  const int64_t base = (int64_t)blockIdx.x * 256 * ITEMS;
  unsigned k[ITEMS];
  int v[ITEMS];
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int64_t g = base + r * 256 + t;
    k[r] = g < n ? kin[g] : 0u;
    v[r] = g < n ? vin[g] : 0;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const bool valid = base + r * 256 + t < n;
    const unsigned dig = (k[r] >> shift) & 255u;
    const uint64_t peers = same_digit(dig, valid);
    const unsigned lower = bits_below(peers);
    if (valid && lower == 0) wcnt[wave][dig] = (unsigned)__popcll(peers);
    __syncthreads();
    if (valid) {
      unsigned p = pos[dig] + lower;
      for (int w = 0; w < wave; ++w) p += wcnt[w][dig];
      // always below n when the counts are consistent; the test keeps a
      // mistake from writing outside the buffers
      if (p < (uint64_t)n) {
        kout[p] = k[r];
        vout[p] = v[r];
      }
    }
    __syncthreads();
    pos[t] += wcnt[0][t] + wcnt[1][t] + wcnt[2][t] + wcnt[3][t];
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w][t] = 0u;
    __syncthreads();
  }
}

__device__ __forceinline__ void tile_coords_p(int64_t t, int64_t nb, int64_t& I,
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

// Keep block pair (I, J), I <= J, unless the fp32 box-gap bound exceeds
// eps2.  Kept pairs are appended to the list (any order).
__global__ void k_tile_list(const float* __restrict__ boxes, int64_t nb, int S,
                            float eps2, uint2* __restrict__ list,
                            unsigned long long cap, Status* __restrict__ st) {
  const int64_t tiles = nb * (nb + 1) / 2;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < tiles;
       t += (int64_t)gridDim.x * blockDim.x) {
    int64_t I, J;
    tile_coords_p(t, nb, I, J);
    const float* bi = boxes + I * 2 * S;
    const float* bj = boxes + J * 2 * S;
    bool keep = bi[0] <= bi[S] && bj[0] <= bj[S];  // both blocks hold points
    if (keep && I != J) {
      // the gap of dimension k, squared, added in ascending k
      float s = 0.f;
      const auto add = [&s](int k, float loi, float hii, float loj, float hij) {
        float g = 0.f;
        if (loj > hii) g = loj - hii;
        else if (loi > hij) g = loi - hij;
        const float q = g * g;
        s = k == 0 ? q : s + q;
      };
      if (S % 4 == 0) {
        // four dimensions a load, several loads in flight (the rows are
        // 16-byte aligned: S is a multiple of 4 and the area 256-aligned)
        const float4* li = reinterpret_cast<const float4*>(bi);
        const float4* hi = reinterpret_cast<const float4*>(bi + S);
        const float4* lj = reinterpret_cast<const float4*>(bj);
        const float4* hj = reinterpret_cast<const float4*>(bj + S);
#pragma unroll 4
        for (int k4 = 0; k4 < S / 4; ++k4) {
          const float4 a = li[k4], b = hi[k4], c = lj[k4], e = hj[k4];
          add(4 * k4, a.x, b.x, c.x, e.x);
          add(4 * k4 + 1, a.y, b.y, c.y, e.y);
          add(4 * k4 + 2, a.z, b.z, c.z, e.z);
          add(4 * k4 + 3, a.w, b.w, c.w, e.w);
        }
      } else {
        for (int k = 0; k < S; ++k) add(k, bi[k], bi[S + k], bj[k], bj[S + k]);
      }
      keep = !(s > eps2);
    }
    if (keep) {
      const unsigned long long slot = atomicAdd(&st->n_tiles, 1ull);
      if (slot < cap) list[slot] = make_uint2((unsigned)I, (unsigned)J);
    }
  }
}

// Keys per thread per tile: 16 from 786,432 keys on (192 or more tiles of
// 4,096), else 4 (more, smaller tiles).  Measured (layout, sort and boxes
// of a pruned fit): 50k x 2 0.146 -> 0.103 ms and 200k x 8 0.171 -> 0.143
// ms with 4; 1M x 3 0.246 ms with 16, 0.274 with 4.
static int sort_items(int64_t n_pad) { return n_pad >= 3 * (1 << 18) ? 16 : 4; }

static int64_t sort_tiles(int64_t n_pad) {
  const int64_t tile = 256 * (int64_t)sort_items(n_pad);
  return (n_pad + tile - 1) / tile;
}

size_t prune_sort_bytes(int64_t n_pad) {
  // the digit totals of the four passes, then one pass's tile counts
  return ((size_t)kSortPasses * 256 + 256 * (size_t)sort_tiles(n_pad)) *
         sizeof(unsigned);
}

hipError_t launch_prune(const Layout& L, int T, float eps2, hipStream_t s) {
  // wide points: six key coordinates separate the blocks better than three
  // (measured on 64-d embedded blobs: 30% fewer block pairs kept)
  const bool wide = L.d >= 16;
  const int KD = wide ? kKeyDims : (L.d < 3 ? L.d : 3);
  const float* pca = wide ? L.pca : nullptr;
  if (wide) k_pca<<<1, 256, 0, s>>>(L.pts, L.n, L.stride, L.d, L.pca);
  unsigned* totals = L.sort_hist;
  unsigned* hist = L.sort_hist + kSortPasses * 256;
  k_bbox_init<<<1, 256, 0, s>>>(L.bbox, KD, totals);
  // at most 512 work-groups (one atomic per bound each), 4+ points per
  // thread
  const unsigned bgrid = grid_for_p(L.n, 256 * 4);
  k_bbox<<<bgrid < 512 ? bgrid : 512, 256, 0, s>>>(L.pts, L.n, L.stride, KD,
                                                     L.d, pca, L.bbox);
  // the keys and indices start where the fourth pass leaves them
  k_keys<<<grid_for_p(L.n_pad, 256 * 4), 256, 0, s>>>(
      L.pts, L.n, L.n_pad, L.stride, KD, L.d, pca, L.bbox, L.keys_out,
      L.perm);
  const int64_t tiles_s = sort_tiles(L.n_pad);
  unsigned* ks = L.keys_out;
  int* vs = L.perm;
  unsigned* kd = L.keys_in;
  int* vd = L.idx_in;
  const bool wide_tiles = sort_items(L.n_pad) == 16;
  for (int p = 0; p < kSortPasses; ++p) {
#define DBK_SORT_PASS(IT)                                                   \
  do {                                                                      \
    if (p == 0)                                                             \
      k_sort_hist<IT, true><<<(unsigned)tiles_s, 256, 0, s>>>(              \
          ks, L.n_pad, 0, tiles_s, hist, totals);                           \
    else                                                                    \
      k_sort_hist<IT, false><<<(unsigned)tiles_s, 256, 0, s>>>(             \
          ks, L.n_pad, 8 * p, tiles_s, hist, nullptr);                      \
    k_sort_offsets<<<256, 256, 0, s>>>(totals + 256 * p, tiles_s, hist);    \
    k_sort_scatter<IT><<<(unsigned)tiles_s, 256, 0, s>>>(                   \
        ks, vs, L.n_pad, 8 * p, tiles_s, hist, kd, vd);                     \
  } while (0)
    if (wide_tiles) DBK_SORT_PASS(16);
    else DBK_SORT_PASS(4);
#undef DBK_SORT_PASS
    unsigned* tk = ks;
    ks = kd;
    kd = tk;
    int* tv = vs;
    vs = vd;
    vd = tv;
  }
  k_gather<<<grid_for_p(L.n_pad * L.stride, 256 * 8), 256, 0, s>>>(
      L.pts, L.perm, L.n_pad * L.stride, L.stride, L.sorted_pts);
  const int64_t nb = L.n_pad / T;
  // boxes of the 64-point row groups (tested inside the count pass), then
  // from them those of the 64*P columns one wave holds and of the blocks
  k_block_boxes<<<(unsigned)(L.n_pad / 64), 256, 0, s>>>(
      L.sorted_pts, L.perm, L.n, 64, L.stride, L.boxes64);
  const int64_t nw = L.n_pad / (T / 4);
  k_box_union<<<grid_for_p(nw * L.stride, 256), 256, 0, s>>>(
      L.boxes64, nw, T / 4 / 64, L.stride, L.boxes_w);
  k_box_union<<<grid_for_p(nb * L.stride, 256), 256, 0, s>>>(
      L.boxes64, nb, T / 64, L.stride, L.boxes);
  const int64_t tiles = nb * (nb + 1) / 2;
  k_tile_list<<<grid_for_p(tiles, 256), 256, 0, s>>>(
      L.boxes, nb, L.stride, eps2, L.tiles, L.tile_cap, L.status);
  return hipGetLastError();
}

}  // namespace dbk

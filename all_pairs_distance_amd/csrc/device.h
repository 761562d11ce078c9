// Device helpers: the fixed fp32 distance, wave64 primitives and the
// lock-free union-find used by the merge kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dbk {

// Squared distance, dimensions in ascending order, each subtraction,
// square and addition rounded on its own (the library is compiled with
// -ffp-contract=off, so no multiply-add is formed).  The first square is
// the first partial sum: adding it to +0 would return it unchanged.
// (Wang et al., Sec. IV-A: compare the squared distance with eps^2.)
template <int D>
__device__ __forceinline__ float dist2(const float* a, const float* b) {
  float t = a[0] - b[0];
  float s = t * t;
#pragma unroll
  for (int k = 1; k < D; ++k) {
    float u = a[k] - b[k];
    float q = u * u;
    s = s + q;
  }
  return s;
}

// The hoisted-norm form of Wang et al. Sec. IV-B2 as a fixed binary32
// evaluation: with ta = |a|^2 and pb = |b|^2 given (rounded squares summed
// in k order), the products (2 a_k) b_k (doubling is exact) rounded and
// summed in k order, then ta + pb, then the subtraction.  Padding dims are
// zero on both sides; their +-0 products leave the result unchanged.
template <int D>
__device__ __forceinline__ float expanded_d2(const float* a, const float* b,
                                             float ta, float pb) {
  float inner = (2.f * a[0]) * b[0];
#pragma unroll
  for (int k = 1; k < D; ++k) {
    const float q = (2.f * a[k]) * b[k];
    inner = inner + q;
  }
  const float s = ta + pb;
  return s - inner;
}

// Item visited at step `step` of `count` under a walk (mul, add); see the
// Walk type.  Products stay below 2^63: |mul| < 2^14 and count < 2^49.
__device__ __forceinline__ int64_t walk_item(int64_t step, int64_t count,
                                             int64_t mul, int64_t add) {
  if (mul == 1) return step;
  const int64_t v = (mul * step + add) % count;
  return v < 0 ? v + count : v;
}

// The same walk re-fitted to another count (a pruned launch learns its
// item count on the device): reverse stays reverse, a shuffle moves to the
// next multiplier coprime with the new count.
__device__ __forceinline__ void walk_refit(int64_t count, int64_t& mul,
                                           int64_t& add) {
  if (mul == 1 || count <= 1) {
    mul = 1;
    add = 0;
    return;
  }
  if (mul == -1) {
    add = count - 1;
    return;
  }
  for (;;) {
    int64_t a = mul, b = count;
    while (b != 0) {
      const int64_t r = a % b;
      a = b;
      b = r;
    }
    if (a == 1) break;
    mul = mul + 1 < 16384 ? mul + 1 : 3;
  }
  add %= count;
}

// Read-only global memory seen through the constant address space: loads
// from wave-uniform addresses through such a pointer become scalar loads.
typedef const float __attribute__((address_space(4)))* const_float_ptr;
typedef const int __attribute__((address_space(4)))* const_int_ptr;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint64_t ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}

// Number of set bits of m below this lane.
__device__ __forceinline__ unsigned bits_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

// Write a wave-uniform value into one lane of a VGPR (v_writelane_b32);
// `lane` must be wave-uniform.  gfx9 reads at most one SGPR per VALU op
// besides M0, so the lane select is passed in M0.
__device__ __forceinline__ int write_lane(int vgpr, int value, int lane) {
  asm("v_writelane_b32 %0, %1, m0" : "+v"(vgpr) : "s"(value), "{m0}"(lane));
  return vgpr;
}

// cnt + (bit `lane` of mask) in one VALU op: v_addc with the wave-uniform
// mask (an SGPR pair) as the carry-in.  Left to itself the compiler may
// spend a v_cndmask and a v_add on it.  The compiler keeps two wait states
// between a VALU write of an SGPR pair and a VALU read of it as a lane
// mask, but cannot see into this asm, and the mask is usually written by a
// compare just before: the s_nop supplies those two wait states.
__device__ __forceinline__ unsigned add_lane_bit(unsigned cnt, uint64_t mask) {
  asm("s_nop 1\n\tv_addc_co_u32_e64 %0, vcc, %0, 0, %1"
      : "+v"(cnt) : "s"(mask) : "vcc");
  return cnt;
}

// add_lane_bit for a mask that a VALU instruction wrote at least two
// instructions earlier: the wait states are already there, no padding
// (the instruction-level tests check the distance in the built kernels).
// 200k x 8 count 7.65 -> 7.58 ms with the shorter stage check beside it.
__device__ __forceinline__ unsigned add_lane_bit_far(unsigned cnt,
                                                     uint64_t mask) {
  asm("v_addc_co_u32_e64 %0, vcc, %0, 0, %1"
      : "+v"(cnt) : "s"(mask) : "vcc");
  return cnt;
}

// 2*v + (bit `lane` of mask): shifts this lane's bit of a wave-uniform
// mask into v, one VALU op (the same add-with-carry as add_lane_bit).
__device__ __forceinline__ unsigned shift_in_lane_bit(unsigned v, uint64_t mask) {
  asm("s_nop 1\n\tv_addc_co_u32_e64 %0, vcc, %0, %0, %1"
      : "+v"(v) : "s"(mask) : "vcc");
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

__device__ __forceinline__ unsigned long long uniform_u64(unsigned long long v) {
  unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
  unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// Lower bound of the fp32 distance between any point of box a and any point
// of box b (each [lo[S], hi[S]]), in the distance's own rounded order: the
// per-dimension gap is rounded like a difference, squared and summed in
// ascending dimension.  Rounding is monotone, so every distance between
// the two boxes is >= this bound.  True when the bound exceeds eps2.
template <int S>
__device__ __forceinline__ bool boxes_apart(const_float_ptr a, const_float_ptr b,
                                            float eps2) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const float alo = a[k], ahi = a[S + k], blo = b[k], bhi = b[S + k];
    float g = 0.f;
    if (blo > ahi) g = blo - ahi;
    else if (alo > bhi) g = alo - bhi;
    const float q = g * g;
    s = k == 0 ? q : s + q;
  }
  return s > eps2;
}

// Sum of v over the 64 lanes, in some fixed tree order (each term passes
// at most 7 additions); the result is in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm 1,0,3,2
  v += dpp_f32<0x4E>(v);   // quad_perm 2,3,0,1
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror: every lane holds its 16-lane row's sum
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

// The box test of boxes_apart computed by the whole wave for wide points:
// lane k forms the rounded square of the rounded gap in dimension k, and
// the squares are summed in a tree instead of in ascending k.  thr
// (box_gap_threshold) is eps2 widened so that a tree sum above it proves
// the ascending-k sum, and so every pair's fp32 distance, above eps2.
template <int S>
__device__ __forceinline__ bool wave_boxes_apart(const float* __restrict__ a,
                                                 const float* __restrict__ b,
                                                 float thr) {
  static_assert(S <= 64, "one dimension per lane");
  const int k = lane_id();
  float q = 0.f;
  if (k < S) {
    const float alo = a[k], ahi = a[S + k], blo = b[k], bhi = b[S + k];
    float g = 0.f;
    if (blo > ahi) g = blo - ahi;
    else if (alo > bhi) g = alo - bhi;
    q = g * g;
  }
  return wave_sum_f32(q) > thr;
}

// Exclusive prefix sum over a 256-thread (4-wave) block; *total gets the
// block's sum.  sh: 4 words of LDS.
__device__ __forceinline__ unsigned block_excl_scan(unsigned v, unsigned* sh,
                                                    unsigned* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  unsigned x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    unsigned y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  unsigned wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += sh[w];
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return wbase + x - v;
}

// ---- union-find over point indices ---------------------------------------
// parent[x] <= x always: a root is only ever hung under a smaller root (by a
// device-scope CAS, which sees the current value), and path halving only
// replaces a parent by one of its ancestors.  Hence the final root of every
// component is its smallest member, independent of the order in which
// threads link.
// Loads are plain (cached) loads.  A stale value is still a pointer that was
// written at some time, and every pointer ever written goes to a strictly
// smaller index, so a walk always terminates, and it ends at a node that
// was, at some time, an ancestor: two walks that meet prove the two points
// connected, since trees only merge.  A stale "root" is caught by the CAS,
// which fails and returns the current parent; the union then continues
// from there.  Measured: 24-51% less merge time than coherent
// (agent-scope) loads on the named workloads.

__device__ __forceinline__ int uf_load(const int* p) { return *p; }

__device__ __forceinline__ void uf_store(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline int uf_find(int* parent, int x) {
  while (true) {
    int p = uf_load(parent + x);
    if (p == x) return x;
    int g = uf_load(parent + p);
    if (g == p) return p;
    uf_store(parent + x, g);  // path halving
    x = g;
  }
}

// Link the components of a and b: CAS the larger root under the smaller.
// The two walks up the forest go in lockstep, so their loads are
// independent and each step costs one round trip for both; the walk stops
// as soon as both sides reach the same node (connected) or two distinct
// roots (link them).  No pointer is rewritten on the way up: on dense
// sets every find ends at a few hot roots, and per-step stores there (path
// halving or splitting) made the merge up to 4x slower on a 50k-point set.
// Only the two start nodes are pointed at the node their walk reached,
// which keeps the trees shallow for the many later pairs that share them.
// Every such store writes a smaller node of the same set into a non-root
// (a walk only leaves a node that was seen as a non-root, and a node never
// becomes a root again), so roots still change only through the CAS.
__device__ inline void uf_union(int* parent, int a0, int b0, int pa, int pb) {
  int a = a0, b = b0;
  while (true) {
    if (pa == pb) break;  // a common ancestor: already connected
    const bool ra = pa == a, rb = pb == b;
    if (ra && rb) {
      const int hi = a > b ? a : b;
      const int lo = a > b ? b : a;
      // A cached walk often ends at a root that was hung elsewhere
      // meanwhile.  One coherent load of its parent skips such a doomed
      // CAS: device-scope CAS on a few hot words serialise.
      const int cur = __hip_atomic_load(parent + hi, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
      const int old = cur == hi ? atomicCAS(parent + hi, hi, lo) : cur;
      if (old == hi) {
        pa = pb = lo;
        break;
      }
      // hi stopped being a root meanwhile: continue from its new parent
      if (hi == a) pa = old;
      else pb = old;
      continue;
    }
    if (!ra) a = pa;
    if (!rb) b = pb;
    const int qa = ra ? pa : uf_load(parent + a);
    const int qb = rb ? pb : uf_load(parent + b);
    pa = qa;
    pb = qb;
  }
  if (a0 != pa && uf_load(parent + a0) > pa) uf_store(parent + a0, pa);
  if (b0 != pb && uf_load(parent + b0) > pb) uf_store(parent + b0, pb);
}

__device__ inline void uf_union(int* parent, int a0, int b0) {
  uf_union(parent, a0, b0, uf_load(parent + a0), uf_load(parent + b0));
}

}  // namespace dbk

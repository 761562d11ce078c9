// Screen tables for the count pass (an opt-in mode).
//
// The exact decision is D(x,y) <= eps2 with D the fp32 direct distance
// (ascending k, every operation rounded).  Wang et al. (Sec. IV-B2) hoist
// the squared norms out of the distance, T + P - 2 t.p; here that form is
// only a screen: the count pass computes
//     v = fl-chain of fused multiply-adds  n_y + sum_k (-2 x_k) * y_k
// with n_y = fl32(|y|^2), which approximates R - |x|^2, R = |x - y|^2 the
// real squared distance, and compares it with two per-row thresholds.
//
// Bounds (u = 2^-24, g_m = m u / (1 - m u), t = 2^-149):
//   direct:  R (1 - g_{D+2}) - (D+2) t <= D(x,y) <= R (1 + g_{D+2}) + (D+2) t
//            (d+2 roundings per term; a subnormal result of a subtraction is
//            exact, of a product or sum off by at most t/2)
//   screen:  |v - (R - |x|^2)| <= k (|x|^2 + |y|^2) + (D+1) t,
//            k = u + 2.01 g_D  (n_y rounded once; D fused steps each rounded
//            once, the partial sums bounded by |y|^2 + sum |2 x_k y_k|
//            <= 2|y|^2 + |x|^2)
// With L = (eps2 - (D+2) t) / (1 + g_{D+2}) and
//      H = (eps2 + (D+2) t) / (1 - g_{D+2}):
//   R <= L  implies D <= eps2;   R > H  implies D > eps2.
// Bounding |y|^2 by the largest squared norm Y of the set, each row x gets
//   lo = RD(L - |x|^2 - m(x)),  hi = RU(H - |x|^2 + m(x)),
//   m(x) = k (|x|^2 + Y) + (D+1) t  (+ 1e-12 of the magnitudes for the fp64
//          evaluation of these expressions),
// rounded down / up to fp32.  Then v <= lo proves R <= L (a neighbour) and
// v > hi proves R > H (not one); anything else is decided exactly.  |x|^2 is
// summed in fp64 from exact fp64 squares.  If any squared norm exceeds
// 2^100 (where products could overflow) every row gets lo = -inf,
// hi = +inf and zero coefficients: all pairs are then decided exactly.
// Padding rows are NaN throughout and never match.
//
// With the hoisted-norm form as the decision (DBSCAN_FLAG_EXPANDED), the
// exact value is E = fl(fl(T + P) - I): T, P the fp32 norms (rounded
// squares summed in k order), I the k-ordered sum of the rounded products
// (2 x_k) y_k.  Each of T, P and I passes at most D roundings and T + P one
// more, so with z = fl(T + P) - I,
//   |z - R| <= (u + 2.01 g_D)(|x|^2 + |y|^2) + 3(D+1) t,
// and, rounding being monotone, z <= eps2 gives E <= eps2 while
// z > eps2 (1 + 2u) + 2t gives E > eps2.  The thresholds then bracket
// those two conditions instead of L and H:
//   lo = RD(eps2 - |x|^2 - m'),  hi = RU(eps2 (1 + 2u) + 2t - |x|^2 + m'),
//   m' = m + (u + 2.01 g_D)(|x|^2 + Y) + 3(D+1) t.
//
// When the count pass forms v on the matrix cores (v_mfma_f32_16x16x4_f32,
// widths >= 16), the order of the additions inside an instruction, whether
// the products are rounded on their own, the rounding mode and the
// handling of subnormals are not specified.  The products are accumulated
// there from zero, and n_y is added last by one fp32 addition rounded to
// nearest.  The products' sum is bounded for any order of its D - 1
// additions, with every product and every sum rounded off by up to 2u
// (any of the usual rounding modes), so each product passes at most D
// roundings:
//   |acc - sum_k P_k| <= g'_D sum |P_k| <= g'_D (|x|^2 + |y|^2),
//   g'_m = 2 m u / (1 - 2 m u),  P_k = (-2 x_k) y_k;
// n_y is off |y|^2 by at most u |y|^2, and the last addition by at most
// u |n_y + acc| <= u (1 + g'_D)(|x|^2 + 2 |y|^2).  Together
//   k = g'_D + 3u (1 + g'_D)   (taken as 1.01 g'_D + 3.01 u (1 + g'_D)),
// plus, for subnormals flushed anywhere in the matrix unit, an absolute
//   (2D + 2) 2^-126 (1 + 2 sqrt(Y)):
// each product or partial sum loses at most 2^-126, and a flushed input
// changes a product by at most 2^-126 times the other factor, itself at
// most 2 sqrt(Y).
#include <cmath>

#include "device.h"
#include "internal.h"

namespace dbk {

static unsigned grid_for_s(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (unsigned)(g < kMaxGrid ? g : kMaxGrid);
}

__device__ __forceinline__ double sq_norm64(const float* __restrict__ p, int S) {
  double s = 0.0;
  for (int k = 0; k < S; ++k) {
    const double x = (double)p[k];
    s += x * x;   // fp64 product of an fp32 value: exact
  }
  return s;
}

// The squared norm as the hoisted-norm form takes it: rounded squares
// summed in k order in fp32 (padding dims are zero and add nothing).
__device__ __forceinline__ float sq_norm32(const float* __restrict__ p, int S) {
  float s = p[0] * p[0];
  for (int k = 1; k < S; ++k) {
    const float q = p[k] * p[k];
    s = s + q;
  }
  return s;
}

// Pass 1: fp32 norms of every point and the largest fp64 squared norm
// (and, for the hoisted-norm form, its own fp32 norm of every point).  The
// maximum is reduced per wave, then per workgroup in LDS: one atomic per
// workgroup (one per wave on the same word serialised the pass).
__global__ __launch_bounds__(256) void k_screen_norms(
    const float* __restrict__ pts, int64_t n_pad, int S,
    float* __restrict__ ncol, float* __restrict__ nexp,
    Status* __restrict__ st) {
  __shared__ double sh[4];
  double ymax = 0.0;
  // four points per thread and step, their loads issued together
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
       i0 < n_pad; i0 += 4 * stride) {
    double s[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      s[u] = i < n_pad ? sq_norm64(pts + i * S, S) : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      if (i >= n_pad) break;
      if (s[u] == s[u]) {              // real point (padding rows are NaN)
        ncol[i] = (float)s[u];         // round to nearest
        ymax = s[u] > ymax ? s[u] : ymax;
      } else {
        ncol[i] = __builtin_nanf("");
      }
      if (nexp) nexp[i] = sq_norm32(pts + i * S, S);
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const double o = __shfl_xor(ymax, off);
    ymax = o > ymax ? o : ymax;
  }
  if (lane_id() == 0) sh[threadIdx.x >> 6] = ymax;
  __syncthreads();
  if (threadIdx.x == 0) {
    ymax = sh[0];
    for (int w = 1; w < 4; ++w) ymax = sh[w] > ymax ? sh[w] : ymax;
    if (ymax > 0.0) {
      // non-negative doubles order like their bit patterns
      atomicMax(&st->ymax_bits, (unsigned long long)__double_as_longlong(ymax));
      if (!(ymax <= 0x1p100)) atomicOr(&st->screen_unsafe, 1u);
    }
  }
}

// Pass 2: the row table: -2 x_k, then lo and hi.
template <int D>
__global__ __launch_bounds__(256) void k_screen_rows(
    const float* __restrict__ pts, int64_t n_pad, float eps2,
    float* __restrict__ srow, float* __restrict__ ncol,
    const Status* __restrict__ st, int matrix, int expanded) {
  constexpr int S = row_stride(D);
  constexpr int SR = screen_stride(D);
  const double u = 0x1p-24, t = 0x1p-149;
  const double gD = D * u / (1.0 - D * u);
  const double g2 = (D + 2) * u / (1.0 - (D + 2) * u);
  const double gM = 2.0 * D * u / (1.0 - 2.0 * D * u);
  const double kap = matrix ? 1.01 * gM + 3.01 * u * (1.0 + gM) : u + 2.01 * gD;
  // the hoisted-norm form's own error against R (see above)
  const double kapE = expanded ? u + 2.01 * gD : 0.0;
  const double e2 = (double)eps2;
  const double L = (e2 - (D + 2) * t) / (1.0 + g2);
  const double H = (e2 + (D + 2) * t) / (1.0 - g2);
  const double Y = __longlong_as_double((long long)st->ymax_bits);
  const bool unsafe = st->screen_unsafe != 0;
  const double flush = matrix ? (2.0 * D + 2.0) * 0x1p-126 * (1.0 + 2.0 * sqrt(Y)) : 0.0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n_pad;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float* p = pts + i * S;
    float* out = srow + i * SR;
    const double x2 = sq_norm64(p, S);
    if (!(x2 == x2)) {               // padding row
      for (int k = 0; k < SR; ++k) out[k] = __builtin_nanf("");
      continue;
    }
    if (unsafe) {
      for (int k = 0; k < D; ++k) out[k] = 0.f;
      out[D] = -__builtin_inff();
      out[D + 1] = __builtin_inff();
      ncol[i] = 0.f;
    } else {
      for (int k = 0; k < D; ++k) out[k] = -2.f * p[k];   // exact
      if (!(e2 < 0x1p128)) {         // eps2 = +inf: every pair is a neighbour
        out[D] = __builtin_inff();
        out[D + 1] = __builtin_inff();
      } else {
        if (expanded) {
          const double hiE = e2 * (1.0 + 2.0 * u) + 2.0 * t;
          const double m = (kap + kapE) * (x2 + Y) + 4.0 * (D + 1) * t +
                           flush + 1e-12 * (e2 + x2 + Y);
          out[D] = __double2float_rd(e2 - x2 - m);
          out[D + 1] = __double2float_ru(hiE - x2 + m);
        } else {
          const double m = kap * (x2 + Y) + (D + 1) * t + flush +
                           1e-12 * (fabs(L) + fabs(H) + x2 + Y);
          out[D] = __double2float_rd(L - x2 - m);
          out[D + 1] = __double2float_ru(H - x2 + m);
        }
      }
    }
    for (int k = D + 2; k < SR; ++k) out[k] = 0.f;
  }
}

hipError_t launch_screen(const Layout& L, const float* pts, float eps2,
                         hipStream_t s) {
  // at most 512 work-groups: one atomic each
  const unsigned ngrid = grid_for_s(L.n_pad, 256 * 4);
  k_screen_norms<<<ngrid < 512 ? ngrid : 512, 256, 0, s>>>(
      pts, L.n_pad, L.stride, L.ncol, L.expanded ? L.nexp : nullptr,
      L.status);
  const unsigned grid = grid_for_s(L.n_pad, 256 * 4);
  switch (L.D) {
#define DBK_CASE(DD)                                                       \
  case DD:                                                                 \
    k_screen_rows<DD><<<grid, 256, 0, s>>>(pts, L.n_pad, eps2, L.srow,     \
                                           L.ncol, L.status,               \
                                           screen_on_matrix_cores(DD),     \
                                           L.expanded ? 1 : 0);            \
    break;
    DBK_CASE(1) DBK_CASE(2) DBK_CASE(3) DBK_CASE(4) DBK_CASE(6) DBK_CASE(8)
    DBK_CASE(12) DBK_CASE(16) DBK_CASE(24) DBK_CASE(32) DBK_CASE(48)
    DBK_CASE(64)
#undef DBK_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dbk

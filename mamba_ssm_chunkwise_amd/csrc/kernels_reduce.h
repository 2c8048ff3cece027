// Non-template kernels of the host dispatcher: the fixed-order reductions of
// the forward's partial moments and the reordering of d_m1. They live apart
// from the kernel headers because those are compiled into more than one
// translation unit, and a non-template kernel may be defined in only one.
#pragma once

#include "kernels_fwd4.h"

namespace mom {

// k_reduce: m2 = sum over the per-workgroup partials, m1 likewise; both
// written in the caller's column order.
__global__ __launch_bounds__(NTH) void k_reduce(Geo g, int R, const float* __restrict__ m2part,
                                                const float* __restrict__ m1part, float* m2,
                                                float* m1) {
  const int bh = blockIdx.x;
  const int e = blockIdx.y * NTH + threadIdx.x;
  const int n2 = g.r * g.r, n1 = g.p * g.r;
  if (e < n2) {
    const int a = inv_perm_rc(g, e / g.r), b = inv_perm_rc(g, e % g.r);
    float s = 0.0f;
    for (int gi = 0; gi < g.NGR; gi++) s += m2part[((size_t)bh * g.NGR + gi) * R * R + a * R + b];
    m2[(size_t)bh * n2 + e] = s;
  } else if (e < n2 + n1) {
    const int f = e - n2;
    const int p0 = f / g.r, rc = inv_perm_rc(g, f % g.r);
    float s = 0.0f;
    for (int gi = 0; gi < g.NGR; gi++) s += m1part[((size_t)bh * g.NGR + gi) * g.p * R + p0 * R + rc];
    m1[(size_t)bh * n1 + f] = s;
  }
}

// d_m1 in the internal column order, rows padded to R: dm1i[bh][p][R].
__global__ __launch_bounds__(NTH) void k_prep_dm1(Geo g, int R, const float* __restrict__ dm1, float* dm1i) {
  const size_t e = (size_t)blockIdx.x * NTH + threadIdx.x;
  const size_t total = (size_t)g.b * g.h * g.p * R;
  if (e >= total) return;
  const int col = (int)(e % R);
  const size_t row = e / R;
  dm1i[e] = col < g.r ? dm1[row * g.r + perm_rc(g, col)] : 0.0f;
}

// Fixed-order sum of the per-wave, per-group partials of k_fwd4, written in
// the caller's column order.
__global__ __launch_bounds__(NTH) void k_reduce4(Geo g, int R, int ord, const float* __restrict__ m2part,
                                                 const float* __restrict__ m1part, float* m2, float* m1) {
  const int bh = blockIdx.x;
  const int e = blockIdx.y * NTH + threadIdx.x;
  const int nR2 = R * R;
  if (e < nR2) {
    const int ia = e / R, ib = e % R;
    const int a = lp_col(g, ord, ia), b = lp_col(g, ord, ib);
    if (a < 0 || b < 0) return;
    float s = 0.0f;
    const int np = g.NGR * NW4;
    for (int k = 0; k < np; k++) s += m2part[((size_t)bh * np + k) * nR2 + e];
    m2[((size_t)bh * g.r + a) * g.r + b] = s;
  } else if (e < nR2 + g.p * R) {
    const int e1 = e - nR2;
    const int pp = e1 / R, ic = e1 % R;
    const int cc = lp_col(g, ord, ic);
    if (cc < 0) return;
    float s = 0.0f;
    for (int gi = 0; gi < g.NGR; gi++) s += m1part[(((size_t)bh * g.NGR + gi) * g.p + pp) * R + ic];
    m1[((size_t)bh * g.p + pp) * g.r + cc] = s;
  }
}

}  // namespace mom

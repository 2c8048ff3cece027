// Rotation-sequence producer and its VJP: per-token increments -> the cumulative
// rotation the moments kernels take ("recalculated.rs" source page: RotPrim
// holds cumulative angles [b,s,h,a] or cumulative unit quaternions [b,s,h,J,4];
// quat_mul_prim is the Hamilton product on the packed (w,x,y,z) axis).
//
//   angles      theta[t] = sum_{t'<=t} inc[t']
//   quaternions Q[t] = N(Q[t-1] (x) q[t]), Q[-1] = 1, N(v) = v/|v|
//               (= the normalised product q[0] (x) ... (x) q[t]: the product is
//               bilinear, so normalising early only rescales)
//
// A chain is one (b, h, angle) or (b, h, block); chains are the innermost index
// of every token row, so the threads of a wave read consecutive chains of one
// token (coalesced, up to 16 bytes per thread) and walk the tokens of one
// segment. Three passes, each a plain streaming kernel (the work is HBM-bound:
// a few flops per loaded element):
//   k_rot_seg    per (segment, chain): the segment's own total (sum, or the
//                renormalised running product);
//   k_rot_carry  per chain: scan of the segment totals -> the value entering
//                each segment;
//   k_rot_apply  per (segment, chain): the walk again from the entering value,
//                writing every token.
//
// VJP. Angles: d_inc[t] = sum_{t'>=t} d_theta[t'] (same three passes, suffix
// order). Quaternions, with P[t] the unnormalised product (|P[t]| = prod |q|):
// the cotangent reaching P[t] through everything at t' >= t is
//   G[t] = (sum_{k>=t} F[k]) (x) Q[t] / |P[t]|,   F[k] = Im(d_Q[k] (x) conj(Q[k]))
// (F[k] is d_Q[k] pushed through N and moved to the identity frame; the sum
// telescopes because P[k] = P[t] (x) q[t+1] (x) ... (x) q[k]), and
//   d_q[t] = conj(P[t-1]) (x) G[t] = conj(Q[t-1]) (x) S[t] (x) Q[t] / |q[t]|,
//   S[t]   = sum_{k>=t} F[k]   (pure quaternions: a plain suffix sum).
// Inside a segment entering with C = Q[t0-1], Q[t] = C (x) R[t] with R the
// segment's running product, so sum_k d_Q[k] (x) conj(R[k]) (one pass, no C)
// gives the segment's F-sum as Im(U (x) conj(C)) once the carries are known.
#pragma once

#include "common.h"

namespace mom {

constexpr int ROT_TPB = 256;  // threads per workgroup of the producer kernels

struct RotGeo {
  int b, s, C;     // batch, tokens, chains per token row
  int seg, nseg;   // tokens per segment, segments per chain
};

__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ f4 ld4(const bf16* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return f4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
}
__device__ __forceinline__ void st4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }
__device__ __forceinline__ void st4(bf16* p, f4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]));
}

// Hamilton product a (x) b, (w, x, y, z).
__device__ __forceinline__ f4 qmul(f4 a, f4 b) {
  return f4{a[0] * b[0] - a[1] * b[1] - a[2] * b[2] - a[3] * b[3],
            a[0] * b[1] + a[1] * b[0] + a[2] * b[3] - a[3] * b[2],
            a[0] * b[2] - a[1] * b[3] + a[2] * b[0] + a[3] * b[1],
            a[0] * b[3] + a[1] * b[2] - a[2] * b[1] + a[3] * b[0]};
}
__device__ __forceinline__ f4 qconj(f4 a) { return f4{a[0], -a[1], -a[2], -a[3]}; }
__device__ __forceinline__ float qdot(f4 a, f4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }
__device__ __forceinline__ f4 qnorm(f4 a) { return a * rsqrtf(qdot(a, a)); }
__device__ __forceinline__ f4 qim(f4 a) { return f4{0.0f, a[1], a[2], a[3]}; }

// N consecutive values of T at p (N * sizeof(T) <= 16 bytes, aligned to that
// size) as floats: one vector load.
template <int N>
__device__ __forceinline__ void ldv(const float* p, float (&o)[N]) {
  if constexpr (N == 4) {
    const f4 v = *reinterpret_cast<const f4*>(p);
    for (int i = 0; i < 4; i++) o[i] = v[i];
  } else if constexpr (N == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    o[0] = v.x;
    o[1] = v.y;
  } else {
    for (int i = 0; i < N; i++) o[i] = p[i];
  }
}
template <int N>
__device__ __forceinline__ void ldv(const bf16* p, float (&o)[N]) {
  if constexpr (N == 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
    for (int i = 0; i < 4; i++) {
      o[2 * i] = bf16_lo(w[i]);
      o[2 * i + 1] = bf16_hi(w[i]);
    }
  } else if constexpr (N == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    o[0] = bf16_lo(v.x);
    o[1] = bf16_hi(v.x);
    o[2] = bf16_lo(v.y);
    o[3] = bf16_hi(v.y);
  } else if constexpr (N == 2) {
    const unsigned v = *reinterpret_cast<const unsigned*>(p);
    o[0] = bf16_lo(v);
    o[1] = bf16_hi(v);
  } else {
    for (int i = 0; i < N; i++) o[i] = (float)p[i];
  }
}
template <int N>
__device__ __forceinline__ void stv(float* p, const float (&o)[N]) {
  if constexpr (N == 4) {
    *reinterpret_cast<f4*>(p) = f4{o[0], o[1], o[2], o[3]};
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(o[0], o[1]);
  } else {
    for (int i = 0; i < N; i++) p[i] = o[i];
  }
}
template <int N>
__device__ __forceinline__ void stv(bf16* p, const float (&o)[N]) {
  if constexpr (N == 8) {
    *reinterpret_cast<uint4*>(p) =
        make_uint4(pk_bf16(o[0], o[1]), pk_bf16(o[2], o[3]), pk_bf16(o[4], o[5]), pk_bf16(o[6], o[7]));
  } else if constexpr (N == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pk_bf16(o[0], o[1]), pk_bf16(o[2], o[3]));
  } else if constexpr (N == 2) {
    *reinterpret_cast<unsigned*>(p) = pk_bf16(o[0], o[1]);
  } else {
    for (int i = 0; i < N; i++) p[i] = (bf16)o[i];
  }
}

// A thread owns V consecutive chains c0 .. c0+V-1 (V * width * sizeof(T) <= 16
// bytes, width = 4 for quaternions), so each token is one vector load per thread
// and a wave reads one contiguous piece of the token row.
template <bool QUAT>
__device__ __forceinline__ size_t rot_off(const RotGeo& g, int bi, int t, int c) {
  const size_t e = ((size_t)bi * g.s + t) * g.C + c;
  return QUAT ? 4 * e : e;
}
// Index of (bi, segment k, chain c) in the per-segment workspace arrays.
__device__ __forceinline__ size_t seg_idx(const RotGeo& g, int bi, int k, int c) {
  return ((size_t)bi * g.nseg + k) * g.C + c;
}

// Pass 1. Forward: tot = segment total of the increments (sum, or running
// product). Backward: angles, tot = segment sum of d_theta; quaternions,
// tot = running product R and aux = sum_t d_Q[t] (x) conj(R[t]).
template <typename T, bool QUAT, bool BWD, int V>
__global__ __launch_bounds__(ROT_TPB) void k_rot_seg(RotGeo g, const T* __restrict__ inc,
                                                      const T* __restrict__ dout, float* __restrict__ tot,
                                                      float* __restrict__ aux) {
  const int c0 = (blockIdx.x * ROT_TPB + threadIdx.x) * V, k = blockIdx.y, bi = blockIdx.z;
  if (c0 >= g.C) return;
  const int t0 = k * g.seg, t1 = min(t0 + g.seg, g.s);
  const size_t i0 = seg_idx(g, bi, k, c0);
  if constexpr (QUAT) {
    f4 R[V], U[V];
    for (int v = 0; v < V; v++) {
      R[v] = f4{1.0f, 0.0f, 0.0f, 0.0f};
      U[v] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll 4
    for (int t = t0; t < t1; t++) {
      const size_t o = rot_off<true>(g, bi, t, c0);
      float q[4 * V], d[4 * V];
      ldv(inc + o, q);
      if constexpr (BWD) ldv(dout + o, d);
      for (int v = 0; v < V; v++) {
        R[v] = qnorm(qmul(R[v], f4{q[4 * v], q[4 * v + 1], q[4 * v + 2], q[4 * v + 3]}));
        if constexpr (BWD) U[v] += qmul(f4{d[4 * v], d[4 * v + 1], d[4 * v + 2], d[4 * v + 3]}, qconj(R[v]));
      }
    }
    for (int v = 0; v < V; v++) {
      st4(tot + 4 * (i0 + v), R[v]);
      if constexpr (BWD) st4(aux + 4 * (i0 + v), U[v]);
    }
  } else {
    const T* src = BWD ? dout : inc;
    float acc[V];
    for (int v = 0; v < V; v++) acc[v] = 0.0f;
#pragma unroll 4
    for (int t = t0; t < t1; t++) {
      float x[V];
      ldv(src + rot_off<false>(g, bi, t, c0), x);
      for (int v = 0; v < V; v++) acc[v] += x[v];
    }
    for (int v = 0; v < V; v++) tot[i0 + v] = acc[v];
  }
}

// Pass 2, one thread per (b, chain). Forward: tot[k] <- the value entering
// segment k. Backward, angles: tot[k] <- sum of d_theta over later segments;
// quaternions: tot[k] <- Q entering segment k, aux[k] <- S at the segment's
// first token (the F-sums of segments k and later). Segments are taken in
// batches of CB whose loads are all issued before the dependent updates.
constexpr int CB = 16;
template <bool QUAT, bool BWD>
__global__ __launch_bounds__(ROT_TPB) void k_rot_carry(RotGeo g, float* __restrict__ tot,
                                                        float* __restrict__ aux) {
  const int i = blockIdx.x * ROT_TPB + threadIdx.x;
  if (i >= g.b * g.C) return;
  const int bi = i / g.C, c = i % g.C;
  if constexpr (QUAT) {
    f4 Cq = {1.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < g.nseg; k0 += CB) {
      f4 R[CB], U[CB];
      for (int j = 0; j < CB; j++) {
        if (k0 + j < g.nseg) {
          R[j] = ld4(tot + 4 * seg_idx(g, bi, k0 + j, c));
          if constexpr (BWD) U[j] = ld4(aux + 4 * seg_idx(g, bi, k0 + j, c));
        }
      }
      for (int j = 0; j < CB; j++) {
        if (k0 + j < g.nseg) {
          st4(tot + 4 * seg_idx(g, bi, k0 + j, c), Cq);
          if constexpr (BWD) st4(aux + 4 * seg_idx(g, bi, k0 + j, c), qim(qmul(U[j], qconj(Cq))));
          Cq = qnorm(qmul(Cq, R[j]));
        }
      }
    }
    if constexpr (BWD) {
      f4 S = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int k1 = g.nseg; k1 > 0; k1 -= CB) {
        f4 F[CB];
        for (int j = 0; j < CB; j++)
          if (k1 - 1 - j >= 0) F[j] = ld4(aux + 4 * seg_idx(g, bi, k1 - 1 - j, c));
        for (int j = 0; j < CB; j++) {
          if (k1 - 1 - j >= 0) {
            S += F[j];
            st4(aux + 4 * seg_idx(g, bi, k1 - 1 - j, c), S);
          }
        }
      }
    }
  } else {
    float run = 0.0f;
    for (int kk0 = 0; kk0 < g.nseg; kk0 += CB) {
      float x[CB];
      for (int j = 0; j < CB; j++) {
        const int kk = kk0 + j, k = BWD ? g.nseg - 1 - kk : kk;
        if (kk < g.nseg) x[j] = tot[seg_idx(g, bi, k, c)];
      }
      for (int j = 0; j < CB; j++) {
        const int kk = kk0 + j, k = BWD ? g.nseg - 1 - kk : kk;
        if (kk < g.nseg) {
          tot[seg_idx(g, bi, k, c)] = run;
          run += x[j];
        }
      }
    }
  }
}

// Pass 3: the segment's walk from its entering value, writing every token.
template <typename T, bool QUAT, bool BWD, int V>
__global__ __launch_bounds__(ROT_TPB) void k_rot_apply(RotGeo g, const T* __restrict__ inc,
                                                        const T* __restrict__ dout, const float* __restrict__ tot,
                                                        const float* __restrict__ aux, T* __restrict__ out) {
  const int c0 = (blockIdx.x * ROT_TPB + threadIdx.x) * V, k = blockIdx.y, bi = blockIdx.z;
  if (c0 >= g.C) return;
  const int t0 = k * g.seg, t1 = min(t0 + g.seg, g.s);
  const size_t i0 = seg_idx(g, bi, k, c0);
  if constexpr (QUAT) {
    f4 R[V], S[V];
    for (int v = 0; v < V; v++) {
      R[v] = ld4(tot + 4 * (i0 + v));
      if constexpr (BWD) S[v] = ld4(aux + 4 * (i0 + v));
    }
#pragma unroll 4
    for (int t = t0; t < t1; t++) {
      const size_t o = rot_off<true>(g, bi, t, c0);
      float q[4 * V], d[4 * V], y[4 * V];
      ldv(inc + o, q);
      if constexpr (BWD) ldv(dout + o, d);
      for (int v = 0; v < V; v++) {
        const f4 qv = {q[4 * v], q[4 * v + 1], q[4 * v + 2], q[4 * v + 3]};
        const f4 Rp = R[v];
        R[v] = qnorm(qmul(R[v], qv));
        f4 r = R[v];
        if constexpr (BWD) {
          r = qmul(qmul(qconj(Rp), S[v]), R[v]) * rsqrtf(qdot(qv, qv));
          S[v] -= qim(qmul(f4{d[4 * v], d[4 * v + 1], d[4 * v + 2], d[4 * v + 3]}, qconj(R[v])));
        }
        for (int e = 0; e < 4; e++) y[4 * v + e] = r[e];
      }
      stv(out + o, y);
    }
  } else {
    float run[V];
    for (int v = 0; v < V; v++) run[v] = tot[i0 + v];
    if constexpr (!BWD) {
#pragma unroll 4
      for (int t = t0; t < t1; t++) {
        const size_t o = rot_off<false>(g, bi, t, c0);
        float x[V];
        ldv(inc + o, x);
        for (int v = 0; v < V; v++) x[v] = run[v] += x[v];
        stv(out + o, x);
      }
    } else {
#pragma unroll 4
      for (int t = t1 - 1; t >= t0; t--) {
        const size_t o = rot_off<false>(g, bi, t, c0);
        float x[V];
        ldv(dout + o, x);
        for (int v = 0; v < V; v++) x[v] = run[v] += x[v];
        stv(out + o, x);
      }
    }
  }
}

}  // namespace mom

// Per-chunk staging into LDS and the de-rotation on accumulator tiles.
//
// chunk_decay (recalculated.rs source page): a = inclusive cumsum of da over the
// chunk, d_t = exp(a_t), L[t,j] = exp(a_t - a_j) on and below the diagonal.
// rotate_chunk (same page): de-rotation R(-theta) on complex pairs, left
// Hamilton product by Q on 4-blocks; the transpose R(+theta) / conj(Q) for
// cotangents. Positions >= V are staged as zero inputs (identity rotation), so
// nothing past valid_len can reach a valid output even if it holds NaN.
#pragma once

#include "common.h"

namespace mom {

// a_t, d_t (ELL each) and L (ELL x (ELL+1), fp32). Needs all NTH threads.
template <typename T>
__device__ __forceinline__ void stage_decay(const Geo& g, const T* __restrict__ da, int bi, int hi, int n,
                                   float* s_a, float* s_d, float* s_L) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int t = tid & 31;
    const int pos = n * ELL + t;
    float v = 0.0f;
    if (tid < 32 && pos < g.V) v = to_f(da[((size_t)bi * g.s + pos) * g.h + hi]);
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const float u = __shfl_up(v, off, 32);
      if (t >= off) v += u;
    }
    if (tid < 32) {
      s_a[t] = v;
      s_d[t] = expf(v);
    }
  }
  __syncthreads();
  for (int idx = tid; idx < ELL * ELL; idx += NTH) {
    const int t = idx / ELL, j = idx % ELL;
    s_L[t * (ELL + 1) + j] = (j <= t) ? expf(s_a[t] - s_a[j]) : 0.0f;
  }
}

// bhat chunk as bs[rc][k] (T), k = j*c + ci, rows rc < R (internal column order),
// zero outside r and past V.
template <typename T, int R>
__device__ __forceinline__ void stage_bhat(const Geo& g, const T* __restrict__ bhat, int bi, int hi, int n,
                                  T* bs) {
  const int K = g.K;
  for (int idx = threadIdx.x; idx < K * R; idx += NTH) {
    const int k = idx / R, rc = idx % R;
    const int j = k / g.c, ci = k - j * g.c;
    const int pos = n * ELL + j;
    float v = 0.0f;
    if (rc < g.r && pos < g.V)
      v = to_f(bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + perm_rc(g, rc)]);
    bs[rc * g.KP + k] = to_t<T>(v);
  }
}

// Lx[t][k] = L[t][k / c] (fp32), the weight of write k in state row t.
__device__ __forceinline__ void stage_lx(const Geo& g, const float* s_L, float* lx) {
  for (int idx = threadIdx.x; idx < ELL * g.K; idx += NTH) {
    const int t = idx / g.K, k = idx % g.K;
    lx[t * g.KP + k] = s_L[t * (ELL + 1) + k / g.c];
  }
}

// Slot-ordered transposes of L used as A operands with K over the chunk's
// tokens: ltp[j][slot] = L[tslot(slot)][j]; ltx[k][slot] = L[tslot(slot)][k/c].
constexpr int SLOTP = 40;  // row length of slot tables (32 slots + 16 bytes pad for bf16)
template <typename T>
__device__ __forceinline__ void stage_lt(const Geo& g, const float* s_L, T* ltp, T* ltx) {
  for (int idx = threadIdx.x; idx < ELL * 32; idx += NTH) {
    const int j = idx / 32, sl = idx % 32;
    ltp[j * SLOTP + sl] = to_t<T>(s_L[tslot<T>(sl) * (ELL + 1) + j]);
  }
  for (int idx = threadIdx.x; idx < g.K * 32; idx += NTH) {
    const int k = idx / 32, sl = idx % 32;
    ltx[k * SLOTP + sl] = to_t<T>(s_L[tslot<T>(sl) * (ELL + 1) + k / g.c]);
  }
}

// Rotation parameters of the chunk: complex -> cos/sin [ELL][A];
// quaternion -> qv [ELL][J][4]. Identity past V.
template <typename T>
__device__ __forceinline__ void stage_rot(const Geo& g, const T* __restrict__ rot, int bi, int hi, int n,
                                 float* cs, float* sn, float* qv) {
  if (g.rot_kind == 1 || g.rot_kind == 2) {
    for (int idx = threadIdx.x; idx < ELL * g.A; idx += NTH) {
      const int t = idx / g.A, a = idx % g.A;
      const int pos = n * ELL + t;
      float th = 0.0f;
      if (pos < g.V) th = to_f(rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + a]);
      float sv, cv;
      sincosf(th, &sv, &cv);
      cs[idx] = cv;
      sn[idx] = sv;
    }
  } else if (g.rot_kind == 3) {
    for (int idx = threadIdx.x; idx < ELL * g.J * 4; idx += NTH) {
      const int t = idx / (g.J * 4), e = idx % (g.J * 4);
      const int pos = n * ELL + t;
      float v = (e & 3) == 0 ? 1.0f : 0.0f;
      if (pos < g.V) v = to_f(rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + e]);
      qv[idx] = v;
    }
  }
}

// De-rotation (TR = false: c = M h) or its transpose (TR = true: M^T v) applied
// in place to an accumulator tile pair v[mt][nt] holding rows t = 16mt+4q+i and
// internal state columns 16nt + (lane % 16).
template <bool TR, int NT>
__device__ __forceinline__ void rotate_tiles(f4 (&v)[2][NT], const Geo& g, const float* cs, const float* sn,
                                    const float* qv) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  if (g.rot_kind == 1 || g.rot_kind == 2) {
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
      const int col = 16 * nt + n;
      const int al = col >> 1;
      const bool act = al < g.A;
      const int alc = act ? al : 0;
      const float sg = (col & 1) ? -1.0f : 1.0f;
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float x = v[mt][nt][i];
          const float px = dpp<QP_SWAP1>(x);
          const int t = 16 * mt + 4 * q + i;
          const float c = cs[t * g.A + alc], s = sg * sn[t * g.A + alc];
          const float y = TR ? (c * x - s * px) : (c * x + s * px);
          v[mt][nt][i] = act ? y : x;
        }
    }
  } else if (g.rot_kind == 3) {
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
      const int col = 16 * nt + n;
      const int jq = col >> 2, k = col & 3;
      const bool act = jq < g.J;
      const int jqc = act ? jq : 0;
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float x = v[mt][nt][i];
          const float v0 = dpp<QP_B0>(x), v1 = dpp<QP_B1>(x), v2 = dpp<QP_B2>(x), v3 = dpp<QP_B3>(x);
          const int t = 16 * mt + 4 * q + i;
          const float* Q = qv + (t * g.J + jqc) * 4;
          const float w = Q[0], qx = Q[1], qy = Q[2], qz = Q[3];
          float m0, m1, m2, m3;
          if (!TR) {  // row k of the left Hamilton matrix of Q
            m0 = k == 0 ? w : k == 1 ? qx : k == 2 ? qy : qz;
            m1 = k == 0 ? -qx : k == 1 ? w : k == 2 ? qz : -qy;
            m2 = k == 0 ? -qy : k == 1 ? -qz : k == 2 ? w : qx;
            m3 = k == 0 ? -qz : k == 1 ? qy : k == 2 ? -qx : w;
          } else {    // column k of it
            m0 = k == 0 ? w : k == 1 ? -qx : k == 2 ? -qy : -qz;
            m1 = k == 0 ? qx : k == 1 ? w : k == 2 ? -qz : qy;
            m2 = k == 0 ? qy : k == 1 ? qz : k == 2 ? w : -qx;
            m3 = k == 0 ? qz : k == 1 ? -qy : k == 2 ? qx : w;
          }
          const float y = m0 * v0 + m1 * v1 + m2 * v2 + m3 * v3;
          v[mt][nt][i] = act ? y : x;
        }
    }
  }
}

// Gradient of the rotation parameters for one state row, accumulated into
// racc (same layout as the tiles). dc = cotangent of c (before the transpose);
// keep = c (complex modes) or the cache-frame state h (quaternion).
//   complex : d_theta = dc_x c_y - dc_y c_x        (held by the even column)
//   quaternion: d_Q = dc (x) conj(h), component k held by column 4j+k
template <int NT>
__device__ __forceinline__ void accum_drot(f4 (&racc)[2][NT], const f4 (&dc)[2][NT], const f4 (&keep)[2][NT],
                                  const Geo& g) {
  const int n = threadIdx.x & 15;
  if (g.rot_kind == 1 || g.rot_kind == 2) {
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float a = dc[mt][nt][i], pa = dpp<QP_SWAP1>(a);
          const float c = keep[mt][nt][i], pc = dpp<QP_SWAP1>(c);
          racc[mt][nt][i] += a * pc - pa * c;
        }
  } else if (g.rot_kind == 3) {
    const int k = n & 3;
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float a = dc[mt][nt][i], h = keep[mt][nt][i];
          const float a0 = dpp<QP_B0>(a), a1 = dpp<QP_B1>(a), a2 = dpp<QP_B2>(a), a3 = dpp<QP_B3>(a);
          const float h0 = dpp<QP_B0>(h), h1 = dpp<QP_B1>(h), h2 = dpp<QP_B2>(h), h3 = dpp<QP_B3>(h);
          float y;
          if (k == 0) y = a0 * h0 + a1 * h1 + a2 * h2 + a3 * h3;
          else if (k == 1) y = -a0 * h1 + a1 * h0 - a2 * h3 + a3 * h2;
          else if (k == 2) y = -a0 * h2 + a1 * h3 + a2 * h0 - a3 * h1;
          else y = -a0 * h3 - a1 * h2 + a2 * h1 + a3 * h0;
          racc[mt][nt][i] += y;
        }
  }
}

}  // namespace mom

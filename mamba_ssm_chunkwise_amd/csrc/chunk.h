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
  for (int idx = tid; idx < ELL * ELL; idx += blockDim.x) {
    const int t = idx / ELL, j = idx % ELL;
    s_L[t * (ELL + 1) + j] = (j <= t) ? expf(s_a[t] - s_a[j]) : 0.0f;
  }
}

// The folded write index of a chunk is k = j*CK + ci with CK >= c channel
// slots (slots ci >= c hold zeros): K = ELL*CK, a compile-time width.
template <typename T> constexpr int pad_of() { return 16 / (int)sizeof(T); }

// bhat chunk as bs[rc][k] (T), rows rc < R (internal column order), zero outside
// r, past V and in unused channel slots.
template <typename T, int R, int CK>
__device__ __forceinline__ void stage_bhat(const Geo& g, const T* __restrict__ bhat, int bi, int hi, int n,
                                  T* bs) {
  constexpr int K = ELL * CK, KP = K + pad_of<T>();
  for (int idx = threadIdx.x; idx < K * R; idx += blockDim.x) {
    const int k = idx / R, rc = idx % R;
    const int j = k / CK, ci = k % CK;
    const int pos = n * ELL + j;
    float v = 0.0f;
    if (rc < g.r && pos < g.V && ci < g.c)
      v = to_f(bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + perm_rc(g, rc)]);
    bs[rc * KP + k] = to_t<T>(v);
  }
}

// Slot-ordered transposes of L used as A operands with K over the chunk's
// tokens: ltp[j][slot] = L[tslot(slot)][j]; ltx[k][slot] = L[tslot(slot)][k/c].
constexpr int SLOTP = 40;  // row length of slot tables (32 slots + 16 bytes pad for bf16)
template <typename T, int CK>
__device__ __forceinline__ void stage_lt(const float* s_L, T* ltp, T* ltx) {
  constexpr int K = ELL * CK;
  for (int idx = threadIdx.x; idx < ELL * 32; idx += blockDim.x) {
    const int j = idx / 32, sl = idx % 32;
    ltp[j * SLOTP + sl] = to_t<T>(s_L[tslot<T>(sl) * (ELL + 1) + j]);
  }
  for (int idx = threadIdx.x; idx < K * 32; idx += blockDim.x) {
    const int k = idx / 32, sl = idx % 32;
    ltx[k * SLOTP + sl] = to_t<T>(s_L[tslot<T>(sl) * (ELL + 1) + k / CK]);
  }
}

// Rotation parameters of the chunk: complex -> cos/sin [A][ELL] (token fastest,
// so a lane's four consecutive rows read as one vector); quaternion ->
// qv [J][ELL][4]. Identity past V.
template <typename T>
__device__ __forceinline__ void stage_rot(const Geo& g, const T* __restrict__ rot, int bi, int hi, int n,
                                 float* cs, float* sn, float* qv) {
  if (g.rot_kind == 1 || g.rot_kind == 2) {
    for (int idx = threadIdx.x; idx < ELL * g.A; idx += blockDim.x) {
      const int t = idx / g.A, a = idx % g.A;
      const int pos = n * ELL + t;
      float th = 0.0f;
      if (pos < g.V) th = to_f(rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + a]);
      float sv, cv;
      sincosf(th, &sv, &cv);
      cs[a * ELL + t] = cv;
      sn[a * ELL + t] = sv;
    }
  } else if (g.rot_kind == 3) {
    for (int idx = threadIdx.x; idx < ELL * g.J * 4; idx += blockDim.x) {
      const int t = idx / (g.J * 4), e = idx % (g.J * 4);
      const int pos = n * ELL + t;
      float v = (e & 3) == 0 ? 1.0f : 0.0f;
      if (pos < g.V) v = to_f(rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + e]);
      qv[((e >> 2) * ELL + t) * 4 + (e & 3)] = v;
    }
  }
}

// De-rotation (TR = false: c = M h) or its transpose (TR = true: M^T v) applied
// in place to an accumulator tile pair v[mt][nt] holding rows t = 16mt+4q+i and
// internal state columns 16nt + (lane % 16).
// col0: internal column of the first tile (the wave's column offset).
// ROT: 0 none, 1 complex (pairwise or half-split, both adjacent internal
// columns), 3 quaternion; fixed at compile time so each kernel carries one path.
template <bool TR, int NT, int ROT>
__device__ __forceinline__ void rotate_tiles(f4 (&v)[2][NT], const Geo& g, const float* cs, const float* sn,
                                    const float* qv, int col0 = 0) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  if constexpr (ROT == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
      const int col = col0 + 16 * nt + n;
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
          const float c = cs[alc * ELL + t], s = sg * sn[alc * ELL + t];
          const float y = TR ? (c * x - s * px) : (c * x + s * px);
          v[mt][nt][i] = act ? y : x;
        }
      __builtin_amdgcn_sched_barrier(0);  // bound the live range of the tile's temporaries
    }
  } else if constexpr (ROT == 3) {
    // Lane k of a quad holds component k of a 4-block. Row k of the left
    // Hamilton matrix of Q pairs Q[m'] with v[m' ^ k] under a sign fixed per
    // (k, m'), so c_k = sum_m' sign * Q[m'] * v[m' ^ k]; v[m' ^ k] is a quad
    // XOR exchange. The transpose (column k) has the same pairing, other signs.
    const int k = n & 3;
    // sign bit set = negative; bit m' of the mask for component k
    constexpr unsigned kRow = 0xE | (0x8 << 4) | (0x2 << 8) | (0x4 << 12);
    constexpr unsigned kCol = 0x0 | (0x6 << 4) | (0xC << 8) | (0xA << 12);
    const unsigned sm = ((TR ? kCol : kRow) >> (4 * k)) & 0xF;
    const float s0 = (sm & 1) ? -1.0f : 1.0f, s1 = (sm & 2) ? -1.0f : 1.0f;
    const float s2 = (sm & 4) ? -1.0f : 1.0f, s3 = (sm & 8) ? -1.0f : 1.0f;
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
      const int col = col0 + 16 * nt + n;
      const int jq = col >> 2;
      const bool act = jq < g.J;
      const int jqc = act ? jq : 0;
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float x = v[mt][nt][i];
          const float x1 = dpp<QP_SWAP1>(x), x2 = dpp<QP_X2>(x), x3 = dpp<QP_X3>(x);
          const int t = 16 * mt + 4 * q + i;
          const f4 Q = *reinterpret_cast<const f4*>(qv + (jqc * ELL + t) * 4);
          const float y = (s0 * Q[0]) * x + (s1 * Q[1]) * x1 + (s2 * Q[2]) * x2 + (s3 * Q[3]) * x3;
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
template <int NT, int ROT>
__device__ __forceinline__ void accum_drot(f4 (&racc)[2][NT], const f4 (&dc)[2][NT], const f4 (&keep)[2][NT],
                                  const Geo& g) {
  const int n = threadIdx.x & 15;
  if constexpr (ROT == 1) {
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
      __builtin_amdgcn_sched_barrier(0);
  } else if constexpr (ROT == 3) {
    // d_Q = d_c (x) conj(h): component k = sum_m' sign * d_c[m'] * h[m' ^ k],
    // d_c[m'] a quad broadcast and h[m' ^ k] a quad XOR exchange.
    const int k = n & 3;
    constexpr unsigned kSg = 0x0 | (0x5 << 4) | (0x9 << 8) | (0x3 << 12);  // bit m' set = negative
    const unsigned sm = (kSg >> (4 * k)) & 0xF;
    const float s0 = (sm & 1) ? -1.0f : 1.0f, s1 = (sm & 2) ? -1.0f : 1.0f;
    const float s2 = (sm & 4) ? -1.0f : 1.0f, s3 = (sm & 8) ? -1.0f : 1.0f;
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float a = dc[mt][nt][i], h = keep[mt][nt][i];
          const float a0 = dpp<QP_B0>(a), a1 = dpp<QP_B1>(a), a2 = dpp<QP_B2>(a), a3 = dpp<QP_B3>(a);
          const float h1 = dpp<QP_SWAP1>(h), h2 = dpp<QP_X2>(h), h3 = dpp<QP_X3>(h);
          racc[mt][nt][i] += (s0 * a0) * h + (s1 * a1) * h1 + (s2 * a2) * h2 + (s3 * a3) * h3;
          __builtin_amdgcn_sched_barrier(0);
        }
  }
}

}  // namespace mom

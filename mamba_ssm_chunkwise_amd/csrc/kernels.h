// Kernels of the state-moments path. One workgroup = 4 waves (256 lanes).
//
// Dataflow (sources: burn-mamba "recalculated.rs" and "backward.rs" source pages):
//   forward : k_carry (per-chunk decay-to-chunk-end GEMM, the pages' boundary
//             carry) -> k_scan (serial carry recurrence over chunks)
//             -> k_fwd (chunk states on MFMA, de-rotation, m2 on MFMA, m1)
//             -> k_reduce (fixed-order sum of per-workgroup partials)
//   backward: k_carry -> k_scan -> k_bwd (recompute states, d_c = c S + d_m1,
//             rotation VJP, d_W = L^T G, d_xhat, d_bhat, d_da; every chunk
//             independent because the carry cotangent enters only through
//             G[l-1]) -> k_dscan (reverse carry-cotangent recurrence, d_h0)
//             -> k_fix (the carry-cotangent terms of d_xhat, d_bhat, d_da)
//             -> k_zero_tail (zeros past the processed chunks).
#pragma once

#include "chunk.h"

namespace mom {

// ---------------------------------------------------------------------------
// LDS plans (shared by host sizing and device carving)
// ---------------------------------------------------------------------------
struct Lds {
  size_t a, d, L, lx, bs, ltp, ltx, rot, xr, S, xg, xgw, red, m1s, total;
};

__host__ __device__ __forceinline__ size_t al16(size_t x) { return (x + 15) & ~size_t(15); }

__host__ __device__ __forceinline__ size_t rot_bytes(const Geo& g) {
  if (g.rot_kind == 1 || g.rot_kind == 2) return al16((size_t)2 * ELL * g.A * 4);
  if (g.rot_kind == 3) return al16((size_t)ELL * g.J * 4 * 4);
  return 16;
}

// Forward main kernel: c exchange cx holds, per wave, the state-row tile as
// MFMA B fragments (K over tokens) for all NT column tiles.
__host__ __device__ __forceinline__ size_t frag_tile_bytes(int NT, int tsz) {
  return tsz == 2 ? (size_t)NT * 64 * 16 : (size_t)NT * 8 * 64 * 4;
}
__host__ __device__ __forceinline__ Lds lds_fwd(const Geo& g, int R, int tsz, int NT) {
  Lds l{};
  size_t o = 0;
  l.a = o; o += al16(ELL * 4);
  l.d = o; o += al16(ELL * 4);
  l.L = o; o += al16(ELL * (ELL + 1) * 4);
  l.bs = o; o += al16((size_t)R * g.KP * tsz);
  l.rot = o; o += rot_bytes(g);
  l.xr = o; o += al16((size_t)NW * g.KP * tsz);
  l.xgw = al16(frag_tile_bytes(NT, tsz));
  l.xg = o; o += l.xgw * NW;
  l.total = o;
  return l;
}

// Backward main kernel (16 waves: 4 state-row slots x 4 column quarters).
__host__ __device__ __forceinline__ Lds lds_bwd(const Geo& g, int R, int tsz, int NT) {
  Lds l{};
  size_t o = 0;
  l.a = o; o += al16(ELL * 4);
  l.d = o; o += al16(ELL * 4);
  l.L = o; o += al16(ELL * (ELL + 1) * 4);
  l.bs = o; o += al16((size_t)R * g.KP * tsz);
  l.ltp = o; o += al16((size_t)ELL * SLOTP * tsz);
  l.ltx = o; o += al16((size_t)g.K * SLOTP * tsz);
  l.rot = o; o += rot_bytes(g);
  l.xr = o; o += al16((size_t)NW * g.KP * tsz);
  l.S = o; o += al16((size_t)R * g.RP * tsz);
  // per state-row slot: the c tile [t][RP] for d_c, then (after a barrier) the
  // G tile as B fragments for d_bhat; the rotation-gradient reduction reuses it.
  const size_t xtile = (size_t)ELL * g.RP * tsz;
  const size_t gb = frag_tile_bytes(NT, tsz);
  l.xgw = al16(xtile > gb ? xtile : gb);
  size_t xg = l.xgw * NW;
  const size_t rb = (size_t)2 * NT * 64 * 16;          // rotation-gradient reduction
  const size_t dbt = (size_t)g.K * g.RP * tsz;          // d_bhat tile
  if (xg < rb) xg = rb;
  if (xg < dbt) xg = dbt;
  l.xg = o; o += al16(xg);
  l.m1s = o; o += al16((size_t)NCW * NW * g.K * 4);     // d_xhat partials of the column quarters
  l.red = o; o += al16((size_t)(4 * NCW * ELL + ELL) * 4);
  l.total = o;
  return l;
}

// Carry kernel: as [PK][KP] and bs [R][KP].
__host__ __device__ __forceinline__ Lds lds_carry(const Geo& g, int R, int tsz, int PK) {
  Lds l{};
  size_t o = 0;
  l.a = o; o += al16(ELL * 4);
  l.d = o; o += al16(ELL * 4);
  l.L = o; o += al16(ELL * (ELL + 1) * 4);
  l.lx = o; o += al16((size_t)PK * g.KP * tsz);  // x^T scaled (A operand)
  l.bs = o; o += al16((size_t)R * g.KP * tsz);
  l.total = o;
  return l;
}

// Correction kernel: dp [PK][RP], dpt [R][PP], bn [K][RP], xn [K][PP].
__host__ __device__ __forceinline__ Lds lds_fix(const Geo& g, int R, int tsz, int PK) {
  Lds l{};
  size_t o = 0;
  l.a = o; o += al16(ELL * 4);
  l.d = o; o += al16(ELL * 4);
  l.L = o; o += al16(ELL * (ELL + 1) * 4);
  l.lx = o; o += al16((size_t)PK * g.RP * tsz);   // dp
  l.ltx = o; o += al16((size_t)R * g.PP * tsz);   // dpt
  l.bs = o; o += al16((size_t)g.K * g.RP * tsz);  // bn
  l.xr = o; o += al16((size_t)g.K * g.PP * tsz);  // xn
  l.red = o; o += al16((size_t)(g.K + NTH + ELL + 4) * 4);
  l.total = o;
  return l;
}

// ---------------------------------------------------------------------------
// Chunk states of one state row p0 over NTC column tiles starting at col0:
// acc[mt][nt] = h~[t = 16mt+4q+i][col0 + 16nt + m]
//   = d_t h_-[p0][col] + sum_{k=(j,c), j<=t} L[t,j] xhat[j,c,p0] bhat[j,c,col]
// (chunk_states of the recalculated.rs source page, folded (j,c) write axis).
// Rows at positions >= V are zeroed.
// ---------------------------------------------------------------------------
template <typename T, int NTC, int CK>
__device__ __forceinline__ void chunk_states_row(f4 (&acc)[2][NTC], const Geo& g, int n, const float* s_d,
                                                 const float* s_L, const T* bs, const T* xrow,
                                                 const float* hrow, int col0) {
  constexpr int KS = MM<T>::KS, E = MM<T>::E, K = ELL * CK, KP = K + pad_of<T>();
  const int lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NTC; nt++) {
    const int col = col0 + 16 * nt + m;
    const float hv = (hrow != nullptr && col < g.r) ? hrow[col] : 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int i = 0; i < 4; i++) acc[mt][nt][i] = s_d[16 * mt + 4 * q + i] * hv;
  }
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
    // writes k = (j, ci) with j <= 16mt + 15 only (L is zero above the diagonal)
    constexpr int NKS0 = (16 * CK + KS - 1) / KS, NKS1 = (32 * CK + KS - 1) / KS;
    const int t = 16 * mt + m;
    const float* Lrow = s_L + t * (ELL + 1);
#pragma unroll
    for (int ks = 0; ks < (mt == 0 ? NKS0 : NKS1); ks++) {
      const int k0 = ks * KS + E * q;
      typename MM<T>::frag a;
      if constexpr (E == 1) {
        a = Lrow[k0 / CK] * to_f(xrow[k0]);
      } else {
        const auto xv = ld_frag(xrow + k0);
#pragma unroll
        for (int e = 0; e < E; e++) a[e] = to_t<T>(Lrow[(k0 + e) / CK] * to_f(xv[e]));
      }
#pragma unroll
      for (int nt = 0; nt < NTC; nt++) {
        const auto b = ld_frag(bs + (col0 + 16 * nt + m) * KP + k0);
        acc[mt][nt] = MM<T>::mma(a, b, acc[mt][nt]);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < 2; mt++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if (n * ELL + 16 * mt + 4 * q + i >= g.V) {
#pragma unroll
        for (int nt = 0; nt < NTC; nt++) acc[mt][nt][i] = 0.0f;
      }
    }
}

// Stage the x row block of one round (4 state rows, one per wave): xr[w][k].
template <typename T, int CK>
__device__ __forceinline__ void stage_xround(const Geo& g, const T* __restrict__ xhat, int bi, int hi, int n,
                                    int round, T* xr) {
  constexpr int K = ELL * CK, KP = K + pad_of<T>();
  for (int idx = threadIdx.x; idx < 4 * K; idx += blockDim.x) {
    const int k = idx >> 2, ww = idx & 3;
    const int p0 = 4 * round + ww;
    const int j = k / CK, ci = k % CK;
    const int pos = n * ELL + j;
    float v = 0.0f;
    if (p0 < g.p && pos < g.V && ci < g.c)
      v = to_f(xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + p0]);
    xr[ww * KP + k] = to_t<T>(v);
  }
}

// ---------------------------------------------------------------------------
// k_carry: U_n[p][col] = sum_{k=(j,c)} exp(a_last - a_j) xhat[j,c,p] bhat[j,c,col]
// for chunks n < NK-1, and dec_n = exp(a_last) (boundary_carries, backward.rs
// source page: the decay-to-chunk-end GEMM).
// ---------------------------------------------------------------------------
template <typename T, int NT, int CK>
__global__ __launch_bounds__(NTH, 1) void k_carry(Geo g, int PK, const T* __restrict__ xhat,
                                                   const T* __restrict__ bhat,
                                                   const T* __restrict__ da, float* carry,
                                                   float* dec) {
  constexpr int R = 16 * NT, KS = MM<T>::KS, E = MM<T>::E, K = ELL * CK, KP = K + pad_of<T>();
  extern __shared__ __align__(16) unsigned char smem[];
  const Lds L = lds_carry(g, R, sizeof(T), PK);
  float* s_a = (float*)(smem + L.a);
  float* s_d = (float*)(smem + L.d);
  float* s_L = (float*)(smem + L.L);
  T* as = (T*)(smem + L.lx);
  T* bs = (T*)(smem + L.bs);
  const int per = g.NK - 1;
  const int bh = blockIdx.x / per, n = blockIdx.x % per;
  const int bi = bh / g.h, hi = bh % g.h;
  g.V = chain_len(g, bi);  // this sequence's valid length (per-sequence lengths)
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;

  stage_decay(g, da, bi, hi, n, s_a, s_d, s_L);
  // bf16 rows of 16-byte pieces (p and r multiples of 8): one wide load per 8
  // values, work items over (j,c) fastest so the LDS writes of a wave are
  // consecutive; otherwise element by element
  constexpr bool BF = sizeof(T) == 2;
  const bool wide = BF && g.p % 8 == 0 && g.r % 8 == 0;
  const float* wl = s_L + (ELL - 1) * (ELL + 1);  // L[l-1][j] = exp(a_last - a_j)
  if constexpr (BF) {
    if (wide) {
      for (int idx = threadIdx.x; idx < K * (R / 8); idx += NTH) {
        const int k = idx % K, c8 = idx / K;
        const int j = k / CK, ci = k % CK, pos = n * ELL + j;
        u4 v = u4{0u, 0u, 0u, 0u};
        if (8 * c8 < g.r && pos < g.V && ci < g.c)
          v = *reinterpret_cast<const u4*>(bhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + 8 * c8);
        const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
        for (int u = 0; u < 8; u++) {
          const int cc = 8 * c8 + u;  // caller column; internal columns interleave half-split pairs
          bs[(cc < g.r ? inv_perm_rc(g, cc) : cc) * KP + k] = e[u];
        }
      }
    }
  }
  if (!wide) stage_bhat<T, R, CK>(g, bhat, bi, hi, n, bs);
  __syncthreads();  // the decays (wl) are staged
  if constexpr (BF) {
    if (wide) {
      for (int idx = threadIdx.x; idx < K * (PK / 8); idx += NTH) {
        const int k = idx % K, p8 = idx / K;
        const int j = k / CK, ci = k % CK, pos = n * ELL + j;
        u4 v = u4{0u, 0u, 0u, 0u};
        if (8 * p8 < g.p && pos < g.V && ci < g.c)
          v = *reinterpret_cast<const u4*>(xhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + 8 * p8);
        const T* e = reinterpret_cast<const T*>(&v);
        const float f = wl[j];
#pragma unroll
        for (int u = 0; u < 8; u++) as[(8 * p8 + u) * KP + k] = to_t<T>(to_f(e[u]) * f);
      }
    }
  }
  if (!wide) {
    for (int idx = threadIdx.x; idx < K * PK; idx += NTH) {
      const int k = idx / PK, pp = idx % PK;
      const int j = k / CK, ci = k % CK;
      const int pos = n * ELL + j;
      float v = 0.0f;
      if (pp < g.p && ci < g.c && pos < g.V)
        v = to_f(xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pp]) * wl[j];
      as[pp * KP + k] = to_t<T>(v);
    }
  }
  __syncthreads();
  const int MT = PK / 16;
  constexpr int nks = K / KS;
#pragma unroll
  for (int mi = 0; mi < 2; mi++) {
    const int mt = w + 4 * mi;
    if (mt >= MT) break;
    f4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++) acc[nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < nks; ks++) {
      const int k0 = ks * KS + E * q;
      const auto a = ld_frag(as + (16 * mt + m) * KP + k0);
#pragma unroll
      for (int nt = 0; nt < NT; nt++) acc[nt] = MM<T>::mma(a, ld_frag(bs + (16 * nt + m) * KP + k0), acc[nt]);
    }
    float* out = carry + ((size_t)bh * g.NK + n) * g.p * g.r;
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
      const int col = 16 * nt + m;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int pp = 16 * mt + 4 * q + i;
        if (pp < g.p && col < g.r) out[(size_t)pp * g.r + col] = acc[nt][i];
      }
    }
  }
  if (threadIdx.x == 0) dec[(size_t)bh * g.NK + n] = s_d[ELL - 1];
}

// k_scan: h_-(0) = h0, h_-(n+1) = dec_n h_-(n) + U_n, written in place over U
// (rows n % cstride == 0; the others keep U).
template <typename T>
__global__ __launch_bounds__(NTH) void k_scan(Geo g, const T* __restrict__ h0, float* carry,
                                              const float* __restrict__ dec) {
  const int bh = blockIdx.x;
  const int e = blockIdx.y * NTH + threadIdx.x;
  const int pr = g.p * g.r;
  if (e >= pr) return;
  const int p0 = e / g.r, rc = e % g.r;
  float h = h0 ? to_f(h0[((size_t)bh * g.p + p0) * g.r + perm_rc(g, rc)]) : 0.0f;
  float* C = carry + (size_t)bh * g.NK * pr + e;
  const float* D = dec + (size_t)bh * g.NK;
  const int last = g.NK - 1;
  for (int n0 = 0; n0 < g.NK; n0 += 8) {
    float u[8], dd[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int n = n0 + k;
      u[k] = n < last ? C[(size_t)n * pr] : 0.0f;
      dd[k] = n < last ? D[n] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int n = n0 + k;
      if (n < g.NK) {
        if (n % g.cstride == 0) C[(size_t)n * pr] = h;
        h = dd[k] * h + u[k];
      }
    }
  }
}

// k_scan4: k_scan on four consecutive state elements per thread (p r a multiple
// of four), 16-byte loads and stores, with the next batch of chunks' U loads in
// flight while the current batch is stored. Each element takes the same fp32
// operations in the same order as in k_scan.
template <typename T>
__global__ __launch_bounds__(NTH) void k_scan4(Geo g, const T* __restrict__ h0, float* carry,
                                               const float* __restrict__ dec) {
  constexpr int B = 8;  // chunks per batch
  const int bh = blockIdx.x;
  const int e = 4 * (blockIdx.y * NTH + threadIdx.x);
  const int pr = g.p * g.r;
  if (e >= pr) return;
  f4 h;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int p0 = (e + i) / g.r, rc = (e + i) % g.r;
    h[i] = h0 ? to_f(h0[((size_t)bh * g.p + p0) * g.r + perm_rc(g, rc)]) : 0.0f;
  }
  float* C = carry + (size_t)bh * g.NK * pr + e;
  const float* D = dec + (size_t)bh * g.NK;
  const int last = g.NK - 1;
  f4 u[B];
  float dd[B];
  auto load = [&](int n0) {
#pragma unroll
    for (int k = 0; k < B; k++) {
      const int n = n0 + k;
      u[k] = n < last ? *reinterpret_cast<const f4*>(C + (size_t)n * pr) : f4{0.0f, 0.0f, 0.0f, 0.0f};
      dd[k] = n < last ? D[n] : 0.0f;
    }
  };
  load(0);
  for (int n0 = 0; n0 < g.NK; n0 += B) {
    f4 uc[B];
    float dc[B];
#pragma unroll
    for (int k = 0; k < B; k++) {
      uc[k] = u[k];
      dc[k] = dd[k];
    }
    if (n0 + B < g.NK) load(n0 + B);  // rows past this batch: not written by it
#pragma unroll
    for (int k = 0; k < B; k++) {
      const int n = n0 + k;
      if (n < g.NK) {
        if (n % g.cstride == 0) *reinterpret_cast<f4*>(C + (size_t)n * pr) = h;
#pragma unroll
        for (int i = 0; i < 4; i++) h[i] = dc[k] * h[i] + uc[k][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_fwd: chunk states, de-rotation, m2 += c^T c and m1 += sum_t c. One workgroup
// walks G chunks of one (b,h) chain; each round, wave w computes state row
// 4*round + w and publishes c as MFMA B fragments (K over tokens); the four
// waves then own a 2x2 tiling of m2 and accumulate the round's four rows.
// Each workgroup writes one m2 partial and owns one m1 partial.
// ---------------------------------------------------------------------------
template <typename T, int NT, int ROT, int CK>
__global__ __launch_bounds__(NTH, 1) void k_fwd(Geo g, const T* __restrict__ xhat,
                                                 const T* __restrict__ bhat,
                                                 const T* __restrict__ da,
                                                 const T* __restrict__ rot,
                                                 const float* __restrict__ carry, float* m2part,
                                                 float* m1part) {
  static_assert(NT >= 2, "column tiles are split in halves");
  constexpr int R = 16 * NT, NKT = ELL / MM<T>::KS, NH = NT / 2, KP = ELL * CK + pad_of<T>();
  extern __shared__ __align__(16) unsigned char smem[];
  const Lds L = lds_fwd(g, R, sizeof(T), NT);
  float* s_a = (float*)(smem + L.a);
  float* s_d = (float*)(smem + L.d);
  float* s_L = (float*)(smem + L.L);
  T* bs = (T*)(smem + L.bs);
  float* cs = (float*)(smem + L.rot);
  float* sn = cs + ELL * g.A;
  float* qv = cs;
  T* xr = (T*)(smem + L.xr);
  unsigned char* cx = smem + L.xg;

  const int bh = blockIdx.x / g.NGR, gi = blockIdx.x % g.NGR;
  const int bi = bh / g.h, hi = bh % g.h;
  g.V = chain_len(g, bi);  // this sequence's valid length (per-sequence lengths)
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;
  const int wi = w >> 1, wj = w & 1;  // this wave's m2 tiles: rows half wi, cols half wj
  const int nrounds = (g.p + 3) / 4;
  float* m1o = m1part + ((size_t)bh * g.NGR + gi) * g.p * R;
  f4 m2acc[NH][NH];
#pragma unroll
  for (int a = 0; a < NH; a++)
#pragma unroll
    for (int b = 0; b < NH; b++) m2acc[a][b] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  const int n0 = gi * g.G;
  const int n1 = (n0 + g.G < g.NK) ? n0 + g.G : g.NK;
  for (int n = n0; n < n1; n++) {
    __syncthreads();
    stage_decay(g, da, bi, hi, n, s_a, s_d, s_L);
    stage_bhat<T, R, CK>(g, bhat, bi, hi, n, bs);
    stage_rot(g, rot, bi, hi, n, cs, sn, qv);
    for (int round = 0; round < nrounds; round++) {
      stage_xround<T, CK>(g, xhat, bi, hi, n, round, xr);
      __syncthreads();
      const int p0 = 4 * round + w;
      const bool valid = p0 < g.p;
      const float* hrow = valid ? carry + (((size_t)bh * g.NK + n) * g.p + p0) * g.r : nullptr;
      f4 acc[2][NT];
      chunk_states_row<T, NT, CK>(acc, g, n, s_d, s_L, bs, xr + w * KP, hrow, 0);
      rotate_tiles<false, NT, ROT>(acc, g, cs, sn, qv);
      // m1[p0][col] += sum over the chunk's tokens (this wave owns row p0)
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        float sum = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++) sum += acc[mt][nt][i];
        sum = col4_sum(sum);
        if (q == 0 && valid) {
          float* dst = m1o + (size_t)p0 * R + 16 * nt + m;
          *dst = (n == n0 ? 0.0f : *dst) + sum;
        }
      }
      // publish c as B fragments: K = tokens (slot order), one tile per column block
      unsigned char* mine = cx + (size_t)w * L.xgw;
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        const f4 v2[2] = {acc[0][nt], acc[1][nt]};
        if constexpr (NKT == 1) {
          ((bf8*)mine)[nt * 64 + lane] = pack_tslots(v2, 0, T{});
        } else {
#pragma unroll
          for (int ks = 0; ks < NKT; ks++) ((float*)mine)[(nt * NKT + ks) * 64 + lane] = pack_tslots(v2, ks, T{});
        }
      }
      __syncthreads();
      // m2 tile (16(wi*NH+a), 16(wj*NH+b)) += sum over the round's rows and tokens
#pragma unroll
      for (int src = 0; src < NW; src++) {
        const unsigned char* fr = cx + (size_t)src * L.xgw;
#pragma unroll
        for (int ks = 0; ks < NKT; ks++) {
          typename MM<T>::frag fa[NH], fb[NH];
#pragma unroll
          for (int a = 0; a < NH; a++) {
            const int ta = wi * NH + a, tb = wj * NH + a;
            if constexpr (NKT == 1) {
              fa[a] = ((const bf8*)fr)[ta * 64 + lane];
              fb[a] = ((const bf8*)fr)[tb * 64 + lane];
            } else {
              fa[a] = ((const float*)fr)[(ta * NKT + ks) * 64 + lane];
              fb[a] = ((const float*)fr)[(tb * NKT + ks) * 64 + lane];
            }
          }
#pragma unroll
          for (int a = 0; a < NH; a++)
#pragma unroll
            for (int b = 0; b < NH; b++) m2acc[a][b] = MM<T>::mma(fa[a], fb[b], m2acc[a][b]);
        }
      }
    }
  }
  // m2 partial: this wave's (NH x NH) tiles, written straight out
  float* m2o = m2part + ((size_t)bh * g.NGR + gi) * R * R;
#pragma unroll
  for (int a = 0; a < NH; a++)
#pragma unroll
    for (int b = 0; b < NH; b++)
#pragma unroll
      for (int i = 0; i < 4; i++)
        m2o[(16 * (wi * NH + a) + 4 * q + i) * R + 16 * (wj * NH + b) + m] = m2acc[a][b][i];
}

}  // namespace mom

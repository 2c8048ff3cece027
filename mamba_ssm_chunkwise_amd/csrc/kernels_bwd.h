// Backward kernels (backward.rs source page, module doc "Gradient math" and
// moments_phys_bwd). Per chunk, with the carry cotangent d_h+ set aside:
//   d_c[t]  = mask_t (c_t (d_m2 + d_m2^T) + d_m1)
//   G[t]    = M_t^T d_c[t]                       (rotation transpose)
//   d_theta = sum_p (d_c_x c_y - d_c_y c_x), d_Q = sum_p d_c (x) conj(h~)
//   local   = sum_t d_t G[t]                     (carry cotangent contribution)
//   d_W_j   = sum_{t>=j} L[t,j] G[t],  d_xhat = d_W bhat,  d_bhat = d_W^T xhat
//   d_da_s  = sum_{t>=s} <G[t], h~[t]> - sum_{j>=s} <d_W_j, W_j>
// The last line is the pages' rev-cumsum identity with its two row sums
// rewritten: scal_t + sum_j A[t,j] = <G[t], h~[t]> (h~[t] = d_t h_- + sum_j L W_j)
// and sum_t A[t,j] = <d_W_j, W_j> = sum_c <xhat[j,c], d_xhat[j,c]>.
// The carry cotangent enters only through G[l-1] += d_h+, which adds
//   d_xhat[j,c] += L[l-1,j] d_h+ bhat[j,c],  d_bhat[j,c] += L[l-1,j] d_h+^T xhat[j,c],
//   d_da_s += <d_h+, h~[l-1]> - sum_{j>=s} L[l-1,j] <d_h+, W_j>
// and is applied by k_fix once the reverse recurrence D(n) = local(n) +
// exp(a_last(n)) D(n+1) has been scanned (k_dscan).
#pragma once

#include <type_traits>

#include "kernels.h"

namespace mom {

// Waves: w = 0..15, state-row slot u = w & 3 (row 4*round + u), column
// quarter v = w >> 2 (column tiles [v*NQ, v*NQ + NQ)). A row's four waves
// share the state A operand, exchange c through LDS for d_c (K over all
// columns), and combine their quarters of the d_xhat dot products.
template <typename T, int NT, int ROT, int CK>
__global__ __launch_bounds__(NTHB, 1) void k_bwd(
    Geo g, const T* __restrict__ xhat, const T* __restrict__ bhat, const T* __restrict__ da,
    const T* __restrict__ rot, const float* __restrict__ carry, const float* __restrict__ dm2,
    const float* __restrict__ dm1, float* Db, T* d_xhat, T* d_bhat, T* d_da, T* d_rot) {
  static_assert(NT >= NCW, "column tiles are split in quarters");
  constexpr int R = 16 * NT, KS = MM<T>::KS, E = MM<T>::E, NKT = ELL / KS, NH = NT / NCW;
  constexpr int K = ELL * CK, KP = K + pad_of<T>(), RP = R + pad_of<T>(), MTB = K / 16;
  extern __shared__ __align__(16) unsigned char smem[];
  const Lds L = lds_bwd(g, R, sizeof(T), NT);
  float* s_a = (float*)(smem + L.a);
  float* s_d = (float*)(smem + L.d);
  float* s_L = (float*)(smem + L.L);
  T* bs = (T*)(smem + L.bs);
  T* ltp = (T*)(smem + L.ltp);
  T* ltx = (T*)(smem + L.ltx);
  float* cs = (float*)(smem + L.rot);
  float* sn = cs + ELL * g.A;
  float* qv = cs;
  T* xr = (T*)(smem + L.xr);
  T* S = (T*)(smem + L.S);
  unsigned char* xg = smem + L.xg;
  float* xpart = (float*)(smem + L.m1s);
  float* rsum = (float*)(smem + L.red);   // [16 waves][ELL]
  float* ddv = rsum + 4 * NCW * ELL;      // [ELL]

  const int bh = blockIdx.x / g.NGR, gi = blockIdx.x % g.NGR;
  const int bi = bh / g.h, hi = bh % g.h;
  g.V = chain_len(g, bi);  // this sequence's valid length (per-sequence lengths)
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;
  const int u = w & 3, v = w >> 2;
  const int col0 = 16 * NH * v;
  const int nrounds = (g.p + 3) / 4;
  constexpr bool cplx = ROT == 1;

  // S = d_m2 + d_m2^T in internal column order (symmetric, so it serves as the
  // K-contiguous B operand of d_c = c S).
  for (int idx = threadIdx.x; idx < R * R; idx += NTHB) {
    const int a = idx / R, b = idx % R;
    float val = 0.0f;
    if (a < g.r && b < g.r) {
      const int pa = perm_rc(g, a), pb = perm_rc(g, b);
      const float* D2 = dm2 + (size_t)bh * g.r * g.r;
      val = D2[pa * g.r + pb] + D2[pb * g.r + pa];
    }
    S[a * RP + b] = to_t<T>(val);
  }

  const int n0 = gi * g.G;
  const int n1 = (n0 + g.G < g.NK) ? n0 + g.G : g.NK;
  for (int n = n0; n < n1; n++) {
    __syncthreads();
    stage_decay(g, da, bi, hi, n, s_a, s_d, s_L);
    stage_bhat<T, R, CK>(g, bhat, bi, hi, n, bs);
    stage_rot(g, rot, bi, hi, n, cs, sn, qv);
    stage_lt<T, CK>(s_L, ltp, ltx);

    f4 racc[2][NH], dbacc[2][NH];
    f4 gacc[2];
    float ccol = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      gacc[mt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int nt = 0; nt < NH; nt++) {
        racc[mt][nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        dbacc[mt][nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }

    for (int round = 0; round < nrounds; round++) {
      stage_xround<T, CK>(g, xhat, bi, hi, n, round, xr);
      __syncthreads();  // (A) xr, and on the first round all chunk staging
      const int p0 = 4 * round + u;
      const bool valid = p0 < g.p;
      const float* hrow = valid ? carry + (((size_t)bh * g.NK + n) * g.p + p0) * g.r : nullptr;
      T* X = (T*)(xg + (size_t)u * L.xgw);

      // states h~ and c for this wave's column half
      f4 keep[2][NH];
      chunk_states_row<T, NH, CK>(keep, g, n, s_d, s_L, bs, xr + u * KP, hrow, col0);
      f4 dc[2][NH];
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nt = 0; nt < NH; nt++) dc[mt][nt] = keep[mt][nt];
      rotate_tiles<false, NH, ROT>(dc, g, cs, sn, qv, col0);  // dc holds c for now
      if constexpr (cplx) {
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int nt = 0; nt < NH; nt++) keep[mt][nt] = dc[mt][nt];
      }
      // c -> X[u] rows [t][col] (A operand of d_c, K over all columns)
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nt = 0; nt < NH; nt++)
#pragma unroll
          for (int i = 0; i < 4; i++)
            X[(16 * mt + 4 * q + i) * RP + col0 + 16 * nt + m] = to_t<T>(dc[mt][nt][i]);
      __syncthreads();  // (B) every quarter of every c row is in X
      // d_c = c S + d_m1 on this wave's columns, masked past V
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nt = 0; nt < NH; nt++) dc[mt][nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < R / KS; ks++) {
        const int k0 = ks * KS + E * q;
        const auto a0 = ld_frag(X + m * RP + k0);
        const auto a1 = ld_frag(X + (16 + m) * RP + k0);
#pragma unroll
        for (int nt = 0; nt < NH; nt++) {
          const auto b = ld_frag(S + (col0 + 16 * nt + m) * RP + k0);
          dc[0][nt] = MM<T>::mma(a0, b, dc[0][nt]);
          dc[1][nt] = MM<T>::mma(a1, b, dc[1][nt]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NH; nt++) {
        const int col = col0 + 16 * nt + m;
        const float dv = (valid && col < g.r) ? dm1[((size_t)bh * g.p + p0) * g.r + perm_rc(g, col)] : 0.0f;
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const bool live = n * ELL + 16 * mt + 4 * q + i < g.V;
            dc[mt][nt][i] = live ? dc[mt][nt][i] + dv : 0.0f;
          }
      }
      // rotation gradient; <d_c, c> = <G, h~> (row term of d_da)
      accum_drot<NH, ROT>(racc, dc, keep, g);
      if constexpr (ROT != 3) {
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int nt = 0; nt < NH; nt++)
#pragma unroll
            for (int i = 0; i < 4; i++) gacc[mt][i] += dc[mt][nt][i] * keep[mt][nt][i];
      }
      rotate_tiles<true, NH, ROT>(dc, g, cs, sn, qv, col0);  // dc now holds G
      if constexpr (ROT == 3) {
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int nt = 0; nt < NH; nt++)
#pragma unroll
            for (int i = 0; i < 4; i++) gacc[mt][i] += dc[mt][nt][i] * keep[mt][nt][i];
      }
      // local(n)[p0][col] = sum_t d_t G[t][col]
#pragma unroll
      for (int nt = 0; nt < NH; nt++) {
        float sum = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++) sum += s_d[16 * mt + 4 * q + i] * dc[mt][nt][i];
        sum = col4_sum(sum);
        const int col = col0 + 16 * nt + m;
        if (q == 0 && valid && col < g.r) Db[(((size_t)bh * g.NK + n) * g.p + p0) * g.r + col] = sum;
      }
      // d_W[j][col] = sum_t L[t][j] G[t][col] (K over tokens, B from registers)
      f4 dw[2][NH];
#pragma unroll
      for (int jt = 0; jt < 2; jt++)
#pragma unroll
        for (int nt = 0; nt < NH; nt++) dw[jt][nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < NKT; ks++) {
#pragma unroll
        for (int jt = 0; jt < 2; jt++) {
          const auto a = ld_frag(ltp + (16 * jt + m) * SLOTP + ks * KS + E * q);
#pragma unroll
          for (int nt = 0; nt < NH; nt++) {
            const f4 gv[2] = {dc[0][nt], dc[1][nt]};
            dw[jt][nt] = MM<T>::mma(a, pack_tslots(gv, ks, T{}), dw[jt][nt]);
          }
        }
      }
      // this quarter's share of d_xhat[j,c,p0] = sum_col d_W[j][col] bhat[j,c,col],
      // dropped into LDS; the quarters are added in a flat pass below
      float* xp = xpart + (v * NW + u) * K;
#pragma unroll
      for (int jt = 0; jt < 2; jt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int j = 16 * jt + 4 * q + i;
#pragma unroll
          for (int ci = 0; ci < CK; ci++) {
            if (ci < g.c) {
              float part = 0.0f;
#pragma unroll
              for (int nt = 0; nt < NH; nt++)
                part += dw[jt][nt][i] * to_f(bs[(col0 + 16 * nt + m) * KP + j * CK + ci]);
              part = row16_sum(part);
              if (m == 0) xp[j * CK + ci] = part;
            }
          }
        }
      __syncthreads();  // (C) X reads done; every quarter's partials visible
      // G as B fragments (K over tokens) for d_bhat, into this row's slot
#pragma unroll
      for (int nt = 0; nt < NH; nt++) {
        const f4 gv[2] = {dc[0][nt], dc[1][nt]};
        const int tile = NH * v + nt;
        if constexpr (NKT == 1) {
          ((bf8*)X)[tile * 64 + lane] = pack_tslots(gv, 0, T{});
        } else {
#pragma unroll
          for (int ks = 0; ks < NKT; ks++) ((float*)X)[(tile * NKT + ks) * 64 + lane] = pack_tslots(gv, ks, T{});
        }
      }
      // d_xhat of the round's rows; thread (uu, k) also keeps its share of the
      // d_da column term sum_c <xhat[j,c], d_xhat[j,c]>
      if (threadIdx.x < NW * K) {
        const int uu = threadIdx.x / K, k = threadIdx.x % K;
        const int pr0 = 4 * round + uu;
        const int j = k / CK, ci = k % CK;
        float val = 0.0f;
        if (ci < g.c) {
#pragma unroll
          for (int vv = 0; vv < NCW; vv++) val += xpart[(vv * NW + uu) * K + k];
        }
        ccol += val * to_f(xr[uu * KP + k]);
        const int pos = n * ELL + j;
        if (d_xhat != nullptr && ci < g.c && pr0 < g.p && pos < g.s)
          d_xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pr0] = to_t<T>(val);
      }
      __syncthreads();  // (D) every row's G fragments are published
      // d_bhat[(j,c)][col] += sum over (t, this round's rows) L[t,j] xhat[j,c,p] G[t][col]
#pragma unroll
      for (int mi = 0; mi < 2; mi++) {
        const int mtb = u + 4 * mi;
        if (mtb < MTB) {
          const int k = 16 * mtb + m;
#pragma unroll
          for (int src = 0; src < NW; src++) {
            const float xs = to_f(xr[src * KP + k]);
            const unsigned char* gb = xg + (size_t)src * L.xgw;
#pragma unroll
            for (int ks = 0; ks < NKT; ks++) {
              typename MM<T>::frag a;
              const T* lt = ltx + k * SLOTP + ks * KS + E * q;
              if constexpr (E == 1) {
                a = to_f(lt[0]) * xs;
              } else {
                const auto lv = ld_frag(lt);
#pragma unroll
                for (int e = 0; e < E; e++) a[e] = to_t<T>(to_f(lv[e]) * xs);
              }
#pragma unroll
              for (int nt = 0; nt < NH; nt++) {
                const int tile = NH * v + nt;
                typename MM<T>::frag b;
                if constexpr (NKT == 1) b = ((const bf8*)gb)[tile * 64 + lane];
                else b = ((const float*)gb)[(tile * NKT + ks) * 64 + lane];
                dbacc[mi][nt] = MM<T>::mma(a, b, dbacc[mi][nt]);
              }
            }
          }
        }
      }
      __syncthreads();  // (E) before the next round overwrites xr and the slots
    }

    // ---- chunk end: d_bhat, staged through LDS and written row by row --------
    if (d_bhat != nullptr) {
      T* DBs = (T*)xg;  // [K][RP]
#pragma unroll
      for (int mi = 0; mi < 2; mi++) {
        const int mtb = u + 4 * mi;
        if (mtb < MTB) {
#pragma unroll
          for (int nt = 0; nt < NH; nt++)
#pragma unroll
            for (int i = 0; i < 4; i++)
              DBs[(16 * mtb + 4 * q + i) * RP + col0 + 16 * nt + m] = to_t<T>(dbacc[mi][nt][i]);
        }
      }
      __syncthreads();
      for (int idx = threadIdx.x; idx < K * g.r; idx += NTHB) {
        const int k = idx / g.r, ra = idx - k * g.r;
        const int j = k / CK, ci = k % CK;
        const int pos = n * ELL + j;
        if (pos < g.s && ci < g.c)
          d_bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + ra] = DBs[k * RP + inv_perm_rc(g, ra)];
      }
      __syncthreads();
    }
    // ---- rotation gradient: fixed-order sum over the four row slots, in the
    // accumulator layout (one vector per lane and tile), then gathered --------
    if (ROT != 0 && d_rot != nullptr) {
      f4* RB = (f4*)xg;  // [2][NT][64]
      for (int uu = 0; uu < NW; uu++) {
        if (u == uu) {
#pragma unroll
          for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int nt = 0; nt < NH; nt++) {
              f4* dst = RB + (mt * NT + NH * v + nt) * 64 + lane;
              *dst = (uu == 0 ? f4{0.0f, 0.0f, 0.0f, 0.0f} : *dst) + racc[mt][nt];
            }
        }
        __syncthreads();
      }
      const int rwi = cplx ? g.A : 4 * g.J;
      const float* RBf = (const float*)RB;
      for (int idx = threadIdx.x; idx < ELL * rwi; idx += NTHB) {
        const int t = idx / rwi, e = idx % rwi;
        const int col = cplx ? 2 * e : e;  // complex: the even column holds d_theta
        const int tl = ((col >> 4) + (t >> 4) * NT) * 64 + 16 * ((t & 15) >> 2) + (col & 15);
        const int pos = n * ELL + t;
        if (pos < g.s) d_rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + e] = to_t<T>(RBf[tl * 4 + (t & 3)]);
      }
    }
    // ---- d_da (without the carry-cotangent terms) ---------------------------
    // row term per token from every wave; column term per (j,c) from the flat pass
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float gs = row16_sum(gacc[mt][i]);
        if (m == 0) rsum[w * ELL + 16 * mt + 4 * q + i] = gs;
      }
    float* cw = xpart;  // reuse: [NW][K] column-term shares
    if (threadIdx.x < NW * K) cw[threadIdx.x] = ccol;
    __syncthreads();
    if (threadIdx.x == 0) {
      float acc = 0.0f;
      for (int t = ELL - 1; t >= 0; t--) {
        float rt = 0.0f, ct = 0.0f;
        for (int ww = 0; ww < 4 * NCW; ww++) rt += rsum[ww * ELL + t];
        for (int uu = 0; uu < NW; uu++)
          for (int ci = 0; ci < g.c; ci++) ct += cw[uu * K + t * CK + ci];
        acc += rt - ct;
        ddv[t] = acc;
      }
    }
    __syncthreads();
    if (threadIdx.x < ELL && d_da != nullptr) {
      const int pos = n * ELL + threadIdx.x;
      if (pos < g.s) d_da[((size_t)bi * g.s + pos) * g.h + hi] = to_t<T>(ddv[threadIdx.x]);
    }
  }
}

// k_dscan: D(n) = local(n) + dec_n D(n+1), D(NK) = 0. Db[n] <- D(n+1) (the
// cotangent entering chunk n from its successor); d_h0 = D(0).
template <typename T>
__global__ __launch_bounds__(NTH) void k_dscan(Geo g, float* Db, const float* __restrict__ dec,
                                               T* d_h0) {
  const int bh = blockIdx.x;
  const int e = blockIdx.y * NTH + threadIdx.x;
  const int pr = g.p * g.r;
  if (e >= pr) return;
  float* C = Db + (size_t)bh * g.NK * pr + e;
  const float* Dc = dec + (size_t)bh * g.NK;
  float D = 0.0f;
  for (int nb = g.NK - 1; nb >= 0; nb -= 8) {
    float l[8], dd[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int n = nb - k;
      l[k] = n >= 0 ? C[(size_t)n * pr] : 0.0f;
      dd[k] = (n >= 0 && n < g.NK - 1) ? Dc[n] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int n = nb - k;
      if (n >= 0) {
        C[(size_t)n * pr] = D;
        D = l[k] + dd[k] * D;
      }
    }
  }
  if (d_h0 != nullptr) {
    const int p0 = e / g.r, rc = e % g.r;
    d_h0[((size_t)bh * g.p + p0) * g.r + perm_rc(g, rc)] = to_t<T>(D);
  }
}

// k_fix: carry-cotangent terms for chunks n < NK-1 (D+ = Db[n] != 0):
//   v[p][(j,c)] = sum_col D+[p][col] bhat[j,c,col]   d_xhat += L[l-1,j] v
//   y[col][(j,c)] = sum_p D+[p][col] xhat[j,c,p]     d_bhat += L[l-1,j] y
//   d_da_s += <D+, h_-(n+1)> - sum_{j>=s} L[l-1,j] sum_c <xhat[j,c], v[:, (j,c)]>
template <typename T, int NT, int CK>
__global__ __launch_bounds__(NTH, 1) void k_fix(Geo g, int PK, const T* __restrict__ xhat,
                                                 const T* __restrict__ bhat,
                                                 const T* __restrict__ da,
                                                 const float* __restrict__ carry,
                                                 const float* __restrict__ Db, T* d_xhat,
                                                 T* d_bhat, T* d_da) {
  constexpr int R = 16 * NT, KS = MM<T>::KS, E = MM<T>::E, K = ELL * CK, RP = R + pad_of<T>();
  extern __shared__ __align__(16) unsigned char smem[];
  const Lds L = lds_fix(g, R, sizeof(T), PK);
  const int PP = g.PP;
  float* s_a = (float*)(smem + L.a);
  float* s_d = (float*)(smem + L.d);
  float* s_L = (float*)(smem + L.L);
  T* dp = (T*)(smem + L.lx);
  T* dpt = (T*)(smem + L.ltx);
  T* bn = (T*)(smem + L.bs);
  T* xn = (T*)(smem + L.xr);
  float* xv = (float*)(smem + L.red);
  float* red = xv + K;
  float* ddv = red + NTH;

  const int per = g.NK - 1;
  const int bh = blockIdx.x / per, n = blockIdx.x % per;
  const int bi = bh / g.h, hi = bh % g.h;
  g.V = chain_len(g, bi);  // this sequence's valid length (per-sequence lengths)
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;
  const int pr = g.p * g.r;
  const float* Dp = Db + ((size_t)bh * g.NK + n) * pr;
  const float* Hn = carry + ((size_t)bh * g.NK + n + 1) * pr;

  stage_decay(g, da, bi, hi, n, s_a, s_d, s_L);
  for (int idx = threadIdx.x; idx < PK * R; idx += NTH) {
    const int pp = idx / R, rc = idx % R;
    const float v = (pp < g.p && rc < g.r) ? Dp[pp * g.r + rc] : 0.0f;
    dp[pp * RP + rc] = to_t<T>(v);
    dpt[rc * PP + pp] = to_t<T>(v);
  }
  for (int idx = threadIdx.x; idx < K * R; idx += NTH) {
    const int k = idx / R, rc = idx % R;
    const int j = k / CK, ci = k % CK;
    const int pos = n * ELL + j;
    float v = 0.0f;
    if (rc < g.r && ci < g.c) v = to_f(bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + perm_rc(g, rc)]);
    bn[k * RP + rc] = to_t<T>(v);
  }
  for (int idx = threadIdx.x; idx < K * PK; idx += NTH) {
    const int k = idx / PK, pp = idx % PK;
    const int j = k / CK, ci = k % CK;
    const int pos = n * ELL + j;
    float v = 0.0f;
    if (pp < g.p && ci < g.c) v = to_f(xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pp]);
    xn[k * PP + pp] = to_t<T>(v);
  }
  float hd = 0.0f;
  for (int e = threadIdx.x; e < pr; e += NTH) hd += Dp[e] * Hn[e];
  red[threadIdx.x] = hd;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.0f;
    for (int i = 0; i < NTH; i++) s += red[i];
    red[0] = s;
  }
  __syncthreads();
  hd = red[0];
  const float* ll = s_L + (ELL - 1) * (ELL + 1);
  constexpr int NTK = K / 16;
  // v = D+ bhat^T: rows p (PK), cols (j,c), K over state columns
  for (int nt = w; nt < NTK; nt += NW) {
    const int k = 16 * nt + m;
    const int j = k / CK, ci = k % CK;
    const int pos = n * ELL + j;
    const float lj = ll[j];
    float xsum = 0.0f;
    for (int mt = 0; mt < PK / 16; mt++) {
      f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int ks = 0; ks < R / KS; ks++) {
        const int k0 = ks * KS + E * q;
        acc = MM<T>::mma(ld_frag(dp + (16 * mt + m) * RP + k0), ld_frag(bn + (16 * nt + m) * RP + k0), acc);
      }
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int pp = 16 * mt + 4 * q + i;
        if (pp < g.p && ci < g.c) {
          xsum += to_f(xn[k * PP + pp]) * acc[i];
          if (d_xhat != nullptr) {
            T* dst = d_xhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pp;
            *dst = to_t<T>(to_f(*dst) + lj * acc[i]);
          }
        }
      }
    }
    xsum = col4_sum(xsum);
    if (q == 0) xv[k] = xsum;
  }
  // y = D+^T xhat^T: rows state columns (R), cols (j,c), K over p
  if (d_bhat != nullptr) {
    for (int nt = w; nt < NTK; nt += NW) {
      const int k = 16 * nt + m;
      const int j = k / CK, ci = k % CK;
      const int pos = n * ELL + j;
      const float lj = ll[j];
      for (int mt = 0; mt < NT; mt++) {
        f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int ks = 0; ks < PK / KS; ks++) {
          const int k0 = ks * KS + E * q;
          acc = MM<T>::mma(ld_frag(dpt + (16 * mt + m) * PP + k0), ld_frag(xn + (16 * nt + m) * PP + k0), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int rc = 16 * mt + 4 * q + i;
          if (rc < g.r && ci < g.c) {
            T* dst = d_bhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + perm_rc(g, rc);
            *dst = to_t<T>(to_f(*dst) + lj * acc[i]);
          }
        }
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float acc = 0.0f;
    for (int j = ELL - 1; j >= 0; j--) {
      float cj = 0.0f;
      for (int ci = 0; ci < g.c; ci++) cj += xv[j * CK + ci];
      acc += ll[j] * cj;
      ddv[j] = hd - acc;
    }
  }
  __syncthreads();
  if (threadIdx.x < ELL && d_da != nullptr) {
    const int pos = n * ELL + threadIdx.x;
    T* dst = d_da + ((size_t)bi * g.s + pos) * g.h + hi;
    *dst = to_t<T>(to_f(*dst) + ddv[threadIdx.x]);
  }
}

// ---------------------------------------------------------------------------
// Group fix-up of the transposed backward (k_bwdt walks each group of chunks
// backward with D = 0 entering at the group's end). For group g covering chunks
// [n0_g, n1_g), with D_in(n) the walk's value and Q_g(n) = prod_{k=n}^{n1_g-1}
// dec_k, the recurrence D(n) = local(n) + dec_n D(n+1) gives
//   D(n) = D_in(n) + Q_g(n) D_B(g),   D_B(g) = D(n1_g) = D(n0_{g+1}),
// so D_B(g) = D_in(n0_{g+1}) + Q_{g+1}(n0_{g+1}) D_B(g+1), D_B(last) = 0, and
// chunk n of group g still lacks the carry cotangent Q_g(n+1) D_B(g).
// ---------------------------------------------------------------------------

// k_gscan: DB[bh][g] = D_B(g) for g < NGR-1, and d_h0 = D(0).
template <typename T>
__global__ __launch_bounds__(NTH) void k_gscan(Geo g, const float* __restrict__ Db,
                                               const float* __restrict__ dec, float* DB, T* d_h0) {
  const int bh = blockIdx.x;
  const int e = blockIdx.y * NTH + threadIdx.x;
  const int pr = g.p * g.r;
  if (e >= pr) return;
  g.V = chain_len(g, bh / g.h);
  // groups holding walked chunks (the others enter nothing: their D_B is zero)
  const int nkc = chain_nk(g), ngc = (nkc + g.G - 1) / g.G;
  const float* Dc = dec + (size_t)bh * g.NK;
  auto qprod = [&](int gr) {  // Q over the whole group gr (its chunks are all < nkc-1 here)
    const int a = gr * g.G, b = (a + g.G < nkc) ? a + g.G : nkc;
    float qv = 1.0f;
    for (int k = a; k < b; k++) qv *= Dc[k];
    return qv;
  };
  float D = 0.0f;  // D_B(g + 1) while walking down
  for (int gr = g.NGR - 2; gr >= 0; gr--) {
    if (gr + 1 >= ngc) {
      DB[((size_t)bh * g.NGR + gr) * pr + e] = 0.0f;
      continue;
    }
    const int n0n = (gr + 1) * g.G;
    const float din = Db[((size_t)bh * g.NK + n0n) * pr + e];
    D = (gr + 1 < ngc - 1) ? din + qprod(gr + 1) * D : din;
    DB[((size_t)bh * g.NGR + gr) * pr + e] = D;
  }
  if (d_h0 != nullptr) {
    float d0 = nkc > 0 ? Db[(size_t)bh * g.NK * pr + e] : 0.0f;
    if (ngc > 1) d0 += qprod(0) * D;
    const int p0 = e / g.r, rc = e % g.r;
    d_h0[((size_t)bh * g.p + p0) * g.r + perm_rc(g, rc)] = to_t<T>(d0);
  }
}

// k_gfix: for group g < NGR-1 of chain bh, chunks n = n1_g-1 down to n0_g while
// the scale Q_g(n+1) is nonzero, add the carry-cotangent terms of
// D+ = Q_g(n+1) D_B(g), the cotangent of h~[l-1] = h_-(n+1):
//   v[p][(j,c)] = sum_col D+[p][col] bhat[j,c,col]   d_xhat += L[l-1,j] v
//   y[col][(j,c)] = sum_p D+[p][col] xhat[j,c,p]     d_bhat += L[l-1,j] y
//   d_da_s += d_{l-1} <D+, h_-(n)> + sum_{j<s} L[l-1,j] sum_c <xhat[j,c], v[:, (j,c)]>
// (d_da in its direct form, as in k_bwdt).
// Once Q underflows to zero every later term is exactly zero, so the walk stops.
// (Two workgroups per CU where LDS allows: the register budget that sets.)
template <typename T, int NT, int CK>
__global__ __launch_bounds__(NTH, 2) void k_gfix(Geo g, int PK, const T* __restrict__ xhat,
                                                  const T* __restrict__ bhat, const T* __restrict__ da,
                                                  const float* __restrict__ carry, const float* __restrict__ dec,
                                                  const float* __restrict__ DB, T* d_xhat, T* d_bhat, T* d_da) {
  constexpr int R = 16 * NT, KS = MM<T>::KS, E = MM<T>::E, K = ELL * CK, RP = R + pad_of<T>();
  extern __shared__ __align__(16) unsigned char smem[];
  const Lds L = lds_fix(g, R, sizeof(T), PK);
  const int PP = g.PP;
  float* s_a = (float*)(smem + L.a);
  float* s_d = (float*)(smem + L.d);
  float* s_L = (float*)(smem + L.L);
  T* dp = (T*)(smem + L.lx);
  T* dpt = (T*)(smem + L.ltx);
  T* bn = (T*)(smem + L.bs);
  T* xn = (T*)(smem + L.xr);
  float* xv = (float*)(smem + L.red);
  float* red = xv + K;
  float* ddv = red + NTH;

  const int ng = g.NGR - 1;
  const int bh = blockIdx.x / ng, grp = blockIdx.x % ng;
  const int bi = bh / g.h, hi = bh % g.h;
  g.V = chain_len(g, bi);  // this sequence's valid length (per-sequence lengths)
  // nothing enters a group whose successor holds no walked chunk
  if (grp + 1 >= (chain_nk(g) + g.G - 1) / g.G) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;
  const int pr = g.p * g.r;
  const float* Dp = DB + ((size_t)bh * g.NGR + grp) * pr;
  for (int idx = threadIdx.x; idx < PK * R; idx += NTH) {
    const int pp = idx / R, rc = idx % R;
    const float v = (pp < g.p && rc < g.r) ? Dp[pp * g.r + rc] : 0.0f;
    dp[pp * RP + rc] = to_t<T>(v);
    dpt[rc * PP + pp] = to_t<T>(v);
  }
  const int n0 = grp * g.G;
  const int n1 = (n0 + g.G < g.NK) ? n0 + g.G : g.NK;
  // bf16 rows of whole 16-byte pieces are staged with 16-byte loads, all issued
  // before the first LDS store
  constexpr bool WIDE_T = std::is_same<T, bf16>::value;
  const bool wide = WIDE_T && g.r % 8 == 0 && g.p % 8 == 0;
  float Q = 1.0f;
  for (int n = n1 - 1; n >= n0 && Q != 0.0f; n--) {
    __syncthreads();
    stage_decay(g, da, bi, hi, n, s_a, s_d, s_L);
    if constexpr (WIDE_T) {
      if (wide) {
        // items (k, piece of 8): bhat rows K x R/8, then xhat rows K x PK/8
        constexpr int NBU = K * R / 8, NBL = (NBU + NTH - 1) / NTH;
        u4 bv[NBL];
#pragma unroll
        for (int i = 0; i < NBL; i++) {
          const int idx = threadIdx.x + i * NTH;
          const int k = idx / (R / 8), c8 = idx % (R / 8);
          const int j = k / CK, ci = k % CK, pos = n * ELL + j;
          bv[i] = u4{0u, 0u, 0u, 0u};
          if (idx < NBU && 8 * c8 < g.r && ci < g.c)
            bv[i] = *reinterpret_cast<const u4*>(bhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + 8 * c8);
        }
        const int NXU = K * PK / 8;
        for (int idx0 = 0; idx0 < NXU; idx0 += 4 * NTH) {
          u4 xv[4];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int idx = idx0 + threadIdx.x + i * NTH;
            const int k = idx / (PK / 8), p8 = idx % (PK / 8);
            const int j = k / CK, ci = k % CK, pos = n * ELL + j;
            xv[i] = u4{0u, 0u, 0u, 0u};
            if (idx < NXU && 8 * p8 < g.p && ci < g.c)
              xv[i] = *reinterpret_cast<const u4*>(xhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + 8 * p8);
          }
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int idx = idx0 + threadIdx.x + i * NTH;
            if (idx < NXU) {
              const int k = idx / (PK / 8), p8 = idx % (PK / 8);
              *reinterpret_cast<u4*>(xn + k * PP + 8 * p8) = xv[i];
            }
          }
        }
#pragma unroll
        for (int i = 0; i < NBL; i++) {
          const int idx = threadIdx.x + i * NTH;
          if (idx >= NBU) continue;
          const int k = idx / (R / 8), c8 = idx % (R / 8);
          const T* v = reinterpret_cast<const T*>(&bv[i]);
          // caller columns 8c8.. sit at internal columns inv_perm_rc(..) < r;
          // internal columns >= r are zero
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const int cc = 8 * c8 + e;
            bn[k * RP + (cc < g.r ? inv_perm_rc(g, cc) : cc)] = v[e];
          }
        }
      }
    }
    // staging and the <D_B, h_-(n)> sum issue their global loads in batches of
    // eight per thread (one wait per batch rather than one per element)
#pragma unroll 8
    for (int idx = threadIdx.x; idx < K * R && !wide; idx += NTH) {
      const int k = idx / R, rc = idx % R;
      const int j = k / CK, ci = k % CK;
      const int pos = n * ELL + j;
      float v = 0.0f;
      if (rc < g.r && ci < g.c) v = to_f(bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + perm_rc(g, rc)]);
      bn[k * RP + rc] = to_t<T>(v);
    }
#pragma unroll 8
    for (int idx = threadIdx.x; idx < K * PK && !wide; idx += NTH) {
      const int k = idx / PK, pp = idx % PK;
      const int j = k / CK, ci = k % CK;
      const int pos = n * ELL + j;
      float v = 0.0f;
      if (pp < g.p && ci < g.c) v = to_f(xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pp]);
      xn[k * PP + pp] = to_t<T>(v);
    }
    const float* Hn = carry + ((size_t)bh * g.NK + n) * pr;  // h_-(n), entering the chunk
    float hd = 0.0f;
    {
      // elements e = tid + i NTH, in blocks of eight (h8[k] takes element k of
      // each block) while a whole block is below pr, the rest into h8[0]; the
      // loads of two blocks are issued together
      float h8[8];
#pragma unroll
      for (int k = 0; k < 8; k++) h8[k] = 0.0f;
      int e = threadIdx.x;
      for (; e + 15 * NTH < pr; e += 16 * NTH) {
        float dv[16], hv[16];
#pragma unroll
        for (int k = 0; k < 16; k++) {
          dv[k] = Dp[e + k * NTH];
          hv[k] = Hn[e + k * NTH];
        }
#pragma unroll
        for (int k = 0; k < 16; k++) h8[k & 7] += dv[k] * hv[k];
      }
      for (; e + 7 * NTH < pr; e += 8 * NTH) {
#pragma unroll
        for (int k = 0; k < 8; k++) h8[k] += Dp[e + k * NTH] * Hn[e + k * NTH];
      }
      for (; e < pr; e += NTH) h8[0] += Dp[e] * Hn[e];
      hd = ((h8[0] + h8[1]) + (h8[2] + h8[3])) + ((h8[4] + h8[5]) + (h8[6] + h8[7]));
    }
    // fixed-order sum over the workgroup: within each wave, then over the waves
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) hd += __shfl_xor(hd, off, 64);
    if (lane == 0) red[w] = hd;
    __syncthreads();
    if (threadIdx.x == 0) {
      float s = 0.0f;
      for (int i = 0; i < NW; i++) s += red[i];
      red[0] = s;
    }
    __syncthreads();
    hd = Q * s_d[ELL - 1] * red[0];
    const float* ll = s_L + (ELL - 1) * (ELL + 1);
    constexpr int NTK = K / 16;
    for (int nt = w; nt < NTK; nt += NW) {
      const int k = 16 * nt + m;
      const int j = k / CK, ci = k % CK;
      const int pos = n * ELL + j;
      const float lj = Q * ll[j];
      float xsum = 0.0f;
      // row tiles in batches of four: the d_xhat loads of a batch are issued
      // together, then its stores
      constexpr int MB = 4;
      const int MT = PK / 16;
      for (int mt0 = 0; mt0 < MT; mt0 += MB) {
        f4 acc[MB];
#pragma unroll
        for (int u = 0; u < MB; u++) {
          acc[u] = f4{0.0f, 0.0f, 0.0f, 0.0f};
          if (mt0 + u < MT) {
            for (int ks = 0; ks < R / KS; ks++) {
              const int k0 = ks * KS + E * q;
              acc[u] = MM<T>::mma(ld_frag(dp + (16 * (mt0 + u) + m) * RP + k0), ld_frag(bn + (16 * nt + m) * RP + k0),
                                  acc[u]);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < MB; u++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int pp = 16 * (mt0 + u) + 4 * q + i;
            if (mt0 + u < MT && pp < g.p && ci < g.c) xsum += to_f(xn[k * PP + pp]) * acc[u][i];
          }
        if (d_xhat != nullptr && ci < g.c) {
          T* xrow = d_xhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p;
          T old[MB][4];
#pragma unroll
          for (int u = 0; u < MB; u++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int pp = 16 * (mt0 + u) + 4 * q + i;
              old[u][i] = mt0 + u < MT && pp < g.p ? xrow[pp] : to_t<T>(0.0f);
            }
#pragma unroll
          for (int u = 0; u < MB; u++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int pp = 16 * (mt0 + u) + 4 * q + i;
              if (mt0 + u < MT && pp < g.p) xrow[pp] = to_t<T>(to_f(old[u][i]) + lj * acc[u][i]);
            }
        }
      }
      xsum = col4_sum(xsum);
      if (q == 0) xv[k] = Q * xsum;
    }
    if (d_bhat != nullptr) {
      for (int nt = w; nt < NTK; nt += NW) {
        const int k = 16 * nt + m;
        const int j = k / CK, ci = k % CK;
        const int pos = n * ELL + j;
        const float lj = Q * ll[j];
        // column tiles in batches of four: the d_bhat loads of a batch are
        // issued together, then its stores
        constexpr int CB = NT < 4 ? NT : 4;
#pragma unroll
        for (int mt0 = 0; mt0 < NT; mt0 += CB) {
          f4 acc[CB];
#pragma unroll
          for (int u = 0; u < CB; u++) {
            acc[u] = f4{0.0f, 0.0f, 0.0f, 0.0f};
            for (int ks = 0; ks < PK / KS; ks++) {
              const int k0 = ks * KS + E * q;
              acc[u] = MM<T>::mma(ld_frag(dpt + (16 * (mt0 + u) + m) * PP + k0), ld_frag(xn + (16 * nt + m) * PP + k0),
                                  acc[u]);
            }
          }
          if (ci < g.c) {
            T* brow = d_bhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r;
            T old[CB][4];
#pragma unroll
            for (int u = 0; u < CB; u++)
#pragma unroll
              for (int i = 0; i < 4; i++) {
                const int rc = 16 * (mt0 + u) + 4 * q + i;
                old[u][i] = rc < g.r ? brow[perm_rc(g, rc)] : to_t<T>(0.0f);
              }
#pragma unroll
            for (int u = 0; u < CB; u++)
#pragma unroll
              for (int i = 0; i < 4; i++) {
                const int rc = 16 * (mt0 + u) + 4 * q + i;
                if (rc < g.r) brow[perm_rc(g, rc)] = to_t<T>(to_f(old[u][i]) + lj * acc[u][i]);
              }
          }
        }
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float acc = 0.0f;
      for (int j = 0; j < ELL; j++) {
        ddv[j] = hd + acc;
        float cj = 0.0f;
        for (int ci = 0; ci < g.c; ci++) cj += xv[j * CK + ci];
        acc += ll[j] * cj;
      }
    }
    __syncthreads();
    if (threadIdx.x < ELL && d_da != nullptr) {
      const int pos = n * ELL + threadIdx.x;
      T* dst = d_da + ((size_t)bi * g.s + pos) * g.h + hi;
      *dst = to_t<T>(to_f(*dst) + ddv[threadIdx.x]);
    }
    Q *= dec[(size_t)bh * g.NK + n];
  }
}

// Zeros for every gradient at positions [z0, s) (chunks never processed); with
// `skip`, from each sequence's first unwalked chunk (grid y = sequence).
template <typename T>
__global__ __launch_bounds__(NTH) void k_zero_tail(Geo g, int z0, T* d_xhat, T* d_bhat, T* d_da,
                                                   T* d_rot) {
  const size_t stride = (size_t)gridDim.x * NTH;
  const size_t start = (size_t)blockIdx.x * NTH + threadIdx.x;
  const T zero = to_t<T>(0.0f);
  const int V0 = g.V;
  // without skip one pass covers every sequence from z0; with it, sequence by sequence
  for (int bfirst = g.skip ? (int)blockIdx.y : 0; bfirst < g.b; bfirst += g.skip ? (int)gridDim.y : g.b) {
    const int bend = g.skip ? bfirst + 1 : g.b;
    if (g.skip) {
      g.V = V0;
      g.V = chain_len(g, bfirst);
      z0 = chain_nk(g) * ELL;
    }
    const size_t npos = (size_t)(g.s > z0 ? g.s - z0 : 0);
    auto fill = [&](T* ptr, size_t per_pos) {
      if (ptr == nullptr) return;
      const size_t total = (size_t)(bend - bfirst) * npos * per_pos;
      for (size_t i = start; i < total; i += stride) {
        const size_t bi = bfirst + i / (npos * per_pos), rest = i % (npos * per_pos);
        ptr[((size_t)bi * g.s + z0) * per_pos + rest] = zero;
      }
    };
    fill(d_xhat, (size_t)g.c * g.h * g.p);
    fill(d_bhat, (size_t)g.c * g.h * g.r);
    fill(d_da, (size_t)g.h);
    fill(d_rot, (size_t)g.h * g.RW);
  }
}

// ---- backward over token pairs (bf16, four channels) -------------------------
// A chain of s tokens with four channels is walked as 2s tokens of two channels
// each: token t becomes pair tokens 2t (channels 0, 1) and 2t+1 (channels 2, 3).
// With da 0 at 2t+1 and da_t at 2t, the state after 2t+1 is the state after t
// (h~[t] = exp(da_t) h~[t-1] + sum over the four channels), and the xhat, bhat,
// d_xhat and d_bhat tensors already have the pair layout ([b,s,4,h,.] is
// [b,2s,2,h,.] in memory). Only odd pair tokens carry moments, so the backward
// masks d_c at even ones (Geo::pair). These kernels build the pair-token da and
// rot (and doubled per-sequence lengths) and take d_da (at 2t) and d_rot (at
// 2t+1) back.
// Rows of `unit`-sized pieces: U is uint4 when a token row of rot is a multiple
// of 16 bytes, else the element type.
template <typename T, typename U>
__global__ __launch_bounds__(NTH) void k_pair_prep(Geo g, const T* __restrict__ da, const U* __restrict__ rot,
                                                   int rot_units, T* __restrict__ da2, U* __restrict__ rot2,
                                                   int* __restrict__ lens2) {
  const size_t stride = (size_t)gridDim.x * NTH;
  const size_t start = (size_t)blockIdx.x * NTH + threadIdx.x;
  const size_t nda = (size_t)g.b * g.s * g.h;
  for (size_t i = start; i < nda; i += stride) {
    const size_t bt = i / g.h, hi = i % g.h;  // bt = bi * s + t
    const size_t bi = bt / g.s, t = bt % g.s;
    const size_t o = ((bi * 2 * g.s + 2 * t) * g.h + hi);
    da2[o] = da[i];
    da2[o + g.h] = to_t<T>(0.0f);
  }
  if (rot != nullptr) {
    const size_t nrot = (size_t)g.b * g.s * rot_units;
    for (size_t i = start; i < nrot; i += stride) {
      const size_t bt = i / rot_units, k = i % rot_units;
      const U v = rot[i];
      rot2[(2 * bt) * rot_units + k] = v;
      rot2[(2 * bt + 1) * rot_units + k] = v;
    }
  }
  if (lens2 != nullptr && start < (size_t)g.b) lens2[start] = 2 * chain_len(g, (int)start);
}

template <typename T, typename U>
__global__ __launch_bounds__(NTH) void k_pair_post(Geo g, const T* __restrict__ dda2, const U* __restrict__ drot2,
                                                   int rot_units, T* __restrict__ d_da, U* __restrict__ d_rot) {
  const size_t stride = (size_t)gridDim.x * NTH;
  const size_t start = (size_t)blockIdx.x * NTH + threadIdx.x;
  if (d_da != nullptr) {
    const size_t nda = (size_t)g.b * g.s * g.h;
    for (size_t i = start; i < nda; i += stride) {
      const size_t bt = i / g.h, hi = i % g.h;
      d_da[i] = dda2[(2 * bt) * g.h + hi];
    }
  }
  if (d_rot != nullptr) {
    const size_t nrot = (size_t)g.b * g.s * rot_units;
    for (size_t i = start; i < nrot; i += stride) {
      const size_t bt = i / rot_units, k = i % rot_units;
      d_rot[i] = drot2[(2 * bt + 1) * rot_units + k];
    }
  }
}

// Debug finiteness check of an output (enabled by MOMENTS_CHECK_FINITE): any
// non-finite element sets flag[0] to 1 (every writer writes the same value).
__global__ __launch_bounds__(NTH) void k_flag_clear(int* flag) {
  if (blockIdx.x == 0 && threadIdx.x == 0) flag[0] = 0;
}
template <typename T>
__global__ __launch_bounds__(NTH) void k_check_finite(const T* __restrict__ x, size_t n, int* flag) {
  const size_t stride = (size_t)gridDim.x * NTH;
  bool bad = false;
  for (size_t i = (size_t)blockIdx.x * NTH + threadIdx.x; i < n; i += stride) bad |= !__builtin_isfinite(to_f(x[i]));
  if (bad) flag[0] = 1;
}

}  // namespace mom

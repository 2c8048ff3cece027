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

#include "kernels.h"

namespace mom {

template <typename T, int NT>
__global__ __launch_bounds__(NTH, 1) void k_bwd(
    Geo g, const T* __restrict__ xhat, const T* __restrict__ bhat, const T* __restrict__ da,
    const T* __restrict__ rot, const float* __restrict__ carry, const float* __restrict__ dm2,
    const float* __restrict__ dm1, float* Db, T* d_xhat, T* d_bhat, T* d_da, T* d_rot) {
  constexpr int R = 16 * NT, KS = MM<T>::KS, E = MM<T>::E, NKT = ELL / KS;
  extern __shared__ __align__(16) unsigned char smem[];
  const Lds L = lds_bwd(g, R, sizeof(T), NT);
  float* s_a = (float*)(smem + L.a);
  float* s_d = (float*)(smem + L.d);
  float* s_L = (float*)(smem + L.L);
  float* lx = (float*)(smem + L.lx);
  T* bs = (T*)(smem + L.bs);
  T* ltp = (T*)(smem + L.ltp);
  T* ltx = (T*)(smem + L.ltx);
  float* cs = (float*)(smem + L.rot);
  float* sn = cs + ELL * g.A;
  float* qv = cs;
  T* xr = (T*)(smem + L.xr);
  T* S = (T*)(smem + L.S);
  unsigned char* xg = smem + L.xg;
  float* rsum = (float*)(smem + L.red);
  float* csum = rsum + NW * ELL;
  float* ddv = csum + NW * ELL;

  const int bh = blockIdx.x / g.NGR, gi = blockIdx.x % g.NGR;
  const int bi = bh / g.h, hi = bh % g.h;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;
  const int nrounds = (g.p + 3) / 4;
  const bool cplx = g.rot_kind == 1 || g.rot_kind == 2;

  // S = d_m2 + d_m2^T in internal column order (symmetric, so it serves as the
  // K-contiguous B operand of d_c = c S).
  for (int idx = threadIdx.x; idx < R * R; idx += NTH) {
    const int a = idx / R, b = idx % R;
    float v = 0.0f;
    if (a < g.r && b < g.r) {
      const int pa = perm_rc(g, a), pb = perm_rc(g, b);
      const float* D2 = dm2 + (size_t)bh * g.r * g.r;
      v = D2[pa * g.r + pb] + D2[pb * g.r + pa];
    }
    S[a * g.RP + b] = to_t<T>(v);
  }

  const int n0 = gi * g.G;
  const int n1 = (n0 + g.G < g.NK) ? n0 + g.G : g.NK;
  for (int n = n0; n < n1; n++) {
    __syncthreads();
    stage_decay(g, da, bi, hi, n, s_a, s_d, s_L);
    stage_bhat<T, R>(g, bhat, bi, hi, n, bs);
    stage_rot(g, rot, bi, hi, n, cs, sn, qv);
    __syncthreads();
    stage_lx(g, s_L, lx);
    stage_lt<T>(g, s_L, ltp, ltx);

    f4 racc[2][NT], dbacc[2][NT];
    f4 gacc[2], cacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      gacc[mt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
      cacc[mt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        racc[mt][nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        dbacc[mt][nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }

    for (int round = 0; round < nrounds; round++) {
      stage_xround(g, xhat, bi, hi, n, round, xr);
      __syncthreads();
      const int p0 = 4 * round + w;
      const bool valid = p0 < g.p;
      const float* hrow = valid ? carry + (((size_t)bh * g.NK + n) * g.p + p0) * g.r : nullptr;
      T* X = (T*)(xg + (size_t)w * L.xgw);

      // states h~ and c
      f4 keep[2][NT];
      chunk_states_row<T, NT>(keep, g, n, s_d, lx, bs, xr + w * g.KP, hrow);
      f4 dc[2][NT];
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++) dc[mt][nt] = keep[mt][nt];
      rotate_tiles<false, NT>(dc, g, cs, sn, qv);  // dc holds c for now
      if (cplx) {
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int nt = 0; nt < NT; nt++) keep[mt][nt] = dc[mt][nt];
      }
      // c -> LDS rows [t][col] for the A operand of d_c (K over columns)
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
#pragma unroll
          for (int i = 0; i < 4; i++) X[(16 * mt + 4 * q + i) * g.RP + 16 * nt + m] = to_t<T>(dc[mt][nt][i]);
      wave_lds_sync();
      // d_c = c S + d_m1, masked
#pragma unroll
      for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++) dc[mt][nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int ks = 0; ks < R / KS; ks++) {
        const int k0 = ks * KS + E * q;
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
          const auto a = ld_frag(X + (16 * mt + m) * g.RP + k0);
#pragma unroll
          for (int nt = 0; nt < NT; nt++)
            dc[mt][nt] = MM<T>::mma(a, ld_frag(S + (16 * nt + m) * g.RP + k0), dc[mt][nt]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        const int col = 16 * nt + m;
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
      accum_drot<NT>(racc, dc, keep, g);
      if (g.rot_kind != 3) {
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int nt = 0; nt < NT; nt++)
#pragma unroll
            for (int i = 0; i < 4; i++) gacc[mt][i] += dc[mt][nt][i] * keep[mt][nt][i];
      }
      rotate_tiles<true, NT>(dc, g, cs, sn, qv);  // dc now holds G
      if (g.rot_kind == 3) {
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int nt = 0; nt < NT; nt++)
#pragma unroll
            for (int i = 0; i < 4; i++) gacc[mt][i] += dc[mt][nt][i] * keep[mt][nt][i];
      }
      // local(n)[p0][col] = sum_t d_t G[t][col]
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        float sum = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++) sum += s_d[16 * mt + 4 * q + i] * dc[mt][nt][i];
        sum = col4_sum(sum);
        const int col = 16 * nt + m;
        if (q == 0 && valid && col < g.r) Db[(((size_t)bh * g.NK + n) * g.p + p0) * g.r + col] = sum;
      }
      // d_W[j][col] = sum_t L[t][j] G[t][col] (K over tokens, B from registers)
      f4 dw[2][NT];
#pragma unroll
      for (int jt = 0; jt < 2; jt++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++) dw[jt][nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < NKT; ks++) {
#pragma unroll
        for (int jt = 0; jt < 2; jt++) {
          const auto a = ld_frag(ltp + (16 * jt + m) * SLOTP + ks * KS + E * q);
#pragma unroll
          for (int nt = 0; nt < NT; nt++) {
            const f4 gv[2] = {dc[0][nt], dc[1][nt]};
            dw[jt][nt] = MM<T>::mma(a, pack_tslots(gv, ks, T{}), dw[jt][nt]);
          }
        }
      }
      // G as B fragments (K over tokens) for d_bhat, in this wave's exchange slot
      wave_lds_sync();
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        const f4 gv[2] = {dc[0][nt], dc[1][nt]};
        if constexpr (E == 1) {
#pragma unroll
          for (int ks = 0; ks < NKT; ks++) ((float*)X)[(nt * NKT + ks) * 64 + lane] = pack_tslots(gv, ks, T{});
        } else {
          ((bf8*)X)[nt * 64 + lane] = pack_tslots(gv, 0, T{});
        }
      }
      // d_xhat[j,c,p0] = sum_col d_W[j][col] bhat[j,c,col]; col term <xhat, d_xhat>
#pragma unroll
      for (int jt = 0; jt < 2; jt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int j = 16 * jt + 4 * q + i;
          const int pos = n * ELL + j;
          for (int ci = 0; ci < g.c; ci++) {
            const int k = j * g.c + ci;
            float part = 0.0f;
#pragma unroll
            for (int nt = 0; nt < NT; nt++) part += dw[jt][nt][i] * to_f(bs[(16 * nt + m) * g.KP + k]);
            const float val = row16_sum(part);
            cacc[jt][i] += val * to_f(xr[w * g.KP + k]);
            if (d_xhat != nullptr && valid && m == ((i * g.c + ci) & 15) && pos < g.s)
              d_xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + p0] = to_t<T>(val);
          }
        }
      __syncthreads();
      // d_bhat[(j,c)][col] += sum over (t, this round's rows) L[t,j] xhat[j,c,p] G[t][col]
#pragma unroll
      for (int mi = 0; mi < 2; mi++) {
        const int mtb = w + 4 * mi;
        if (16 * mtb < g.K) {
          const int k = 16 * mtb + m;
          for (int ww = 0; ww < NW; ww++) {
            const float xs = to_f(xr[ww * g.KP + k]);
            const unsigned char* gb = xg + (size_t)ww * L.xgw;
#pragma unroll
            for (int ks = 0; ks < NKT; ks++) {
              typename MM<T>::frag a;
              const T* lt = ltx + k * SLOTP + ks * KS + E * q;
              if constexpr (E == 1) {
                a = lt[0] * xs;
              } else {
#pragma unroll
                for (int e = 0; e < E; e++) a[e] = to_t<T>(to_f(lt[e]) * xs);
              }
#pragma unroll
              for (int nt = 0; nt < NT; nt++) {
                typename MM<T>::frag b;
                if constexpr (E == 1) b = ((const float*)gb)[(nt * NKT + ks) * 64 + lane];
                else b = ((const bf8*)gb)[nt * 64 + lane];
                dbacc[mi][nt] = MM<T>::mma(a, b, dbacc[mi][nt]);
              }
            }
          }
        }
      }
      __syncthreads();
    }

    // ---- chunk end: d_bhat --------------------------------------------------
#pragma unroll
    for (int mi = 0; mi < 2; mi++) {
      const int mtb = w + 4 * mi;
      if (16 * mtb < g.K && d_bhat != nullptr) {
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
          const int col = 16 * nt + m;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int k = 16 * mtb + 4 * q + i;
            const int j = k / g.c, ci = k - j * g.c;
            const int pos = n * ELL + j;
            if (k < g.K && col < g.r && pos < g.s)
              d_bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + perm_rc(g, col)] =
                  to_t<T>(dbacc[mi][nt][i]);
          }
        }
      }
    }
    // ---- rotation gradient: fixed-order sum over the four waves --------------
    if (g.rot_kind != 0 && d_rot != nullptr) {
      float* RB = (float*)xg;
      const int rwi = cplx ? g.A : 4 * g.J;
      for (int ww = 0; ww < NW; ww++) {
        if (w == ww) {
#pragma unroll
          for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
              const int col = 16 * nt + m;
              int idx = -1;
              if (cplx) {
                if ((col & 1) == 0 && (col >> 1) < g.A) idx = col >> 1;
              } else if (col < 4 * g.J) {
                idx = col;
              }
              if (idx >= 0) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                  float* dst = RB + (16 * mt + 4 * q + i) * rwi + idx;
                  *dst = (ww == 0 ? 0.0f : *dst) + racc[mt][nt][i];
                }
              }
            }
        }
        __syncthreads();
      }
      for (int idx = threadIdx.x; idx < ELL * rwi; idx += NTH) {
        const int t = idx / rwi, e = idx % rwi;
        const int pos = n * ELL + t;
        if (pos < g.s) d_rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + e] = to_t<T>(RB[idx]);
      }
    }
    // ---- d_da (without the carry-cotangent terms) ---------------------------
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float gs = row16_sum(gacc[mt][i]);
        if (m == 0) {
          rsum[w * ELL + 16 * mt + 4 * q + i] = gs;
          csum[w * ELL + 16 * mt + 4 * q + i] = cacc[mt][i];
        }
      }
    __syncthreads();
    if (threadIdx.x == 0) {
      float acc = 0.0f;
      for (int t = ELL - 1; t >= 0; t--) {
        float rt = 0.0f, ct = 0.0f;
        for (int ww = 0; ww < NW; ww++) {
          rt += rsum[ww * ELL + t];
          ct += csum[ww * ELL + t];
        }
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
template <typename T, int NT>
__global__ __launch_bounds__(NTH, 1) void k_fix(Geo g, int PK, const T* __restrict__ xhat,
                                                 const T* __restrict__ bhat,
                                                 const T* __restrict__ da,
                                                 const float* __restrict__ carry,
                                                 const float* __restrict__ Db, T* d_xhat,
                                                 T* d_bhat, T* d_da) {
  constexpr int R = 16 * NT, KS = MM<T>::KS, E = MM<T>::E;
  extern __shared__ __align__(16) unsigned char smem[];
  const Lds L = lds_fix(g, R, sizeof(T), PK);
  float* s_a = (float*)(smem + L.a);
  float* s_d = (float*)(smem + L.d);
  float* s_L = (float*)(smem + L.L);
  T* dp = (T*)(smem + L.lx);
  T* dpt = (T*)(smem + L.ltx);
  T* bn = (T*)(smem + L.bs);
  T* xn = (T*)(smem + L.xr);
  float* xv = (float*)(smem + L.red);
  float* red = xv + g.K;
  float* ddv = red + NTH;

  const int per = g.NK - 1;
  const int bh = blockIdx.x / per, n = blockIdx.x % per;
  const int bi = bh / g.h, hi = bh % g.h;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;
  const int pr = g.p * g.r;
  const float* Dp = Db + ((size_t)bh * g.NK + n) * pr;
  const float* Hn = carry + ((size_t)bh * g.NK + n + 1) * pr;

  stage_decay(g, da, bi, hi, n, s_a, s_d, s_L);
  for (int idx = threadIdx.x; idx < PK * R; idx += NTH) {
    const int pp = idx / R, rc = idx % R;
    const float v = (pp < g.p && rc < g.r) ? Dp[pp * g.r + rc] : 0.0f;
    dp[pp * g.RP + rc] = to_t<T>(v);
    dpt[rc * g.PP + pp] = to_t<T>(v);
  }
  for (int idx = threadIdx.x; idx < g.K * R; idx += NTH) {
    const int k = idx / R, rc = idx % R;
    const int j = k / g.c, ci = k - j * g.c;
    const int pos = n * ELL + j;
    float v = 0.0f;
    if (rc < g.r) v = to_f(bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + perm_rc(g, rc)]);
    bn[k * g.RP + rc] = to_t<T>(v);
  }
  for (int idx = threadIdx.x; idx < g.K * PK; idx += NTH) {
    const int k = idx / PK, pp = idx % PK;
    const int j = k / g.c, ci = k - j * g.c;
    const int pos = n * ELL + j;
    float v = 0.0f;
    if (pp < g.p) v = to_f(xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pp]);
    xn[k * g.PP + pp] = to_t<T>(v);
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
  const int NTK = g.K / 16;
  // v = D+ bhat^T: rows p (PK), cols (j,c), K over state columns
  for (int nt = w; nt < NTK; nt += NW) {
    const int k = 16 * nt + m;
    const int j = k / g.c, ci = k - j * g.c;
    const int pos = n * ELL + j;
    const float lj = ll[j];
    float xsum = 0.0f;
    for (int mt = 0; mt < PK / 16; mt++) {
      f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int ks = 0; ks < R / KS; ks++) {
        const int k0 = ks * KS + E * q;
        acc = MM<T>::mma(ld_frag(dp + (16 * mt + m) * g.RP + k0), ld_frag(bn + (16 * nt + m) * g.RP + k0), acc);
      }
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int pp = 16 * mt + 4 * q + i;
        if (pp < g.p) {
          xsum += to_f(xn[k * g.PP + pp]) * acc[i];
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
      const int j = k / g.c, ci = k - j * g.c;
      const int pos = n * ELL + j;
      const float lj = ll[j];
      for (int mt = 0; mt < NT; mt++) {
        f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int ks = 0; ks < PK / KS; ks++) {
          const int k0 = ks * KS + E * q;
          acc = MM<T>::mma(ld_frag(dpt + (16 * mt + m) * g.PP + k0), ld_frag(xn + (16 * nt + m) * g.PP + k0), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int rc = 16 * mt + 4 * q + i;
          if (rc < g.r) {
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
      for (int ci = 0; ci < g.c; ci++) cj += xv[j * g.c + ci];
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

// Zeros for every gradient at positions [z0, s) (chunks never processed).
template <typename T>
__global__ __launch_bounds__(NTH) void k_zero_tail(Geo g, int z0, T* d_xhat, T* d_bhat, T* d_da,
                                                   T* d_rot) {
  const size_t npos = (size_t)(g.s - z0);
  const size_t stride = (size_t)gridDim.x * NTH;
  const size_t start = (size_t)blockIdx.x * NTH + threadIdx.x;
  const T zero = to_t<T>(0.0f);
  auto fill = [&](T* ptr, size_t per_pos) {
    if (ptr == nullptr) return;
    const size_t total = (size_t)g.b * npos * per_pos;
    for (size_t i = start; i < total; i += stride) {
      const size_t bi = i / (npos * per_pos), rest = i % (npos * per_pos);
      ptr[((size_t)bi * g.s + z0) * per_pos + rest] = zero;
    }
  };
  fill(d_xhat, (size_t)g.c * g.h * g.p);
  fill(d_bhat, (size_t)g.c * g.h * g.r);
  fill(d_da, (size_t)g.h);
  fill(d_rot, (size_t)g.h * g.RW);
}

}  // namespace mom

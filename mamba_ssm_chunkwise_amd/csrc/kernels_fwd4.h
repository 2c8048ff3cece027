// Forward main kernel in the lane-pair layout (bf16 inputs): four waves, one
// per SIMD, each owning whole state rows.
//
// Source: burn-mamba "recalculated.rs" source page, moments_phys_fwd (chunk
// states, de-rotation, masked moments) and "backward.rs", module doc "Gradient
// math" (h~[t] = d_t h_- + sum_{j<=t} L[t,j] W_j). Per (b,h) chain a workgroup
// walks a group of kernel chunks; wave w handles state rows p = w, w+4, ... for
// all 32 tokens of each chunk and keeps everything of a row in its own lanes:
//
//   states   h~[t][col] = sum_{(j,c)} W[t][(j,c)] bhat[(j,c)][col] on MFMA with
//            the token as the row index (W[t][(j,c)] = L[t,j] xhat[j,c,p] built
//            per lane), so a lane ends up holding one state column for eight
//            tokens (rows 4q+i of both 16-token tiles);
//   carry    + d_t h_-[p][col] (one value per lane and tile);
//   rotation in the lane: the internal column order puts the two members of a
//            complex pair (or the four components of a quaternion block) in the
//            same lane of consecutive column tiles;
//   moments  the packed bf16 values of a column tile are, as they stand, the
//            MFMA operand that contracts over the eight tokens (K slot 8q+e =
//            token 4q+e or 16+4q+e-4), so m2 += c^T c is accumulated for the upper
//            triangle of 16x16 tiles straight from registers (no LDS round trip,
//            half the tile products), and m1 through an operand that selects one
//            accumulator row per state row.
//
// Every wave holds its own partial m2 (upper triangle) and m1 rows; the fixed-
// order reduction k_reduce4 adds the partials and restores the caller's column
// order. With one group per chain the state entering each chunk is carried in
// LDS (rows are private to a wave, so no barrier guards them).
#pragma once

#include "kernels_bwdt.h"

namespace mom {

constexpr int NW4 = 4;          // waves of k_fwd4
constexpr int NT4 = 64 * NW4;   // threads of k_fwd4

// Internal column ic = 16*ct + n of the lane-pair order -> caller column, or -1
// for padding. ord: 0 identity, 1 complex pairs (x in tile 2k, y in tile 2k+1,
// pair 16k+n; g.half selects the half-split pairing), 3 quaternion blocks
// (component m in tile 4k+m, block 16k+n).
__host__ __device__ __forceinline__ int lp_col(const Geo& g, int ord, int ic) {
  const int ct = ic >> 4, n = ic & 15;
  int cc;
  if (ord == 1) {
    const int i = 16 * (ct >> 1) + n, m = ct & 1;
    if (g.half) cc = (i < (g.r >> 1)) ? (m ? (g.r >> 1) + i : i) : g.r;
    else cc = 2 * i + m;
  } else if (ord == 3) {
    cc = 4 * (16 * (ct >> 2) + n) + (ct & 3);
  } else {
    cc = ic;
  }
  return cc < g.r ? cc : -1;
}
// Caller column cc < r -> internal column of the lane-pair order.
__host__ __device__ __forceinline__ int lp_ic(const Geo& g, int ord, int cc) {
  if (ord == 1) {
    int i, m;
    if (g.half) {
      const int hr = g.r >> 1;
      m = cc >= hr;
      i = m ? cc - hr : cc;
    } else {
      i = cc >> 1;
      m = cc & 1;
    }
    return 16 * (2 * (i >> 4) + m) + (i & 15);
  }
  if (ord == 3) {
    const int j = cc >> 2, m = cc & 3;
    return 16 * (4 * (j >> 4) + m) + (j & 15);
  }
  return cc;
}

// LDS plan of k_fwd4 (byte offsets).
template <int NT, int CK>
struct LdsF4 {
  static constexpr int R = 16 * NT, K = ELL * CK, KP = cf_pitch(K);
  static constexpr size_t bsT = 0;                                     // bhat^T [col][(j,c)]
  __host__ __device__ static size_t xs() { return bsT + (size_t)R * KP * 2; }   // xhat [p][(j,c)]
  __host__ __device__ static size_t a(int pp) { return xs() + (size_t)pp * KP * 2; }
  __host__ __device__ static size_t d(int pp) { return a(pp) + ELL * 4; }
  __host__ __device__ static size_t rot(int pp) { return al16(d(pp) + ELL * 4); }
  // rotation table: complex [t][16*RG] (cos, sin); quaternion [t][16*RG] (w,x,y,z);
  // rows padded by 8 floats
  __host__ __device__ static int rpitch(int rot_kind, int RG) {
    return (rot_kind == 3 ? 64 * RG : 32 * RG) + 8;
  }
  __host__ __device__ static size_t carryL(int pp, int rot_kind, int RG) {
    return al16(rot(pp) + (RG > 0 ? (size_t)ELL * rpitch(rot_kind, RG) * 4 : 0));
  }
  // a scratch slot per lane (and wave) for the carry stores of lanes that do
  // not hold the last token: their values are discarded
  __host__ __device__ static size_t dummy(int pp, int rot_kind, int RG, bool inc) {
    return carryL(pp, rot_kind, RG) + (inc ? (size_t)pp * R * 4 : 0);
  }
  // total: with the state rows carried in LDS ([p][R] fp32) or not
  __host__ __device__ static size_t total(int pp, int rot_kind, int RG, bool inc) {
    return dummy(pp, rot_kind, RG, inc) + (inc ? (size_t)NW4 * 64 * 4 : 0);
  }
};

// Rotated column groups (compile-time RG, a power of two; 0 = none): complex
// pairs come 16 to a group of two tiles, quaternion blocks 16 to a group of four.
__host__ __device__ __forceinline__ int rot_groups(const Geo& g) {
  const int need = (g.rot_kind == 1 || g.rot_kind == 2) ? (g.A + 15) / 16 : g.rot_kind == 3 ? (g.J + 15) / 16 : 0;
  if (need == 0) return 0;
  int rg = 1;
  while (rg < need) rg *= 2;
  return rg;
}

// Inclusive cumsum of da over the 32 tokens of a chunk (lanes 0..31 of wave 0
// hold da), stored as a_t and d_t = exp(a_t).
__device__ __forceinline__ void scan_store_decay(float v, int tid, float* s_a, float* s_d) {
  const int tk = tid & 31;
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    const float up = __shfl_up(v, off, 32);
    if (tk >= off) v += up;
  }
  if (tid < 32) {
    s_a[tk] = v;
    s_d[tk] = expf(v);
  }
}

// Chunk inputs of k_fwd4 staged with wide loads, all issued before the first
// LDS store (one memory latency per chunk instead of one per element). Used
// when every caller row is 16-byte aligned (r and p multiples of 8; an even
// number of angles). Work items run over (j,c) fastest, so the lanes of a wave
// write consecutive (j,c) of one LDS row.
template <int NT, int CK, int ROT, int RG>
struct Stage4 {
  static constexpr int R = 16 * NT, K = ELL * CK, KP = cf_pitch(K);
  static constexpr int NBU = K * R / 8, NBL = (NBU + NT4 - 1) / NT4;        // bhat: 8 columns per load
  static constexpr int NXL = (K * 128 / 8 + NT4 - 1) / NT4;                // xhat: 8 rows per load, p <= 128
  static constexpr int NRU = ROT == 1 ? ELL * 8 * RG : ROT == 3 ? ELL * 16 * RG : 0;  // 2 angles | 1 quaternion
  static constexpr int NRL = NRU > 0 ? (NRU + NT4 - 1) / NT4 : 1;
  u4 bv[NBL];
  u4 xv[NXL];
  unsigned r1[NRL];
  unsigned long long r3[NRL];
  float dav;

  __device__ static bool usable(const Geo& g) {
    return (g.r % 8) == 0 && (g.p % 8) == 0 && (ROT != 1 || (g.A % 2) == 0);
  }
  __device__ void load(const Geo& g, const bf16* __restrict__ xhat, const bf16* __restrict__ bhat,
                       const bf16* __restrict__ rot, const bf16* __restrict__ da, int nc, int bi, int hi, int tid,
                       int PP) {
    dav = (tid < 32 && nc * ELL + tid < g.V) ? (float)da[((size_t)bi * g.s + nc * ELL + tid) * g.h + hi] : 0.0f;
#pragma unroll
    for (int i = 0; i < NBL; i++) {
      const int idx = tid + i * NT4;
      const int k = idx % K, c8 = idx / K;
      const int j = k / CK, ci = k % CK, pos = nc * ELL + j;
      bv[i] = u4{0u, 0u, 0u, 0u};
      if (idx < NBU && 8 * c8 < g.r && ci < g.c && pos < g.V)
        bv[i] = *reinterpret_cast<const u4*>(bhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + 8 * c8);
    }
#pragma unroll
    for (int i = 0; i < NXL; i++) {
      const int idx = tid + i * NT4;
      const int k = idx % K, p8 = idx / K;
      const int j = k / CK, ci = k % CK, pos = nc * ELL + j;
      xv[i] = u4{0u, 0u, 0u, 0u};
      if (8 * p8 < PP && 8 * p8 < g.p && ci < g.c && pos < g.V)
        xv[i] = *reinterpret_cast<const u4*>(xhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + 8 * p8);
    }
#pragma unroll
    for (int i = 0; i < NRL; i++) {
      const int idx = tid + i * NT4;
      if constexpr (ROT == 1) {
        const int tk = idx / (8 * RG), a2 = idx % (8 * RG), pos = nc * ELL + tk;
        r1[i] = 0u;
        if (idx < NRU && 2 * a2 < g.A && pos < g.V)
          r1[i] = *reinterpret_cast<const unsigned*>(rot + (((size_t)bi * g.s + pos) * g.h + hi) * g.RW + 2 * a2);
      } else if constexpr (ROT == 3) {
        const int tk = idx / (16 * RG), jb = idx % (16 * RG), pos = nc * ELL + tk;
        r3[i] = 0x3f80ull;  // bf16 (1, 0, 0, 0): the identity quaternion
        if (idx < NRU && jb < g.J && pos < g.V)
          r3[i] = *reinterpret_cast<const unsigned long long*>(rot + (((size_t)bi * g.s + pos) * g.h + hi) * g.RW + 4 * jb);
      }
    }
  }
  __device__ void store(const Geo& g, bf16* bsT, bf16* xs, float* rt, float* s_a, float* s_d, int tid,
                        int rpitch) const {
    if (tid < 64) scan_store_decay(dav, tid, s_a, s_d);
#pragma unroll
    for (int i = 0; i < NBL; i++) {
      const int idx = tid + i * NT4;
      if (idx >= NBU) continue;
      const int k = idx % K, c8 = idx / K;
      if (8 * c8 >= g.r) continue;
      const bf16* v = reinterpret_cast<const bf16*>(&bv[i]);
#pragma unroll
      for (int e = 0; e < 8; e++) bsT[lp_ic(g, ROT, 8 * c8 + e) * KP + k] = v[e];
    }
#pragma unroll
    for (int i = 0; i < NXL; i++) {
      const int idx = tid + i * NT4;
      const int k = idx % K, p8 = idx / K;
      if (8 * p8 >= g.p) continue;
      const bf16* v = reinterpret_cast<const bf16*>(&xv[i]);
#pragma unroll
      for (int e = 0; e < 8; e++) xs[(8 * p8 + e) * KP + k] = v[e];
    }
#pragma unroll
    for (int i = 0; i < NRL; i++) {
      const int idx = tid + i * NT4;
      if (idx >= NRU) continue;
      if constexpr (ROT == 1) {
        const int tk = idx / (8 * RG), a2 = idx % (8 * RG);
        float s0, c0, s1, c1;
        sincosf(bf16_lo(r1[i]), &s0, &c0);
        sincosf(bf16_hi(r1[i]), &s1, &c1);
        *reinterpret_cast<f4*>(rt + tk * rpitch + 4 * a2) = f4{c0, s0, c1, s1};
      } else if constexpr (ROT == 3) {
        const int tk = idx / (16 * RG), jb = idx % (16 * RG);
        const unsigned lo = (unsigned)r3[i], hi = (unsigned)(r3[i] >> 32);
        *reinterpret_cast<f4*>(rt + tk * rpitch + 4 * jb) = f4{bf16_lo(lo), bf16_hi(lo), bf16_lo(hi), bf16_hi(hi)};
      }
    }
  }
};

// Index of the upper-triangle tile (a <= b) in a flat array.
template <int NT>
__host__ __device__ constexpr int tri(int a, int b) {
  return a * NT - a * (a - 1) / 2 + (b - a);
}

template <int NT, int ROT, int CK, int RG, int M1T, int INC>
__global__ __launch_bounds__(NT4, 1) void k_fwd4(Geo g, const bf16* __restrict__ xhat,
                                                  const bf16* __restrict__ bhat, const bf16* __restrict__ da,
                                                  const bf16* __restrict__ rot, const float* __restrict__ carry,
                                                  const bf16* __restrict__ h0, float* m2part, float* m1part,
                                                  float* __restrict__ save, float* __restrict__ save_dec) {
  constexpr int R = 16 * NT, K = ELL * CK, KP = cf_pitch(K);
  constexpr int NKS0 = CK >= 2 ? CK / 2 : 1;   // K-steps seen by tokens 0..15 (j <= 15)
  constexpr int NTRI = NT * (NT + 1) / 2;
  constexpr int ORD = ROT;                      // column order of the kernel
  constexpr int RGS = ROT == 3 ? 4 : 2;         // tiles per rotated group
  constexpr int GS = RGS, NG = NT / GS;         // column tiles per group of the row work
  static_assert((ROT == 0) == (RG == 0) && RG * RGS <= NT, "rotation groups");
  using L = LdsF4<NT, CK>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int PP = 4 * ((g.p + 3) / 4);
  const int rpitch = L::rpitch(ROT, RG);
  bf16* bsT = (bf16*)(smem + L::bsT);
  bf16* xs = (bf16*)(smem + L::xs());
  float* s_a = (float*)(smem + L::a(PP));
  float* s_d = (float*)(smem + L::d(PP));
  float* rt = (float*)(smem + L::rot(PP));
  float* carryL = (float*)(smem + L::carryL(PP, ROT, RG));

  const int bh = blockIdx.x / g.NGR, gi = blockIdx.x % g.NGR;
  const int bi = bh / g.h, hi = bh % g.h;
  g.V = chain_len(g, bi);  // this sequence's valid length (per-sequence lengths)
  int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, n = lane & 15, q = lane >> 4;
  const int nrow = (g.p - w + 3) / 4;  // rows of this wave: p = w + 4k

  // INC 0: entering states from the carry pass; 1: carried in LDS (carry ==
  // nullptr); 2: carried, and also written to `save` / `save_dec`; 3: carried in
  // LDS through the group, from the carry pass's state entering its first chunk
  // (the only one of the group's states that carry pass stores)
  constexpr bool inc = INC != 0;
  // index of this lane's columns in the carry-pass rows (their column order
  // interleaves half-split pairs), -1 for padding
  int cidx[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ct++) {
    const int cc = lp_col(g, ORD, 16 * ct + n);
    cidx[ct] = cc >= 0 ? inv_perm_rc(g, cc) : -1;
  }
  // saving the carries: lane-pair column of carry-pass column 64u + lane (-1 past r)
  int sic[(R + 63) / 64];
#pragma unroll
  for (int u = 0; u < (R + 63) / 64; u++) {
    const int col = 64 * u + lane;
    sic[u] = INC == 2 && col < g.r ? lp_ic(g, ORD, perm_rc(g, col)) : -1;
  }
  if (inc) {
    const float* c0 = INC == 3 ? carry + ((size_t)bh * g.NK + (size_t)gi * g.G) * g.p * g.r : nullptr;
    for (int idx = tid; idx < g.p * R; idx += NT4) {
      const int pp = idx / R, ic = idx % R;
      const int cc = lp_col(g, ORD, ic);
      float v = 0.0f;
      if (INC == 3) {
        if (cc >= 0) v = c0[(size_t)pp * g.r + inv_perm_rc(g, cc)];  // carry-pass column order
      } else if (h0 != nullptr && cc >= 0) {
        v = (float)h0[((size_t)bh * g.p + pp) * g.r + cc];
      }
      carryL[idx] = v;
    }
  }

  f4 m2acc[NTRI];
#pragma unroll
  for (int i = 0; i < NTRI; i++) m2acc[i] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  static_assert(M1T == 1 || M1T == 2, "m1 tiles: 16 rows of the wave each (p <= 64 or 128)");
  f4 m1acc[M1T][NT];
#pragma unroll
  for (int a = 0; a < M1T; a++)
#pragma unroll
    for (int b = 0; b < NT; b++) m1acc[a][b] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  int nc = 0;  // the chunk being processed
  // The row work of one chunk (see the software pipeline at its call). Tokens
  // past valid_len have zero W factors and decays, so their states, and c,
  // come out as exact zeros.
  float* dummyL = (float*)(smem + L::dummy(PP, ROT, RG, inc)) + (size_t)w * 64;
  auto rows = [&](const float (&dtok)[2][4], const float (&lw)[2][CK][8 / CK]) {
    if (nrow == 0) return;
    using RV = typename std::conditional<ROT == 3, f4, fl2>::type;
    constexpr int NRV = RG > 0 ? RG * 8 : 1;
    auto rowp = [&](int kk) { return w + 4 * (kk < nrow ? kk : nrow - 1); };
    auto load_x = [&](int pr, u4 (&x8)[CK]) {
#pragma unroll
      for (int ks = 0; ks < CK; ks++) x8[ks] = *reinterpret_cast<const u4*>(xs + pr * KP + 32 * ks + 8 * q);
    };
    // W fragments (A operand: token rows, (j,c) K-slots): L[t][j] xhat[(j,c)][p]
    auto build_w = [&](const u4 (&x8)[CK], u4 (&Wf)[2][CK]) {
#pragma unroll
      for (int ks = 0; ks < CK; ks++) {
        float xv[8];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          xv[2 * e] = bf16_lo(x8[ks][e]);
          xv[2 * e + 1] = bf16_hi(x8[ks][e]);
        }
#pragma unroll
        for (int tt = 0; tt < 2; tt++) {
          if (tt == 0 && ks >= NKS0) continue;
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            Wf[tt][ks][e / 2] = pk_bf16(lw[tt][ks][e / CK] * xv[e], lw[tt][ks][(e + 1) / CK] * xv[e + 1]);
        }
      }
    };
    auto load_hv = [&](int pr, float (&hv)[NT]) {
      if constexpr (inc) {
#pragma unroll
        for (int ct = 0; ct < NT; ct++) hv[ct] = carryL[pr * R + 16 * ct + n];
      } else {
        const float* crow = carry + (((size_t)bh * g.NK + nc) * g.p + pr) * g.r;
#pragma unroll
        for (int ct = 0; ct < NT; ct++) hv[ct] = cidx[ct] >= 0 ? crow[cidx[ct]] : 0.0f;
      }
    };
    auto load_rv = [&](RV (&rv)[NRV]) {
#pragma unroll
      for (int k = 0; k < RG; k++)
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
          for (int i = 0; i < 4; i++)
            rv[(k * 2 + tt) * 4 + i] =
                *reinterpret_cast<const RV*>(rt + (16 * tt + 4 * q + i) * rpitch + GS * (16 * k + n));
    };
    // states of a row: column tile ct, token tile tt
    auto states = [&](const u4 (&Wf)[2][CK], f4 (&h)[2][NT]) {
#pragma unroll
      for (int ct = 0; ct < NT; ct++) {
        bf8 bfr[CK];
#pragma unroll
        for (int ks = 0; ks < CK; ks++) bfr[ks] = ld_frag(bsT + (16 * ct + n) * KP + 32 * ks + 8 * q);
#pragma unroll
        for (int tt = 0; tt < 2; tt++) {
          f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < CK; ks++)
            if (tt == 1 || ks < NKS0) acc = MM<bf16>::mma(as_bf8(Wf[tt][ks]), bfr[ks], acc);
          h[tt][ct] = acc;
        }
      }
    };
    // carry, carry out of the chunk, de-rotation, mask, packing of a row
    auto finish = [&](int pr, bool real, f4 (&h)[2][NT], const float (&hv)[NT], const RV (&rv)[NRV],
                      bf8 (&cf)[NT]) {
#pragma unroll
      for (int ct = 0; ct < NT; ct++)
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
          for (int i = 0; i < 4; i++) h[tt][ct][i] += dtok[tt][i] * hv[ct];
      if constexpr (inc) {
        // the state at the chunk's last token (lanes q = 3) enters the next chunk;
        // the other lanes, and repeated rows, store to their scratch slot instead
        float* dst = (q == 3 && real) ? carryL + pr * R + n : dummyL + lane;
        const int step = (q == 3 && real) ? 16 : 0;
#pragma unroll
        for (int ct = 0; ct < NT; ct++) dst[ct * step] = h[1][ct][3];
      }
      if constexpr (ROT == 1) {
#pragma unroll
        for (int k = 0; k < RG; k++)
#pragma unroll
          for (int tt = 0; tt < 2; tt++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const fl2 cs = rv[(k * 2 + tt) * 4 + i];
              const float x = h[tt][2 * k][i], y = h[tt][2 * k + 1][i];
              h[tt][2 * k][i] = cs[0] * x + cs[1] * y;
              h[tt][2 * k + 1][i] = cs[0] * y - cs[1] * x;
            }
      } else if constexpr (ROT == 3) {
#pragma unroll
        for (int k = 0; k < RG; k++)
#pragma unroll
          for (int tt = 0; tt < 2; tt++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const f4 Q = rv[(k * 2 + tt) * 4 + i];
              const float h0v = h[tt][4 * k][i], h1 = h[tt][4 * k + 1][i];
              const float h2 = h[tt][4 * k + 2][i], h3 = h[tt][4 * k + 3][i];
              h[tt][4 * k][i] = Q[0] * h0v - Q[1] * h1 - Q[2] * h2 - Q[3] * h3;
              h[tt][4 * k + 1][i] = Q[0] * h1 + Q[1] * h0v + Q[2] * h3 - Q[3] * h2;
              h[tt][4 * k + 2][i] = Q[0] * h2 - Q[1] * h3 + Q[2] * h0v + Q[3] * h1;
              h[tt][4 * k + 3][i] = Q[0] * h3 + Q[1] * h2 - Q[2] * h1 + Q[3] * h0v;
            }
      }
#pragma unroll
      for (int ct = 0; ct < NT; ct++) {
        const u4 v = u4{pk_bf16(h[0][ct][0], h[0][ct][1]), pk_bf16(h[0][ct][2], h[0][ct][3]),
                        pk_bf16(h[1][ct][0], h[1][ct][1]), pk_bf16(h[1][ct][2], h[1][ct][3])};
        cf[ct] = as_bf8(v);
      }
    };
    // prologue: row 0 finished, W of row 1, xhat of row 2 requested
    bf8 cf[NT];
    u4 W[2][CK];
    u4 x8[CK];
    {
      load_x(rowp(0), x8);
      build_w(x8, W);
      float hv[NT];
      load_hv(rowp(0), hv);
      RV rv[NRV];
      load_rv(rv);
      f4 h[2][NT];
      states(W, h);
      finish(rowp(0), true, h, hv, rv, cf);
      load_x(rowp(1), x8);
      build_w(x8, W);
      load_x(rowp(2), x8);
    }
    // W fragments of K-step ks only (a piece of build_w)
    auto build_w_ks = [&](int ks, const u4 (&x8)[CK], u4 (&Wf)[2][CK]) {
      float xv[8];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        xv[2 * e] = bf16_lo(x8[ks][e]);
        xv[2 * e + 1] = bf16_hi(x8[ks][e]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; tt++) {
        if (tt == 0 && ks >= NKS0) continue;
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          Wf[tt][ks][e / 2] = pk_bf16(lw[tt][ks][e / CK] * xv[e], lw[tt][ks][(e + 1) / CK] * xv[e + 1]);
      }
    };
    // carry, carry out of the chunk, de-rotation and packing of column group gr
    auto finish_g = [&](int gr, int pr, bool real, f4 (&h)[2][NT], const float (&hv)[NT], const RV (&rv)[NRV],
                        bf8 (&cfo)[NT]) {
#pragma unroll
      for (int u = 0; u < GS; u++)
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
          for (int i = 0; i < 4; i++) h[tt][gr * GS + u][i] += dtok[tt][i] * hv[gr * GS + u];
      if constexpr (inc) {
        float* dst = (q == 3 && real) ? carryL + pr * R + n : dummyL + lane;
        const int stp = (q == 3 && real) ? 16 : 0;
#pragma unroll
        for (int u = 0; u < GS; u++) dst[(gr * GS + u) * stp] = h[1][gr * GS + u][3];
      }
      if (gr < RG) {
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            if constexpr (ROT == 1) {
              const fl2 cs = rv[(gr * 2 + tt) * 4 + i];
              const float x = h[tt][2 * gr][i], y = h[tt][2 * gr + 1][i];
              h[tt][2 * gr][i] = cs[0] * x + cs[1] * y;
              h[tt][2 * gr + 1][i] = cs[0] * y - cs[1] * x;
            } else if constexpr (ROT == 3) {
              const f4 Q = rv[(gr * 2 + tt) * 4 + i];
              const float h0v = h[tt][4 * gr][i], h1 = h[tt][4 * gr + 1][i];
              const float h2 = h[tt][4 * gr + 2][i], h3 = h[tt][4 * gr + 3][i];
              h[tt][4 * gr][i] = Q[0] * h0v - Q[1] * h1 - Q[2] * h2 - Q[3] * h3;
              h[tt][4 * gr + 1][i] = Q[0] * h1 + Q[1] * h0v + Q[2] * h3 - Q[3] * h2;
              h[tt][4 * gr + 2][i] = Q[0] * h2 - Q[1] * h3 + Q[2] * h0v + Q[3] * h1;
              h[tt][4 * gr + 3][i] = Q[0] * h3 + Q[1] * h2 - Q[2] * h1 + Q[3] * h0v;
            }
          }
      }
#pragma unroll
      for (int u = 0; u < GS; u++) {
        const int ct = gr * GS + u;
        const u4 v = u4{pk_bf16(h[0][ct][0], h[0][ct][1]), pk_bf16(h[0][ct][2], h[0][ct][3]),
                        pk_bf16(h[1][ct][0], h[1][ct][1]), pk_bf16(h[1][ct][2], h[1][ct][3])};
        cfo[ct] = as_bf8(v);
      }
    };
    constexpr int NMF = NTRI + NT;  // moment MFMAs of a row: the m2 tiles, then the m1 tiles
    auto step = [&](int kk, auto m1i_c) {
      constexpr int M1I = decltype(m1i_c)::value;
      const int p1 = rowp(kk + 1);
      float hvn[NT];
      load_hv(p1, hvn);
      RV rvn[NRV];
      load_rv(rvn);
      const bf16 one = (bf16)(n == (kk & 15) ? 1.0f : 0.0f);
      bf8 sel;
#pragma unroll
      for (int e = 0; e < 8; e++) sel[e] = one;
      // phase 1: the states of row kk+1 (bhat^T fragments one tile ahead), with
      // the W fragments of row kk+2 built in between
      f4 hn[2][NT];
      u4 Wn[2][CK];
      bf8 bfn[CK];
#pragma unroll
      for (int ks = 0; ks < CK; ks++) bfn[ks] = ld_frag(bsT + n * KP + 32 * ks + 8 * q);
#pragma unroll
      for (int ct = 0; ct < NT; ct++) {
        bf8 bfr[CK];
#pragma unroll
        for (int ks = 0; ks < CK; ks++) bfr[ks] = bfn[ks];
        if (ct + 1 < NT) {
#pragma unroll
          for (int ks = 0; ks < CK; ks++) bfn[ks] = ld_frag(bsT + (16 * (ct + 1) + n) * KP + 32 * ks + 8 * q);
        }
#pragma unroll
        for (int tt = 0; tt < 2; tt++) {
          f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < CK; ks++)
            if (tt == 1 || ks < NKS0) acc = MM<bf16>::mma(as_bf8(W[tt][ks]), bfr[ks], acc);
          hn[tt][ct] = acc;
        }
        if (ct < CK) build_w_ks(ct, x8, Wn);
        __builtin_amdgcn_sched_barrier(0);
      }
      load_x(rowp(kk + 3), x8);
      // phase 2: the moment MFMAs of row kk, a share after each column group's
      // carry, rotation and packing of row kk+1
      bf8 cfn[NT];
#pragma unroll
      for (int gr = 0; gr < NG; gr++) {
        finish_g(gr, p1, kk + 1 < nrow, hn, hvn, rvn, cfn);
#pragma unroll
        for (int i = gr * NMF / NG; i < (gr + 1) * NMF / NG; i++) {
          if (i < NTRI) {
            int a = 0, b = 0, r = i;
#pragma unroll
            for (int aa = 0; aa < NT; aa++) {
              if (r >= 0 && r < NT - aa) { a = aa; b = aa + r; }
              r -= NT - aa;
            }
            m2acc[i] = MM<bf16>::mma(cf[a], cf[b], m2acc[i]);
          } else {
            const int ct = i - NTRI;
            m1acc[M1I][ct] = MM<bf16>::mma(sel, cf[ct], m1acc[M1I][ct]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int ct = 0; ct < NT; ct++) cf[ct] = cfn[ct];
#pragma unroll
      for (int tt = 0; tt < 2; tt++)
#pragma unroll
        for (int ks = 0; ks < CK; ks++) W[tt][ks] = Wn[tt][ks];
    };
    const int nlo = nrow < 16 ? nrow : 16;
    for (int kk = 0; kk < nlo; kk++) step(kk, IC4<0>{});
    if constexpr (M1T > 1) {
      for (int kk = 16; kk < nrow; kk++) step(kk, IC4<M1T - 1>{});
    }
  };

  const int n0 = gi * g.G;
  const int nkc = chain_nk(g);  // chunks walked
  const int n1 = (n0 + g.G < nkc) ? n0 + g.G : nkc;
  using ST = Stage4<NT, CK, ROT, RG>;
  const bool wide = ST::usable(g);
  ST st;
  // columns no caller column maps to stay zero in bhat^T
  for (int idx = tid; idx < R * KP; idx += NT4) bsT[idx] = (bf16)0.0f;
  for (nc = n0; nc < n1; nc++) {
    asm volatile("" : "+v"(tid));
    // ---- chunk staging -------------------------------------------------------
    if (wide) st.load(g, xhat, bhat, rot, da, nc, bi, hi, tid, PP);
    __syncthreads();  // the previous chunk's rows are done with the tables
    if (wide) {
      st.store(g, bsT, xs, rt, s_a, s_d, tid, rpitch);
    } else {
      if (tid < 64) {
        const int tk = tid & 31;
        float v = (tid < 32 && nc * ELL + tk < g.V) ? (float)da[((size_t)bi * g.s + nc * ELL + tk) * g.h + hi] : 0.0f;
        scan_store_decay(v, tid, s_a, s_d);
      }
      // bhat^T in the internal column order; work items over (j,c) fastest
      for (int idx = tid; idx < K * R; idx += NT4) {
        const int k = idx % K, ic = idx / K;
        const int j = k / CK, ci = k % CK, pos = nc * ELL + j;
        const int cc = lp_col(g, ORD, ic);
        bf16 v = (bf16)0.0f;
        if (cc >= 0 && ci < g.c && pos < g.V) v = bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + cc];
        bsT[ic * KP + k] = v;
      }
      for (int idx = tid; idx < K * PP; idx += NT4) {
        const int k = idx % K, pp = idx / K;
        const int j = k / CK, ci = k % CK, pos = nc * ELL + j;
        bf16 v = (bf16)0.0f;
        if (pp < g.p && ci < g.c && pos < g.V) v = xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pp];
        xs[pp * KP + k] = v;
      }
      if constexpr (ROT == 1) {
        for (int idx = tid; idx < ELL * 16 * RG; idx += NT4) {
          const int tk = idx / (16 * RG), i = idx % (16 * RG), pos = nc * ELL + tk;
          float th = 0.0f;
          if (i < g.A && pos < g.V) th = (float)rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + i];
          float sv, cv;
          sincosf(th, &sv, &cv);
          *reinterpret_cast<fl2*>(rt + tk * rpitch + 2 * i) = fl2{cv, sv};
        }
      } else if constexpr (ROT == 3) {
        for (int idx = tid; idx < ELL * 16 * RG; idx += NT4) {
          const int tk = idx / (16 * RG), jb = idx % (16 * RG), pos = nc * ELL + tk;
          f4 v = f4{1.0f, 0.0f, 0.0f, 0.0f};
          if (jb < g.J && pos < g.V) {
            const bf16* src = rot + (((size_t)bi * g.s + pos) * g.h + hi) * g.RW + 4 * jb;
            v = f4{(float)src[0], (float)src[1], (float)src[2], (float)src[3]};
          }
          *reinterpret_cast<f4*>(rt + tk * rpitch + 4 * jb) = v;
        }
      }
    }
    __syncthreads();

    // ---- per-lane chunk constants -------------------------------------------
    const int tv = g.V - nc * ELL;  // valid tokens of this chunk (<= 0: none)
    float dtok[2][4];               // d_t at the lane's tokens 16tt + 4q + i (0 past valid_len)
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      const f4 v = *reinterpret_cast<const f4*>(s_d + 16 * tt + 4 * q);
#pragma unroll
      for (int i = 0; i < 4; i++) dtok[tt][i] = 16 * tt + 4 * q + i < tv ? v[i] : 0.0f;
    }
    // W factors L[t][j] for the lane's token t = 16tt + n and its K-slots
    // 32ks + 8q + e ((j,c) folded, j = slot / CK); zero above the diagonal
    float lw[2][CK][8 / CK];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      const int tk = 16 * tt + n;
      const float at = s_a[tk];
#pragma unroll
      for (int ks = 0; ks < CK; ks++)
#pragma unroll
        for (int v = 0; v < 8 / CK; v++) {
          const int j = (32 * ks + 8 * q) / CK + v;
          lw[tt][ks][v] = (tt == 1 || ks < NKS0) && j <= tk && tk < tv ? expf(at - s_a[j]) : 0.0f;
        }
    }

    // ---- the wave's rows -----------------------------------------------------
    // Software pipeline over the wave's rows: one step issues the states MFMAs of
    // row kk+1 and the moment MFMAs of row kk, and between them the VALU work of
    // row kk+1 (carry, rotation, packing) and the W fragments of row kk+2, so the
    // single wave of the SIMD keeps its MFMA pipe fed while it does the lane work.
    // Steps past the last row work on the last row again and discard the result.
    if constexpr (INC == 2) {
      // With INC == 2 (one group per chain) the state entering the chunk, and the
      // chunk's decay, are also written out in the carry pass's layout (fp32,
      // [p][r] in its column order), so that a later backward can skip its
      // carry pass. The rows are the wave's own, as in LDS; one store per 64
      // consecutive columns.
      float* dst = save + ((size_t)bh * g.NK + nc) * g.p * g.r;
      for (int pr = w; pr < g.p; pr += 4)
#pragma unroll
        for (int u = 0; u < (R + 63) / 64; u++)
          if (sic[u] >= 0) dst[(size_t)pr * g.r + 64 * u + lane] = carryL[pr * R + sic[u]];
      if (tid == 0 && nc + 1 < g.NK) save_dec[(size_t)bh * g.NK + nc] = s_d[ELL - 1];
    }
    rows(dtok, lw);
  }
  // ---- this wave's partials: m2 tiles (upper triangle mirrored) and m1 rows ----
  float* m2o = m2part + (((size_t)bh * g.NGR + gi) * NW4 + w) * R * R;
#pragma unroll
  for (int a = 0; a < NT; a++)
#pragma unroll
    for (int b = a; b < NT; b++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float v = m2acc[tri<NT>(a, b)][i];
        m2o[(16 * a + 4 * q + i) * R + 16 * b + n] = v;
        if (a < b) m2o[(16 * b + n) * R + 16 * a + 4 * q + i] = v;
      }
  float* m1o = m1part + ((size_t)bh * g.NGR + gi) * g.p * R;
#pragma unroll
  for (int a = 0; a < M1T; a++)
#pragma unroll
    for (int b = 0; b < NT; b++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int pp = w + 4 * (16 * a + 4 * q + i);
        if (pp < g.p) m1o[(size_t)pp * R + 16 * b + n] = m1acc[a][b][i];
      }
}

}  // namespace mom

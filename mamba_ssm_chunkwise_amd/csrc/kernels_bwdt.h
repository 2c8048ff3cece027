// Backward main kernel in the transposed state layout (bf16 inputs, K <= 64).
//
// Same contract as k_bwd (sources: burn-mamba "recalculated.rs" and
// "backward.rs" source pages, moments_phys_bwd and its module doc "Gradient
// math"): per (b,h) chain and kernel chunk it recomputes the states, applies
// the de-rotation, and writes d_xhat, d_bhat, d_da without the carry-cotangent
// terms, d_rot complete, and local(n)[p][col] = sum_t d_t G[t][p][col] for the
// carry-cotangent recurrence.
//
// Layout. One wave owns whole state rows p (all columns, all 32 tokens of the
// chunk). The states are computed transposed, h~^T[col][t] = bhat^T W^T with
// W[t][(j,c)] = L[t,j] xhat[j,c,p], so an accumulator lane holds one token and
// four consecutive state columns: complex pairs and quaternion 4-blocks sit in
// one lane's registers and the rotation, its transpose and its gradient need
// no lane exchange. The packed c^T fragments feed d_c^T = S c^T directly
// (S = d_m2 + d_m2^T). G^T is the A operand of Y = G bhat^T, from which
// d_xhat[(j,c)] = sum_t L[t,j] Y[t,(j,c)]. The token contractions that need
// tokens in registers (d_bhat over (t,p), local over t) read G through a small
// per-row LDS transpose.
//
// Per round, wave w handles row 4*round + w; after a barrier the four waves
// accumulate d_bhat for the round's rows, each owning a quarter of the
// (j,c) x column tiles.
#pragma once

#include "kernels.h"

namespace mom {

constexpr int NWT = 4;          // waves of k_bwdt
constexpr int NTT = 64 * NWT;   // threads of k_bwdt
constexpr int GSP = 40;         // G transpose: bf16 per state column (32 tokens + pad)
constexpr int LTP = 36;         // row pitch of LT[j][t] (floats)
constexpr int XPB = 32;         // state rows per staged xhat block

// Column-contracting fragments built from accumulator registers: K-slot
// 32ks + 8q + e holds state column 32ks + 16(e/4) + 4q + e%4, i.e. register
// e%4 of column tile 2ks + e/4 in lane group q.
__host__ __device__ __forceinline__ int col_of_slot(int s) {
  const int ks = s >> 5, q = (s >> 3) & 3, e = s & 7;
  return 32 * ks + 16 * (e >> 2) + 4 * q + (e & 3);
}
__host__ __device__ __forceinline__ int slot_of_col(int c) {
  const int ks = c >> 5, h = (c >> 4) & 1, q = (c >> 2) & 3, e = c & 3;
  return 32 * ks + 8 * q + 4 * h + e;
}

// Column tiles of 16 internal state columns that carry a rotation, rounded up
// to a power of two (0: no rotation). Complex pairs 8 per tile, quaternion
// blocks 4 per tile. The rotation tables of k_bwdt hold RT tiles per token,
// padded with the identity: complex [t][8RT][cos, sin], quaternion [t][4RT][4],
// each token row padded by 4 floats so consecutive tokens start in different
// banks.
__host__ __device__ __forceinline__ int rot_tiles(const Geo& g) {
  const int need = (g.rot_kind == 1 || g.rot_kind == 2) ? (g.A + 7) / 8 : g.rot_kind == 3 ? (g.J + 3) / 4 : 0;
  if (need == 0) return 0;
  int rt = 1;
  while (rt < need) rt *= 2;
  return rt;
}

// LDS plan: every region at a compile-time offset (so LDS addresses fold into
// instruction offsets); the rotation table, sized at run time, comes last.
// Per-lane chunk constants are float4 rows interleaved by lane ([entry][lane]
// of 16 bytes, conflict-free): LWE entries of W factors, 2*NKT of d_xhat
// factors.
constexpr int LWE = 4;
template <int NT, int CK>
struct LdsT {
  static constexpr int R = 16 * NT, K = ELL * CK, SP = R + 8, KP = K + 8;
  static constexpr size_t Ss = 0;                                     // S rows, K-slot order
  static constexpr size_t bsT = Ss + (size_t)R * SP * 2;              // bhat^T [col][(j,c)]
  static constexpr size_t bsY = bsT + (size_t)R * KP * 2;             // bhat [(j,c)][col slot]
  static constexpr size_t xs = bsY + (size_t)K * SP * 2;              // xhat block [p][(j,c)]
  static constexpr size_t dXs = xs + (size_t)XPB * KP * 2;            // d_xhat block [p][(j,c)]
  static constexpr size_t LT = dXs + (size_t)XPB * KP * 2;            // L^T [j][t]
  static constexpr size_t a = LT + (size_t)ELL * LTP * 4;
  static constexpr size_t d = a + ELL * 4;
  static constexpr size_t lw = d + ELL * 4;
  static constexpr size_t cst = lw + (size_t)(LWE + 2 * (K / 16)) * 64 * 16;  // carry, d_m1 rows [2][4][R]
  static constexpr size_t red = cst + (size_t)2 * 4 * R * 4;
  // G transposes of the round's rows; at chunk end the d_bhat tile and the
  // rotation-gradient reduction reuse the space
  static constexpr size_t gsb = (size_t)NWT * R * GSP * 2 > (size_t)K * SP * 2 ? (size_t)NWT * R * GSP * 2
                                                                                : (size_t)K * SP * 2;
  static constexpr size_t Gs = red + (size_t)(NWT * 4 * ELL + NWT * K + ELL) * 4;
  static constexpr size_t rot = Gs + gsb;
  static_assert(Gs % 16 == 0 && rot % 16 == 0 && lw % 16 == 0, "aligned regions");
  // rotation table (RT rotated tiles): 16*RT + 4 floats per token
  __host__ __device__ static size_t total(int RT) { return rot + (size_t)ELL * (16 * RT + 4) * 4; }
  // the rotation-gradient reduction [wave][t][8RT or 16RT] must fit the G space
  __host__ __device__ static bool fits(int rot_kind, int RT) {
    const size_t rw = rot_kind == 3 ? (size_t)16 * RT : (size_t)8 * RT;
    return (size_t)NWT * ELL * rw * 4 <= gsb;
  }
};

// d_m1 in the internal column order, rows padded to R: dm1i[bh][p][R].
__global__ __launch_bounds__(NTH) void k_prep_dm1(Geo g, int R, const float* __restrict__ dm1, float* dm1i) {
  const size_t e = (size_t)blockIdx.x * NTH + threadIdx.x;
  const size_t total = (size_t)g.b * g.h * g.p * R;
  if (e >= total) return;
  const int col = (int)(e % R);
  const size_t row = e / R;
  dm1i[e] = col < g.r ? dm1[row * g.r + perm_rc(g, col)] : 0.0f;
}

// Four consecutive internal columns 4q.. of a state row (zero past r).
__device__ __forceinline__ f4 load_cols4(const float* row, int r, int col) {
  if ((r & 3) == 0) {
    if (col < r) return *reinterpret_cast<const f4*>(row + col);
    return f4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  f4 v;
#pragma unroll
  for (int i = 0; i < 4; i++) v[i] = col + i < r ? row[col + i] : 0.0f;
  return v;
}

// RT: column tiles carrying a rotation (compile time; the tables are padded
// with the identity up to 8*RT complex pairs or 4*RT quaternion blocks).
template <int NT, int ROT, int CK, int RT>
__global__ __launch_bounds__(NTT, 1) void k_bwdt(
    Geo g, const bf16* __restrict__ xhat, const bf16* __restrict__ bhat, const bf16* __restrict__ da,
    const bf16* __restrict__ rot, const float* __restrict__ carry, const float* __restrict__ dm2,
    const float* __restrict__ dm1i, float* Db, bf16* d_xhat, bf16* d_bhat, bf16* d_da, bf16* d_rot) {
  constexpr int R = 16 * NT, K = ELL * CK, SP = R + 8, KP = K + 8;
  constexpr int NKT = K / 16;     // (j,c) tiles
  constexpr int KSR = NT / 2;     // K-steps over state columns
  constexpr int KH = NKT / 2;     // d_bhat (j,c) tiles per wave
  constexpr int CH = NT / 2;      // d_bhat column tiles per wave
  constexpr int NRC = ROT == 3 ? 4 : 2;  // rotation-gradient values per (t, rotated tile)
  constexpr int RTA = RT > 0 ? RT : 1;
  static_assert((ROT == 0) == (RT == 0) && RT <= NT, "rotated tiles");
  extern __shared__ __align__(16) unsigned char smem[];
  using L = LdsT<NT, CK>;
  bf16* Ss = (bf16*)(smem + L::Ss);
  bf16* bsT = (bf16*)(smem + L::bsT);
  bf16* bsY = (bf16*)(smem + L::bsY);
  bf16* xs = (bf16*)(smem + L::xs);
  float* LT = (float*)(smem + L::LT);
  float* s_a = (float*)(smem + L::a);
  float* s_d = (float*)(smem + L::d);
  float* rt = (float*)(smem + L::rot);
  bf16* Gs = (bf16*)(smem + L::Gs);
  bf16* dXs = (bf16*)(smem + L::dXs);
  float* red = (float*)(smem + L::red);
  f4* LWt = (f4*)(smem + L::lw);           // [LWE][64]
  f4* LYt = LWt + LWE * 64;               // [2*NKT][64]
  float* cst = (float*)(smem + L::cst);   // [carry | d_m1][row of the round][R]

  const int bh = blockIdx.x / g.NGR, gi = blockIdx.x % g.NGR;
  const int bi = bh / g.h, hi = bh % g.h;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, n = lane & 15, q = lane >> 4;
  constexpr int RTP = 16 * RT + 4;  // rotation table floats per token (padded)
  const int kh = w >> 1, ch = w & 1;  // this wave's d_bhat tiles: (j,c) half kh, column half ch

  // S = d_m2 + d_m2^T: rows internal columns, K-slots in col_of_slot order.
  {
    const float* D2 = dm2 + (size_t)bh * g.r * g.r;
    for (int idx = tid; idx < R * R; idx += NTT) {
      const int a = idx / R, s = idx % R;
      const int b = col_of_slot(s);
      float v = 0.0f;
      if (a < g.r && b < g.r) {
        const int pa = perm_rc(g, a), pb = perm_rc(g, b);
        v = D2[pa * g.r + pb] + D2[pb * g.r + pa];
      }
      Ss[a * SP + s] = (bf16)v;
    }
  }

  auto stage_x = [&](int nc, int pblk) {
    for (int idx = tid; idx < K * XPB; idx += NTT) {
      const int k = idx / XPB, pl = idx % XPB;
      const int j = k / CK, ci = k % CK;
      const int pos = nc * ELL + j;
      float v = 0.0f;
      if (pblk + pl < g.p && ci < g.c && pos < g.V)
        v = (float)xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pblk + pl];
      xs[pl * KP + k] = (bf16)v;
    }
  };
  auto flush_dx = [&](int nc, int pblk) {
    if (d_xhat == nullptr) return;
    const int rows = g.p - pblk < XPB ? g.p - pblk : XPB;
    for (int idx = tid; idx < K * rows; idx += NTT) {
      const int k = idx / rows, pl = idx % rows;
      const int j = k / CK, ci = k % CK;
      const int pos = nc * ELL + j;
      if (ci < g.c && pos < g.s)
        d_xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pblk + pl] = dXs[pl * KP + k];
    }
  };

  // The carry rows h_-(n)[p][:] and the d_m1 rows of a round (4 state rows)
  // travel through LDS: every thread fetches one float4 of them a round ahead
  // and stores it after the round's d_bhat work, off the rows' critical path.
  constexpr int CQ = 2 * 4 * R / 4;  // float4 pieces per round
  auto fetch_round = [&](int nc, int pr0) -> f4 {
    f4 v = f4{0.0f, 0.0f, 0.0f, 0.0f};
    if (tid < CQ) {
      const int arr = tid / (4 * R / 4), rest = tid % (4 * R / 4);
      const int rr = rest / (R / 4), col = 4 * (rest % (R / 4));
      const int pp = pr0 + rr;
      if (pp < g.p) {
        if (arr == 0) v = load_cols4(carry + (((size_t)bh * g.NK + nc) * g.p + pp) * g.r, g.r, col);
        else v = *reinterpret_cast<const f4*>(dm1i + ((size_t)bh * g.p + pp) * R + col);
      }
    }
    return v;
  };
  auto store_round = [&](f4 v) {
    if (tid < CQ) reinterpret_cast<f4*>(cst)[tid] = v;
  };

  const int n0 = gi * g.G;
  const int n1 = (n0 + g.G < g.NK) ? n0 + g.G : g.NK;
  const int nrounds = (g.p + 3) / 4;
  for (int nc = n0; nc < n1; nc++) {
    __syncthreads();
    // ---- chunk staging --------------------------------------------------
    if (tid < 64) {
      const int t = tid & 31;
      const int pos = nc * ELL + t;
      float v = 0.0f;
      if (tid < 32 && pos < g.V) v = (float)da[((size_t)bi * g.s + pos) * g.h + hi];
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
    for (int idx = tid; idx < K * R; idx += NTT) {
      const int k = idx / R, col = idx % R;
      const int j = k / CK, ci = k % CK;
      const int pos = nc * ELL + j;
      bf16 v = (bf16)0.0f;
      if (col < g.r && pos < g.V && ci < g.c)
        v = bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + perm_rc(g, col)];
      bsT[col * KP + k] = v;
      bsY[k * SP + slot_of_col(col)] = v;
    }
    if constexpr (ROT == 1) {
      for (int idx = tid; idx < ELL * 8 * RT; idx += NTT) {
        const int t = idx / (8 * RT), a = idx % (8 * RT);
        const int pos = nc * ELL + t;
        float th = 0.0f;
        if (a < g.A && pos < g.V) th = (float)rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + a];
        float sv, cv;
        sincosf(th, &sv, &cv);
        rt[t * RTP + 2 * a] = cv;
        rt[t * RTP + 2 * a + 1] = sv;
      }
    } else if constexpr (ROT == 3) {
      for (int idx = tid; idx < ELL * 16 * RT; idx += NTT) {
        const int t = idx / (16 * RT), e = idx % (16 * RT);
        const int pos = nc * ELL + t;
        float v = (e & 3) == 0 ? 1.0f : 0.0f;
        if ((e >> 2) < g.J && pos < g.V) v = (float)rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + e];
        rt[t * RTP + e] = v;
      }
    }
    stage_x(nc, 0);
    store_round(fetch_round(nc, 0));
    __syncthreads();
    for (int idx = tid; idx < ELL * ELL; idx += NTT) {
      const int j = idx / ELL, t = idx % ELL;
      LT[j * LTP + t] = (j <= t) ? expf(s_a[t] - s_a[j]) : 0.0f;
    }
    __syncthreads();

    // ---- per-lane chunk constants (LDS tables, this wave's lanes) ----------
    const int tv = g.V - nc * ELL;  // valid tokens of this chunk (>= 1)
    if (w == 0) {
      // W factors: L[16tt+n][j of the slots 32ks+8q..], flattened (tt*CK+ks)*(8/CK)+u
#pragma unroll
      for (int f = 0; f < 16; f++) {
        const int tt = f / 8, rest = f % 8, ks = rest / (8 / CK), u = rest % (8 / CK);
        reinterpret_cast<float*>(LWt + (f >> 2) * 64 + lane)[f & 3] =
            LT[((32 * ks + 8 * q) / CK + u) * LTP + 16 * tt + n];
      }
      // d_xhat factors: L[16tt+4q+i][j of (j,c) = 16kt+n], entry tt*NKT+kt
#pragma unroll
      for (int tt = 0; tt < 2; tt++)
#pragma unroll
        for (int kt = 0; kt < NKT; kt++) {
          f4 v;
#pragma unroll
          for (int i = 0; i < 4; i++) v[i] = LT[((16 * kt + n) / CK) * LTP + 16 * tt + 4 * q + i];
          LYt[(tt * NKT + kt) * 64 + lane] = v;
        }
    }
    __syncthreads();

    f4 dbacc[KH][CH];
#pragma unroll
    for (int a = 0; a < KH; a++)
#pragma unroll
      for (int b = 0; b < CH; b++) dbacc[a][b] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    float racc[2][RTA][NRC];
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
      for (int ct = 0; ct < RTA; ct++)
#pragma unroll
        for (int u = 0; u < NRC; u++) racc[tt][ct][u] = 0.0f;
    float gacc[2] = {0.0f, 0.0f};
    float cc[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; kt++) cc[kt] = 0.0f;

    for (int round = 0; round < nrounds; round++) {
      const int pr0 = 4 * round;
      const int pblk = pr0 - pr0 % XPB;
      if (round > 0 && pr0 % XPB == 0) {
        flush_dx(nc, pblk - XPB);
        __syncthreads();
        stage_x(nc, pblk);
        __syncthreads();
      }
      const int p = pr0 + w;
      const f4 pf = fetch_round(nc, pr0 + 4);  // next round's rows, stored after the d_bhat work
      // One state row, all columns and tokens; MASK zeroes d_c at tokens >= tv
      // (only the chunk holding valid_len needs it).
      auto row = [&](auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int pl = p - pblk;
        // carry row h_-[p][16ct+4q..] for the lane's columns, fetched first
        const float* hrow = cst + w * R;
        f4 hv[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ct++) hv[ct] = *reinterpret_cast<const f4*>(hrow + 16 * ct + 4 * q);
        // ---- W fragments: W[t][(j,c)] = L[t,j] xhat[(j,c)][p], t = 16tt+n ----
        u4 Wf[2][CK];
        {
          float xv[CK][8];
#pragma unroll
          for (int ks = 0; ks < CK; ks++) {
            const u4 x8 = *reinterpret_cast<const u4*>(xs + pl * KP + 32 * ks + 8 * q);
#pragma unroll
            for (int e = 0; e < 4; e++) {
              xv[ks][2 * e] = bf16_lo(x8[e]);
              xv[ks][2 * e + 1] = bf16_hi(x8[e]);
            }
          }
          float lw[16];
#pragma unroll
          for (int e4 = 0; e4 < 4; e4++) {
            const f4 v = LWt[e4 * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; i++) lw[4 * e4 + i] = v[i];
          }
#pragma unroll
          for (int tt = 0; tt < 2; tt++)
#pragma unroll
            for (int ks = 0; ks < CK; ks++)
#pragma unroll
              for (int e = 0; e < 8; e += 2) {
                const int b0 = (tt * CK + ks) * (8 / CK);
                Wf[tt][ks][e / 2] = pk_bf16(lw[b0 + e / CK] * xv[ks][e], lw[b0 + (e + 1) / CK] * xv[ks][e + 1]);
              }
        }
        // ---- states, transposed: h~^T[col][t] (carry added on read-out) ----
        f4 hT[NT][2];
#pragma unroll
        for (int ct = 0; ct < NT; ct++)
#pragma unroll
          for (int tt = 0; tt < 2; tt++) hT[ct][tt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < CK; ks++)
#pragma unroll
          for (int ct = 0; ct < NT; ct++) {
            const bf8 a = ld_frag(bsT + (16 * ct + n) * KP + 32 * ks + 8 * q);
#pragma unroll
            for (int tt = 0; tt < 2; tt++) {
              if (tt == 0 && 2 * ks >= CK) continue;  // tokens 0..15 see j <= 15 only
              hT[ct][tt] = MM<bf16>::mma(a, as_bf8(Wf[tt][ks]), hT[ct][tt]);
            }
          }
        // ---- carry, de-rotation in the lane; c^T (and h~^T) packed ---------
        u4 cP[KSR][2];
        u4 hP[ROT == 3 ? KSR : 1][2];
        const float dt[2] = {s_d[n], s_d[16 + n]};
#pragma unroll
        for (int ct = 0; ct < NT; ct++)
#pragma unroll
          for (int tt = 0; tt < 2; tt++) {
            f4 h;
#pragma unroll
            for (int i = 0; i < 4; i++) h[i] = hT[ct][tt][i] + dt[tt] * hv[ct][i];
            f4 c = h;
            const int t = 16 * tt + n;
            if constexpr (ROT == 1) {
              if (ct < RT) {
                const f4 r4 = *reinterpret_cast<const f4*>(rt + t * RTP + 16 * ct + 4 * q);
                c[0] = r4[0] * h[0] + r4[1] * h[1];
                c[1] = r4[0] * h[1] - r4[1] * h[0];
                c[2] = r4[2] * h[2] + r4[3] * h[3];
                c[3] = r4[2] * h[3] - r4[3] * h[2];
              }
            } else if constexpr (ROT == 3) {
              if (ct < RT) {
                const f4 Q = *reinterpret_cast<const f4*>(rt + t * RTP + 16 * ct + 4 * q);
                c[0] = Q[0] * h[0] - Q[1] * h[1] - Q[2] * h[2] - Q[3] * h[3];
                c[1] = Q[0] * h[1] + Q[1] * h[0] + Q[2] * h[3] - Q[3] * h[2];
                c[2] = Q[0] * h[2] - Q[1] * h[3] + Q[2] * h[0] + Q[3] * h[1];
                c[3] = Q[0] * h[3] + Q[1] * h[2] - Q[2] * h[1] + Q[3] * h[0];
              }
              hP[ROT == 3 ? ct >> 1 : 0][tt][2 * (ct & 1)] = pk_bf16(h[0], h[1]);
              hP[ROT == 3 ? ct >> 1 : 0][tt][2 * (ct & 1) + 1] = pk_bf16(h[2], h[3]);
            }
            cP[ct >> 1][tt][2 * (ct & 1)] = pk_bf16(c[0], c[1]);
            cP[ct >> 1][tt][2 * (ct & 1) + 1] = pk_bf16(c[2], c[3]);
          }
        // ---- d_c^T = S c^T + d_m1, rotation VJP, G, Y = G bhat^T ------------
        const float* dmrow = cst + (4 + w) * R;
        f4 Y[NKT][2];
#pragma unroll
        for (int kt = 0; kt < NKT; kt++)
#pragma unroll
          for (int tt = 0; tt < 2; tt++) Y[kt][tt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        bf16* Gw = Gs + (size_t)w * R * GSP;
#pragma unroll
        for (int ky = 0; ky < KSR; ky++) {
          u4 GP[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; h2++) {
            const int ct = 2 * ky + h2;
            const f4 dmv = *reinterpret_cast<const f4*>(dmrow + 16 * ct + 4 * q);
            f4 dc[2] = {dmv, dmv};
#pragma unroll
            for (int ks = 0; ks < KSR; ks++) {
              const bf8 a = ld_frag(Ss + (16 * ct + n) * SP + 32 * ks + 8 * q);
#pragma unroll
              for (int tt = 0; tt < 2; tt++) dc[tt] = MM<bf16>::mma(a, as_bf8(cP[ks][tt]), dc[tt]);
            }
#pragma unroll
            for (int tt = 0; tt < 2; tt++) {
              const int t = 16 * tt + n;
              f4 d = dc[tt];
              if constexpr (MASK) {
                if (t >= tv) d = f4{0.0f, 0.0f, 0.0f, 0.0f};
              }
              f4 hc;  // c (complex, none) or h~ (quaternion), from the packed fragments
              {
                const unsigned w0 = ROT == 3 ? hP[ROT == 3 ? ky : 0][tt][2 * h2] : cP[ky][tt][2 * h2];
                const unsigned w1 = ROT == 3 ? hP[ROT == 3 ? ky : 0][tt][2 * h2 + 1] : cP[ky][tt][2 * h2 + 1];
                hc[0] = bf16_lo(w0);
                hc[1] = bf16_hi(w0);
                hc[2] = bf16_lo(w1);
                hc[3] = bf16_hi(w1);
              }
              f4 G = d;
              if constexpr (ROT == 3) {
                if (ct < RT) {
                  const f4 Q = *reinterpret_cast<const f4*>(rt + t * RTP + 16 * ct + 4 * q);
                  G[0] = Q[0] * d[0] + Q[1] * d[1] + Q[2] * d[2] + Q[3] * d[3];
                  G[1] = Q[0] * d[1] - Q[1] * d[0] - Q[2] * d[3] + Q[3] * d[2];
                  G[2] = Q[0] * d[2] + Q[1] * d[3] - Q[2] * d[0] - Q[3] * d[1];
                  G[3] = Q[0] * d[3] - Q[1] * d[2] + Q[2] * d[1] - Q[3] * d[0];
                  racc[tt][ct < RT ? ct : 0][0] += d[0] * hc[0] + d[1] * hc[1] + d[2] * hc[2] + d[3] * hc[3];
                  racc[tt][ct < RT ? ct : 0][1] += -d[0] * hc[1] + d[1] * hc[0] - d[2] * hc[3] + d[3] * hc[2];
                  racc[tt][ct < RT ? ct : 0][2] += -d[0] * hc[2] + d[1] * hc[3] + d[2] * hc[0] - d[3] * hc[1];
                  racc[tt][ct < RT ? ct : 0][3] += -d[0] * hc[3] - d[1] * hc[2] + d[2] * hc[1] + d[3] * hc[0];
                }
                gacc[tt] += G[0] * hc[0] + G[1] * hc[1] + G[2] * hc[2] + G[3] * hc[3];
              } else {
                gacc[tt] += d[0] * hc[0] + d[1] * hc[1] + d[2] * hc[2] + d[3] * hc[3];
                if constexpr (ROT == 1) {
                  if (ct < RT) {
                    const f4 r4 = *reinterpret_cast<const f4*>(rt + t * RTP + 16 * ct + 4 * q);
                    racc[tt][ct < RT ? ct : 0][0] += d[0] * hc[1] - d[1] * hc[0];
                    racc[tt][ct < RT ? ct : 0][1] += d[2] * hc[3] - d[3] * hc[2];
                    G[0] = r4[0] * d[0] - r4[1] * d[1];
                    G[1] = r4[1] * d[0] + r4[0] * d[1];
                    G[2] = r4[2] * d[2] - r4[3] * d[3];
                    G[3] = r4[3] * d[2] + r4[2] * d[3];
                  }
                }
              }
              GP[tt][2 * h2] = pk_bf16(G[0], G[1]);
              GP[tt][2 * h2 + 1] = pk_bf16(G[2], G[3]);
            }
          }
          // Y[t][(j,c)] += sum over this K-step's columns of G[t][col] bhat[(j,c)][col]
#pragma unroll
          for (int kt = 0; kt < NKT; kt++) {
            const bf8 b = ld_frag(bsY + (16 * kt + n) * SP + 32 * ky + 8 * q);
#pragma unroll
            for (int tt = 0; tt < 2; tt++) Y[kt][tt] = MM<bf16>::mma(as_bf8(GP[tt]), b, Y[kt][tt]);
          }
          // G^T into the row's transpose buffer, [col][t]
#pragma unroll
          for (int tt = 0; tt < 2; tt++)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const int col = 32 * ky + 16 * (e >> 2) + 4 * q + (e & 3);
              unsigned short* gw = reinterpret_cast<unsigned short*>(Gw) + col * GSP + 16 * tt + n;
              const unsigned word = GP[tt][e / 2];
              gw[0] = (unsigned short)(word & 0xffffu);
              gw[GSP] = (unsigned short)(word >> 16);
            }
        }
        // ---- d_xhat[(j,c)][p] = sum_t L[t,j] Y[t][(j,c)] ----------------------
#pragma unroll
        for (int kt = 0; kt < NKT; kt++) {
          float v = 0.0f;
#pragma unroll
          for (int tt = 0; tt < 2; tt++) {
            const f4 ly = LYt[(tt * NKT + kt) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; i++) v += ly[i] * Y[kt][tt][i];
          }
          v = col4_sum(v);
          const int k = 16 * kt + n;
          if (q == 0) dXs[pl * KP + k] = (bf16)v;
          cc[kt] += v * (float)xs[pl * KP + k];
        }
      };
      if (p < g.p) {
        if (tv >= ELL) row(std::false_type{});
        else row(std::true_type{});
      }
      __syncthreads();  // the round's G transposes are complete
      float LB[KH][8];  // L[8q+e][j of (j,c) = 16(kh*KH+kt)+n]
#pragma unroll
      for (int kt = 0; kt < KH; kt++) {
        const float* src = LT + ((16 * (kh * KH + kt) + n) / CK) * LTP + 8 * q;
        const f4 l0 = *reinterpret_cast<const f4*>(src);
        const f4 l1 = *reinterpret_cast<const f4*>(src + 4);
#pragma unroll
        for (int e = 0; e < 4; e++) {
          LB[kt][e] = l0[e];
          LB[kt][e + 4] = l1[e];
        }
      }
      bf8 dA;  // A operand of local: row 0 = d_t over the K-slots t = 8q+e
#pragma unroll
      for (int e = 0; e < 8; e++) dA[e] = (bf16)(n == 0 ? s_d[8 * q + e] : 0.0f);
      // ---- d_bhat[(j,c)][col] += sum_t L[t,j] xhat[(j,c)][p] G[t][col]; local ----
#pragma unroll 1
      for (int rr = 0; rr < 4; rr++) {
        const int pp = pr0 + rr;
        if (pp >= g.p) break;
        const int pl = pp - pblk;
        u4 Ab[KH];
#pragma unroll
        for (int kt = 0; kt < KH; kt++) {
          const float xk = (float)xs[pl * KP + 16 * (kh * KH + kt) + n];
#pragma unroll
          for (int e = 0; e < 8; e += 2) Ab[kt][e / 2] = pk_bf16(LB[kt][e] * xk, LB[kt][e + 1] * xk);
        }
        const bf16* Gr = Gs + (size_t)rr * R * GSP;
        float* dbrow = Db + (((size_t)bh * g.NK + nc) * g.p + pp) * g.r;
#pragma unroll
        for (int cb = 0; cb < CH; cb++) {
          const int ct = ch * CH + cb;
          const bf8 gb = ld_frag(Gr + (16 * ct + n) * GSP + 8 * q);
#pragma unroll
          for (int kt = 0; kt < KH; kt++) dbacc[kt][cb] = MM<bf16>::mma(as_bf8(Ab[kt]), gb, dbacc[kt][cb]);
          if (kh == (rr & 1)) {
            const f4 lo = MM<bf16>::mma(dA, gb, f4{0.0f, 0.0f, 0.0f, 0.0f});
            const int col = 16 * ct + n;
            if (q == 0 && col < g.r) dbrow[col] = lo[0];
          }
        }
      }
      store_round(pf);
      __syncthreads();  // transposes consumed; next round's rows staged
    }
    flush_dx(nc, (nrounds - 1) * 4 - ((nrounds - 1) * 4) % XPB);

    // ---- chunk end: d_bhat through LDS, written row by row --------------------
    if (d_bhat != nullptr) {
      bf16* DBs = Gs;  // [K][SP]
#pragma unroll
      for (int kt = 0; kt < KH; kt++)
#pragma unroll
        for (int cb = 0; cb < CH; cb++)
#pragma unroll
          for (int i = 0; i < 4; i++)
            DBs[(16 * (kh * KH + kt) + 4 * q + i) * SP + 16 * (ch * CH + cb) + n] = (bf16)dbacc[kt][cb][i];
      __syncthreads();
      for (int idx = tid; idx < K * g.r; idx += NTT) {
        const int k = idx / g.r, ra = idx - k * g.r;
        const int j = k / CK, ci = k % CK;
        const int pos = nc * ELL + j;
        if (pos < g.s && ci < g.c)
          d_bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + ra] = DBs[k * SP + inv_perm_rc(g, ra)];
      }
      __syncthreads();
    }
    // ---- rotation gradient: fixed-order sum over the waves ---------------------
    if constexpr (ROT != 0) {
      if (d_rot != nullptr) {
        constexpr int rw = ROT == 3 ? 16 * RTA : 8 * RTA;
        float* RB = (float*)Gs;  // [w][t][rw]
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
          for (int ct = 0; ct < RTA; ct++) {
            const int t = 16 * tt + n;
            if constexpr (ROT == 1) {
              RB[(w * ELL + t) * rw + 8 * ct + 2 * q] = racc[tt][ct][0];
              RB[(w * ELL + t) * rw + 8 * ct + 2 * q + 1] = racc[tt][ct][1];
            } else {
#pragma unroll
              for (int u = 0; u < 4; u++) RB[(w * ELL + t) * rw + 4 * (4 * ct + q) + u] = racc[tt][ct][u];
            }
          }
        __syncthreads();
        for (int idx = tid; idx < ELL * g.RW; idx += NTT) {
          const int t = idx / g.RW, e = idx % g.RW;
          float s = 0.0f;
#pragma unroll
          for (int ww = 0; ww < NWT; ww++) s += RB[(ww * ELL + t) * rw + e];
          const int pos = nc * ELL + t;
          if (pos < g.s) d_rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + e] = (bf16)s;
        }
      }
    }
    // ---- d_da without the carry-cotangent terms --------------------------------
    float* rsum = red;                    // [w][q][t]
    float* csum = red + NWT * 4 * ELL;    // [w][(j,c)]
    float* ddv = csum + NWT * K;          // [t]
#pragma unroll
    for (int tt = 0; tt < 2; tt++) rsum[(w * 4 + q) * ELL + 16 * tt + n] = gacc[tt];
    if (q == 0) {
#pragma unroll
      for (int kt = 0; kt < NKT; kt++) csum[w * K + 16 * kt + n] = cc[kt];
    }
    __syncthreads();
    if (tid == 0) {
      float acc = 0.0f;
      for (int t = ELL - 1; t >= 0; t--) {
        float rtm = 0.0f, ctm = 0.0f;
        for (int e = 0; e < NWT * 4; e++) rtm += rsum[e * ELL + t];
        for (int ww = 0; ww < NWT; ww++)
          for (int ci = 0; ci < g.c; ci++) ctm += csum[ww * K + t * CK + ci];
        acc += rtm - ctm;
        ddv[t] = acc;
      }
    }
    __syncthreads();
    if (tid < ELL && d_da != nullptr) {
      const int pos = nc * ELL + tid;
      if (pos < g.s) d_da[((size_t)bi * g.s + pos) * g.h + hi] = (bf16)ddv[tid];
    }
  }
}

}  // namespace mom

// Forward main kernel in the transposed state layout (bf16 inputs, K <= 64).
//
// Same contract as k_fwd (source: burn-mamba "recalculated.rs" source page,
// moments_phys_fwd): per (b,h) chain, for a group of kernel chunks, the states
// h~ (chunk_states plus the boundary carry), the de-rotation c = M h~, and
// the partial moments m2 += c^T c and m1 += sum_t c over the group.
//
// The row work follows k_bwdt: eight waves, wave w computes state row
// 4*round + (w % 4) for the tokens of half w / 4, transposed (one token per
// lane, four consecutive state columns per lane), de-rotates in the lane and
// writes c^T through a per-row LDS transpose. After a barrier every wave
// reads the round's c fragments (tokens in registers) and accumulates a 2 x 4
// block of 16 x 16 m2 tiles on MFMA; m1 comes from the same fragments through
// an MFMA whose A operand selects one accumulator row per round.
#pragma once

#include "kernels_bwdt.h"

namespace mom {

template <int NT, int CK>
struct LdsF {
  static constexpr int R = 16 * NT, K = ELL * CK, KP = cf_pitch(K), GTP = R + 16;
  static constexpr size_t bsT = 0;                                    // bhat^T [col][(j,c)]
  static constexpr size_t xs = bsT + (size_t)R * KP * 2;              // xhat block [p][(j,c)]
  static constexpr size_t a = xs + (size_t)XPB * KP * 2;
  static constexpr size_t d = a + ELL * 4;
  static constexpr size_t lw = d + ELL * 4;                           // W factors [LWE][64] float4
  // carry rows and c blocks of a round, double-buffered by round parity
  static constexpr size_t cst = lw + (size_t)LWE * 64 * 16;           // carry rows [2][4][R]
  static constexpr size_t Gs = cst + (size_t)2 * 4 * R * 4;           // c blocks [2][4][token][column]
  static constexpr size_t rot = Gs + (size_t)2 * 4 * ELL * GTP * 2;
  static_assert(Gs % 16 == 0 && rot % 16 == 0 && lw % 16 == 0 && cst % 16 == 0, "aligned regions");
  // the rotation table (RT rotated tiles) comes last
  __host__ __device__ static size_t total(int RT, int) { return rot + (size_t)ELL * rt_pitch(16 * RT) * 4; }
  // with the state rows carried in LDS across the chain: [p][R] fp32 after the m1 table
  __host__ __device__ static size_t total_inc(int RT, int p) { return total(RT, p) + (size_t)p * R * 4; }
};

template <int NT, int ROT, int CK, int RT>
__global__ __launch_bounds__(NTT, 1) void k_fwdt(Geo g, const bf16* __restrict__ xhat,
                                                  const bf16* __restrict__ bhat, const bf16* __restrict__ da,
                                                  const bf16* __restrict__ rot, const float* __restrict__ carry,
                                                  const bf16* __restrict__ h0, float* m2part, float* m1part) {
  constexpr int R = 16 * NT, K = ELL * CK, KP = cf_pitch(K), GTP = R + 16;
  constexpr int RTP = rt_pitch(16 * RT);
  constexpr int MA = NT / 4, MB = NT / 2;  // m2 tiles per wave: MA row tiles x MB column tiles
  static_assert((ROT == 0) == (RT == 0) && RT <= NT && NT % 4 == 0, "tiling");
  using L = LdsF<NT, CK>;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* bsT = (bf16*)(smem + L::bsT);
  bf16* xs = (bf16*)(smem + L::xs);
  float* s_a = (float*)(smem + L::a);
  float* s_d = (float*)(smem + L::d);
  f4* LWt = (f4*)(smem + L::lw);
  float* cst = (float*)(smem + L::cst);
  bf16* Gs = (bf16*)(smem + L::Gs);
  float* rt = (float*)(smem + L::rot);

  const int bh = blockIdx.x / g.NGR, gi = blockIdx.x % g.NGR;
  const int bi = bh / g.h, hi = bh % g.h;
  g.V = chain_len(g, bi);  // this sequence's valid length (per-sequence lengths)
  // tid is refreshed through an empty asm at every chunk, so the per-thread
  // addresses of the chunk staging are recomputed per chunk rather than held
  // (spilled) across the rounds
  int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform in the wave
  const int lane = tid & 63, n = lane & 15, q = lane >> 4;
  const int u = w & 3, tt = w >> 2;
  const int t = 16 * tt + n;
  const int ta0 = MA * (w >> 1), tb0 = MB * (w & 1);  // this wave's m2 tiles

  // carry == nullptr: one group per chain, and the state entering each chunk is
  // carried in LDS: the rows start at h0 and the lanes holding the chunk's last
  // token replace them with the state there, h_-(n+1) = h_{n, last}
  const bool inc = carry == nullptr;
  float* carryL = (float*)(smem + L::total(RT, g.p));  // [p][R]
  if (inc) {
    for (int idx = tid; idx < g.p * R; idx += NTT) {
      const int pp = idx / R, col = idx % R;
      carryL[idx] = (h0 != nullptr && col < g.r) ? (float)h0[((size_t)bh * g.p + pp) * g.r + perm_rc(g, col)] : 0.0f;
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
  // carry rows of a round through LDS, fetched a round ahead (one float4 per thread)
  static_assert(R % 64 == 0, "whole waves fetch the carry rows");
  auto fetch_round = [&](int nc, int pr0) -> f4 {
    f4 v = f4{0.0f, 0.0f, 0.0f, 0.0f};
    if (w < R / 64) {
      const int rr = tid / (R / 4), col = 4 * (tid % (R / 4));
      const int pp = pr0 + rr;
      if (pp < g.p)
        v = inc ? *reinterpret_cast<const f4*>(carryL + (size_t)pp * R + col)
                : load_cols4(carry + (((size_t)bh * g.NK + nc) * g.p + pp) * g.r, g.r, col, R);
    }
    return v;
  };
  auto store_round = [&](f4 v, int buf) {
    if (w < R / 64) reinterpret_cast<f4*>(cst + (size_t)buf * 4 * R)[tid] = v;
  };

  f4 m2acc[MA][MB];
#pragma unroll
  for (int a = 0; a < MA; a++)
#pragma unroll
    for (int b = 0; b < MB; b++) m2acc[a][b] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  // m1 stays in MFMA accumulators: wave w adds row 4*round + w/2 of every round
  // (its column tiles tb0..) into accumulator row round % 16 of round tile
  // round / 16, through an A operand that is one in that row only
  constexpr int M1T = 2;  // round tiles: 32 rounds, state rows <= 128
  f4 m1acc[M1T][MB];
#pragma unroll
  for (int a = 0; a < M1T; a++)
#pragma unroll
    for (int b = 0; b < MB; b++) m1acc[a][b] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  auto m1_add = [&](int round, const bf8 (&fbr)[MB]) {
    const bf16 one = (bf16)(n == (round & 15) ? 1.0f : 0.0f);
    bf8 sel;
#pragma unroll
    for (int e = 0; e < 8; e++) sel[e] = one;
    if (round < 16) {
#pragma unroll
      for (int b = 0; b < MB; b++) m1acc[0][b] = MM<bf16>::mma(sel, fbr[b], m1acc[0][b]);
    } else {
#pragma unroll
      for (int b = 0; b < MB; b++) m1acc[1][b] = MM<bf16>::mma(sel, fbr[b], m1acc[1][b]);
    }
  };

  const int n0 = gi * g.G;
  const int n1 = (n0 + g.G < g.NK) ? n0 + g.G : g.NK;
  const int nrounds = (g.p + 3) / 4;
  using WS = WideStage<NT, CK, ROT, RT, false>;
  const bool wide = WS::usable(g);
  WS wst;
  float dav = 0.0f;
  // the global loads of a chunk's inputs, all issued before the first is used
  auto load_chunk = [&](int ncl) {
    dav = 0.0f;
    if (tid < 32 && ncl * ELL + tid < g.V) dav = (float)da[((size_t)bi * g.s + ncl * ELL + tid) * g.h + hi];
    if (wide) wst.load(g, xhat, bhat, rot, ncl, bi, hi, tid);
  };
  for (int nc = n0; nc < n1; nc++) {
    asm volatile("" : "+v"(tid));
    load_chunk(nc);  // in flight while the waves meet at the barrier
    __syncthreads();
    // ---- chunk staging
    if (tid < 64) {
      const int tk = tid & 31;
      float v = dav;
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
    if (wide) {
      wst.store(g, bsT, nullptr, xs, rt, tid);
    } else {
      for (int idx = tid; idx < K * R; idx += NTT) {
        const int k = idx / R, col = idx % R;
        const int j = k / CK, ci = k % CK;
        const int pos = nc * ELL + j;
        bf16 v = (bf16)0.0f;
        if (col < g.r && pos < g.V && ci < g.c)
          v = bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + perm_rc(g, col)];
        bsT[col * KP + k] = v;
      }
      if constexpr (ROT == 1) {
        for (int idx = tid; idx < ELL * 8 * RT; idx += NTT) {
          const int tk = idx / (8 * RT), a = idx % (8 * RT);
          const int pos = nc * ELL + tk;
          float th = 0.0f;
          if (a < g.A && pos < g.V) th = (float)rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + a];
          float sv, cv;
          sincosf(th, &sv, &cv);
          rt[tk * RTP + 2 * a] = cv;
          rt[tk * RTP + 2 * a + 1] = sv;
        }
      } else if constexpr (ROT == 3) {
        for (int idx = tid; idx < ELL * 16 * RT; idx += NTT) {
          const int tk = idx / (16 * RT), e = idx % (16 * RT);
          const int pos = nc * ELL + tk;
          float v = (e & 3) == 0 ? 1.0f : 0.0f;
          if ((e >> 2) < g.J && pos < g.V) v = (float)rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + e];
          rt[tk * RTP + e] = v;
        }
      }
      stage_x(nc, 0);
    }
    store_round(fetch_round(nc, 0), 0);
    __syncthreads();
    const int tv = g.V - nc * ELL;  // valid tokens of this chunk (<= 0: none)
    if (w < LWE) {
      // W factor entry w: L[t][j] = exp(a_t - a_j) for j <= t (else 0) at the
      // four flattened f = (h*CK+ks)*(8/CK)+v, t = 16h + n, j of slot 32ks+8q+v
      f4 v;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int f = 4 * w + i;
        const int hh = f / 8, rest = f % 8, ks = rest / (8 / CK), vv = rest % (8 / CK);
        const int j = (32 * ks + 8 * q) / CK + vv, tk = 16 * hh + n;
        v[i] = (j <= tk) ? expf(s_a[tk] - s_a[j]) : 0.0f;
      }
      LWt[w * 64 + lane] = v;
    }
    __syncthreads();
    const float dtl = s_d[t];
    const bool live = t < tv;  // tokens past valid_len contribute nothing

    for (int round = 0; round < nrounds; round++) {
      const int pr0 = 4 * round;
      const int pblk = pr0 - pr0 % XPB;
      if (round > 0 && pr0 % XPB == 0) {
        if (wide) {
          wst.load_x(g, xhat, nc, pblk, bi, hi, tid);
          wst.store_x(xs, tid);
        } else {
          stage_x(nc, pblk);
        }
        __syncthreads();
      }
      const int p = pr0 + u;
      bf16* Gsb = Gs + (size_t)(round & 1) * 4 * ELL * GTP;  // this round's c blocks
      const f4 pf = fetch_round(nc, pr0 + 4);
      if (p < g.p) {
        const int pl = p - pblk;
        // ---- W fragment --------------------------------------------------------
        u4 Wf[CK];
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
          float lw[8];
#pragma unroll
          for (int e4 = 0; e4 < 2; e4++) {
            const f4 v = LWt[(2 * tt + e4) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; i++) lw[4 * e4 + i] = v[i];
          }
#pragma unroll
          for (int ks = 0; ks < CK; ks++)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const int b0 = ks * (8 / CK);
              Wf[ks][e / 2] = pk_bf16(lw[b0 + e / CK] * xv[ks][e], lw[b0 + (e + 1) / CK] * xv[ks][e + 1]);
            }
        }
        // ---- states, transposed ---------------------------------------------------
        f4 hT[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ct++) hT[ct] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        const int nks = tt == 0 ? (CK + 1) / 2 : CK;
#pragma unroll
        for (int ks = 0; ks < CK; ks++) {
          if (ks < nks) {
            // the K-step's fragments are all requested before the first MFMA
            bf8 af[NT];
#pragma unroll
            for (int ct = 0; ct < NT; ct++) af[ct] = ld_frag(bsT + (16 * ct + n) * KP + 32 * ks + 8 * q);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ct = 0; ct < NT; ct++) hT[ct] = MM<bf16>::mma(af[ct], as_bf8(Wf[ks]), hT[ct]);
          }
        }
        // ---- carry, de-rotation, c^T into the row's transpose buffer --------------
        const float* hrow = cst + ((size_t)(round & 1) * 4 + u) * R;
        bf16* Gw = Gsb + ((size_t)u * ELL + t) * GTP + 4 * gpiece(q, t);  // this lane's piece of its token row
        f4 hl[NT];  // the state row at this lane's token (kept for the last token's carry)
        // carry and rotation rows pipelined one column tile ahead
        f4 hvn = *reinterpret_cast<const f4*>(hrow + 4 * q);
        f4 rtn = RT > 0 ? *reinterpret_cast<const f4*>(rt + t * RTP + 4 * q) : f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ct = 0; ct < NT; ct++) {
          const f4 hv = hvn, rtc = rtn;
          if (ct + 1 < NT) {
            hvn = *reinterpret_cast<const f4*>(hrow + 16 * (ct + 1) + 4 * q);
            if (ct + 1 < RT) rtn = *reinterpret_cast<const f4*>(rt + t * RTP + 16 * (ct + 1) + 4 * q);
          }
          f4 h;
#pragma unroll
          for (int i = 0; i < 4; i++) h[i] = hT[ct][i] + dtl * hv[i];
          hl[ct] = h;
          f4 c = h;
          if constexpr (ROT == 1) {
            if (ct < RT) {
              const f4 r4 = rtc;
              c[0] = r4[0] * h[0] + r4[1] * h[1];
              c[1] = r4[0] * h[1] - r4[1] * h[0];
              c[2] = r4[2] * h[2] + r4[3] * h[3];
              c[3] = r4[2] * h[3] - r4[3] * h[2];
            }
          } else if constexpr (ROT == 3) {
            if (ct < RT) {
              const f4 Q = rtc;
              c[0] = Q[0] * h[0] - Q[1] * h[1] - Q[2] * h[2] - Q[3] * h[3];
              c[1] = Q[0] * h[1] + Q[1] * h[0] + Q[2] * h[3] - Q[3] * h[2];
              c[2] = Q[0] * h[2] - Q[1] * h[3] + Q[2] * h[0] + Q[3] * h[1];
              c[3] = Q[0] * h[3] + Q[1] * h[2] - Q[2] * h[1] + Q[3] * h[0];
            }
          }
          const unsigned w0 = live ? pk_bf16(c[0], c[1]) : 0u;
          const unsigned w1 = live ? pk_bf16(c[2], c[3]) : 0u;
          const unsigned pr[2] = {w0, w1};  // columns 16ct+4q..
          *reinterpret_cast<unsigned long long*>(Gw + 16 * ct) = __builtin_bit_cast(unsigned long long, pr);
        }
        if (inc && t == ELL - 1) {
#pragma unroll
          for (int ct = 0; ct < NT; ct++) *reinterpret_cast<f4*>(carryL + (size_t)p * R + 16 * ct + 4 * q) = hl[ct];
        }
      }
      // the next round's carry rows go to the other buffer: its last readers
      // (the row work two rounds back) are behind the previous barrier
      store_round(pf, (round + 1) & 1);
      __syncthreads();  // the round's c blocks are complete
      // No barrier closes the round: a wave done with this m2 work starts the
      // next round's rows, which write the other c buffer; the next barrier
      // orders this round's reads before the writes two rounds on.
      // ---- m2 += c^T c over the round's rows and tokens; m1 row sums -------------
      // all four rows present: their fragments are loaded up front (one LDS
      // latency for the round); otherwise row by row
      const int nrr = g.p - pr0 < 4 ? g.p - pr0 : 4;
      // the second token half has the longer row work ahead of it: its waves get
      // issue priority for their m2 work, so the first half's m2 work fills in
      // under their row work instead of the other way round
      if (tt == 1) __builtin_amdgcn_s_setprio(2);
      if (nrr == 4) {
        bf8 fa[4][MA], fb[4][MB];
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
          const bf16* Gr = Gsb + (size_t)rr * ELL * GTP;
#pragma unroll
          for (int a = 0; a < MA; a++) fa[rr][a] = ld_tok_frag<GTP>(Gr, ta0 + a, lane);
#pragma unroll
          for (int b = 0; b < MB; b++) fb[rr][b] = ld_tok_frag<GTP>(Gr, tb0 + b, lane);
        }
#pragma unroll
        for (int rr = 0; rr < 4; rr++)
#pragma unroll
          for (int a = 0; a < MA; a++)
#pragma unroll
            for (int b = 0; b < MB; b++) m2acc[a][b] = MM<bf16>::mma(fa[rr][a], fb[rr][b], m2acc[a][b]);
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++)  // m1 of row w / 2 over this wave's column tiles
          if (r4 == (w >> 1)) m1_add(round, fb[r4]);
      }
#pragma unroll 1
      for (int rr = 0; rr < nrr && nrr < 4; rr++) {
        const int pp = pr0 + rr;
        const bf16* Gr = Gsb + (size_t)rr * ELL * GTP;
        bf8 fa[MA], fb[MB];
#pragma unroll
        for (int a = 0; a < MA; a++) fa[a] = ld_tok_frag<GTP>(Gr, ta0 + a, lane);
#pragma unroll
        for (int b = 0; b < MB; b++) fb[b] = ld_tok_frag<GTP>(Gr, tb0 + b, lane);
#pragma unroll
        for (int a = 0; a < MA; a++)
#pragma unroll
          for (int b = 0; b < MB; b++) m2acc[a][b] = MM<bf16>::mma(fa[a], fb[b], m2acc[a][b]);
        if ((w >> 1) == rr) m1_add(round, fb);  // m1 of this row over this wave's column tiles
      }
      __builtin_amdgcn_s_setprio(0);
    }
  }
  __syncthreads();
  // ---- the group's partials: m2 and m1 tiles straight out of the accumulators --
  float* m2o = m2part + ((size_t)bh * g.NGR + gi) * R * R;
#pragma unroll
  for (int a = 0; a < MA; a++)
#pragma unroll
    for (int b = 0; b < MB; b++)
#pragma unroll
      for (int i = 0; i < 4; i++) m2o[(16 * (ta0 + a) + 4 * q + i) * R + 16 * (tb0 + b) + n] = m2acc[a][b][i];
  float* m1o = m1part + ((size_t)bh * g.NGR + gi) * g.p * R;
#pragma unroll
  for (int a = 0; a < M1T; a++)
#pragma unroll
    for (int b = 0; b < MB; b++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int pp = 4 * (16 * a + 4 * q + i) + (w >> 1);  // row of round 16a + 4q + i
        if (pp < g.p) m1o[(size_t)pp * R + 16 * (tb0 + b) + n] = m1acc[a][b][i];
      }
}

}  // namespace mom

// Backward main kernel in the transposed state layout (bf16 inputs, K <= 64).
//
// Sources: burn-mamba "recalculated.rs" and "backward.rs" source pages,
// moments_phys_bwd and its module doc "Gradient math". Per (b,h) chain a
// workgroup owns a group of consecutive kernel chunks and walks them from the
// last to the first. For each chunk it recomputes the states, applies the
// de-rotation and forms G = M^T d_c; the cotangent D(n+1) of the state leaving
// the chunk (computed by the previous step of the walk, zero at the group's
// end) is added to G at the chunk's last token. Then
//   D(n) = sum_t d_t G[t]            (the carry-cotangent recurrence, written
//                                     to Db[n] for the next step of the walk)
// and d_xhat, d_bhat, d_da and d_rot of the chunk follow from G. d_da: with
// a_t = cumsum da inside L and d, and E[t][j] = L[t,j] <G[t], W_j> where
// <G[t], W_j> = sum_c sum_p xhat[j,c,p] Y_p[t,(j,c)],
//   d_da_s = sum_{t>=s} d_t <G[t], h_->  +  sum_{j<s<=t} E[t][j]
//          = sum_{t>=s} d_t <G[t], h_->  +  sum_{s'<s} (C[s'] - Rw[s']),
// C[j] = sum_t E[t][j] (column sums: sum_c sum_p xhat d_xhat) and Rw[t] =
// sum_j E[t][j] (row sums). Both sums take the same E values, so the large
// diagonal terms E[t][t], which the reverse-cumsum identity subtracts between
// two differently rounded quantities, cancel up to fp32 rounding only. They are exact
// except for the cotangent entering at the group's end, which the group fix-up
// adds afterwards (k_gscan, k_gfix).
//
// Layout. The states are computed transposed, h~^T[col][t] = bhat^T W^T with
// W[t][(j,c)] = L[t,j] xhat[j,c,p], so an accumulator lane holds one token and
// four consecutive state columns: complex pairs and quaternion 4-blocks sit in
// one lane's registers and the rotation, its transpose and its gradient need
// no lane exchange. The packed c^T fragments feed d_c^T = S c^T directly
// (S = d_m2 + d_m2^T). G^T is the A operand of Y = G bhat^T, from which
// d_xhat[(j,c)] = sum_t L[t,j] Y[t,(j,c)]. The token contractions that need
// tokens in registers (d_bhat over (t,p), local over t) read G through a small
// per-row LDS transpose.
//
// Work split. Eight waves, two per SIMD. Each round covers four state rows;
// wave w handles row 4*round + (w % 4) for the tokens of half w / 4 (0..15 or
// 16..31): nothing in the row computation couples the two halves except the
// token sum of d_xhat, whose two partials meet in LDS. After a barrier the
// eight waves accumulate d_bhat for the round's rows, each owning a block of
// the (j,c) x column tiles.
//
// Four channels are walked as token pairs (pair token 2t: channels 0, 1 of token
// t; 2t+1: channels 2, 3, whose state is token t's). Only odd pair tokens carry
// moments, so the pair form (PO) puts the even pair tokens in slots 0..15 and
// the odd ones in 16..31 and gives every wave the odd slots: a round then takes
// eight state rows (the first half's waves rows 4..7), and each G block holds
// two rows, one per half of its slots, for the d_bhat contraction.
#pragma once

#include "kernels.h"

namespace mom {

constexpr int NWT = 8;          // waves of k_bwdt
constexpr int NTT = 64 * NWT;   // threads of k_bwdt
constexpr int LTP = 36;         // row pitch of LT[j][t] (floats)
constexpr int XPB = 32;         // state rows per staged xhat block

// Token slots of a chunk. A chain walked in token pairs (four channels: pair
// token 2t holds channels 0, 1 of token t, pair token 2t+1 channels 2, 3; the
// PO kernels) puts its even pair tokens in slots 0..15 and its odd ones in slots
// 16..31: slot s holds pair token 2 (s mod 16) + s / 16. Otherwise slot = token.
template <bool PO>
__host__ __device__ __forceinline__ int slot_tok(int s) { return PO ? 2 * (s & 15) + (s >> 4) : s; }
template <bool PO>
__host__ __device__ __forceinline__ int tok_slot(int t) { return PO ? 16 * (t & 1) + (t >> 1) : t; }

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

// gfx950 transposing LDS read of four 16-bit values: within each group of 16
// lanes, lane j receives element j % 4 of the 8-byte pieces addressed by lanes
// 4r + j / 4 of its group, r = 0..3 in that order.
typedef short s4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s4 lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)p);
}

// Row pitch (elements of 2 bytes) of the LDS operand tiles: the smallest
// n' >= n with n' = 16 (mod 64). Row-per-lane 16-byte operand reads, and the
// transposing reads below, are free of bank conflicts at such pitches on
// gfx950 (72 or 136 are two-way conflicted).
__host__ __device__ constexpr int cf_pitch(int n) { return n + ((16 - n % 64) + 64) % 64; }
// Row pitch (floats) of the rotation tables: >= n and = 8 (mod 32), the same
// rule for 4-byte elements.
__host__ __device__ constexpr int rt_pitch(int n) { return n + ((8 - n % 32) + 32) % 32; }

// [token][column] blocks of G (and of c in the forward) store the 4-column
// pieces of each 16-column tile swizzled by token: logical piece v of token t
// sits at piece v ^ ((t >> 2) & 3). Writes of a lane's piece and the
// transposing reads are then both free of bank conflicts (pitch R + 16).
__device__ __forceinline__ int gpiece(int v, int t) { return v ^ ((t >> 2) & 3); }

// MFMA operand over the 32 tokens of a chunk from a [token][column] block of
// pitch P (bf16): lane (q, n) gets state column 16ct + n at K-slots 8q+e =
// tokens tslot(8q+e), i.e. 4q+e (e < 4) and 16+4q+e-4. Each of the two reads
// covers four tokens; lane 4r+s of a group addresses token 4q+r (+16), logical
// columns 16ct+4s.. (piece s, swizzled by gpiece; tokens t and t+16 share it).
template <int P>
__device__ __forceinline__ bf8 ld_tok_frag(const bf16* blk, int ct, int lane) {
  const int row = 4 * (lane >> 4) + ((lane >> 2) & 3);
  const bf16* p0 = blk + row * P + 4 * gpiece(lane & 3, row) + 16 * ct;
  const s4 a = lds_read_tr16(p0), b = lds_read_tr16(p0 + 16 * P);
  const s4 v[2] = {a, b};
  return __builtin_bit_cast(bf8, v);
}

// Column tiles of 16 internal state columns that carry a rotation, rounded up
// to a power of two (0: no rotation). Complex pairs 8 per tile, quaternion
// blocks 4 per tile. The rotation tables of k_bwdt hold RT tiles per token,
// padded with the identity: complex [t][8RT][cos, sin], quaternion [t][4RT][4],
// each token row padded to rt_pitch floats.
__host__ __device__ __forceinline__ int rot_tiles(const Geo& g) {
  const int need = (g.rot_kind == 1 || g.rot_kind == 2) ? (g.A + 7) / 8 : g.rot_kind == 3 ? (g.J + 3) / 4 : 0;
  if (need == 0) return 0;
  int rt = 1;
  while (rt < need) rt *= 2;
  return rt;
}

// LDS plan: every region at a compile-time offset (so LDS addresses fold into
// instruction offsets); the rotation table, sized by RT, comes last.
// Per-lane chunk constants are float4 rows interleaved by lane ([entry][lane]
// of 16 bytes, conflict-free): LWE entries of W factors, 2*NKT of d_xhat
// factors.
// PO (pair mode, odd pair tokens): eight state rows per round, every wave on the
// sixteen odd token slots; the tables of the first token half are not needed and
// the rotation table holds the odd slots only.
constexpr int LWE = 4;
template <int NT, int CK, bool PO = false>
struct LdsT {
  static constexpr int R = 16 * NT, K = ELL * CK, SP = cf_pitch(R), KP = cf_pitch(K), GTP = R + 16;
  static constexpr int RR = PO ? 8 : 4;                  // state rows of a round
  static constexpr int LWN = PO ? LWE / 2 : LWE;         // W-factor entries per lane
  static constexpr int LYN = (PO ? 1 : 2) * (K / 16);    // d_xhat factor entries per lane
  static constexpr int RTK = PO ? ELL / 2 : ELL;         // token slots of the rotation table
  static constexpr size_t Ss = 0;                                     // S rows, K-slot order
  static constexpr size_t bsT = Ss + (size_t)R * SP * 2;              // bhat^T [col][(j,c)]
  static constexpr size_t bsY = bsT + (size_t)R * KP * 2;             // bhat [(j,c)][col slot]
  static constexpr size_t xs = bsY + (size_t)K * SP * 2;              // xhat block [p][(j,c)]
  static constexpr size_t dXs = xs + (size_t)XPB * KP * 2;            // d_xhat block [p][(j,c)]
  static constexpr size_t LT = dXs + (size_t)XPB * KP * 2;            // L^T [j][t]
  static constexpr size_t a = LT + (size_t)ELL * LTP * 4;
  static constexpr size_t d = a + ELL * 4;
  static constexpr size_t lw = d + ELL * 4;
  // rows of a round: carry [2 buffers][RR][R], then d_m1 [RR][R] and D+ [RR][R]
  static constexpr size_t cst = lw + (size_t)(LWN + LYN) * 64 * 16;
  static constexpr size_t dxp = cst + (size_t)4 * RR * R * 4;                  // d_xhat partials [8 wave slots][K]
  static constexpr size_t red = dxp + (size_t)2 * 4 * K * 4;
  static constexpr size_t nred = (size_t)NWT * 4 * 16 + NWT * 16 + RR * K + ELL;  // floats of red
  // G of the round's rows, [row][token][column] (pitch GTP); at chunk end the
  // d_bhat tile and the rotation-gradient reduction reuse the space
  static constexpr size_t gs0 = (size_t)4 * ELL * GTP * 2;                     // G blocks
  static constexpr size_t gs1 = (size_t)K * SP * 2;                            // d_bhat tile
  static constexpr size_t gsb = gs0 > gs1 ? gs0 : gs1;
  static constexpr size_t Gs = red + nred * 4;
  static constexpr size_t rot = Gs + gsb;
  static_assert(Gs % 16 == 0 && rot % 16 == 0 && lw % 16 == 0 && cst % 16 == 0, "aligned regions");
  // rotation table (RT rotated tiles), rt_pitch(16*RT) entries per token: fp32
  // cos/sin pairs for complex modes, the bf16 input quaternions as they are
  __host__ __device__ static size_t total(int RT, int rot_kind) {
    return rot + (size_t)RTK * rt_pitch(16 * RT) * (rot_kind == 3 ? 2 : 4);
  }
  // the rotation-gradient reduction [wave][16 tokens][8RT or 16RT] runs in at
  // most four passes over the G space
  __host__ __device__ static bool fits(int rot_kind, int RT) {
    const size_t rw = rot_kind == 3 ? (size_t)16 * RT : (size_t)8 * RT;
    const size_t full = (size_t)NWT * 16 * rw * 4;
    return full <= gsb || (RT >= 2 && full <= 2 * gsb) || (RT >= 4 && full <= 4 * gsb);
  }
};

// Chunk inputs staged into LDS with wide loads. Used when every caller row is
// 16-byte aligned (r and p multiples of 8; an even number of angles or of
// quaternion blocks): each thread issues all of its global loads for the
// chunk before its first LDS store, so a chunk waits for memory once instead
// of once per element. BY also fills the bhat tile in (j,c)-row order used by
// the backward. Rows past r, tokens past valid_len and channels past c are
// written as zeros (identity rotations), like the element-wise staging.
template <int NT, int CK, int ROT, int RT, bool BY, bool PO = false>
struct WideStage {
  static constexpr int TK = PO ? ELL / 2 : ELL, T0 = PO ? ELL / 2 : 0;  // rotation-table slots: T0.. (TK of them)
  static constexpr int R = 16 * NT, K = ELL * CK, KP = cf_pitch(K), SP = cf_pitch(R), RTP = rt_pitch(16 * RT);
  static constexpr int NBU = K * R / 8, NBL = (NBU + NTT - 1) / NTT;   // bhat: 8 columns per load
  static constexpr int NXU = K * XPB / 8, NXL = (NXU + NTT - 1) / NTT; // xhat block: 8 rows per load
  // rotation: complex 2 angles per load (4RT pairs per token), quaternion 2 blocks per load
  static constexpr int NRU = ROT == 1 ? TK * 4 * RT : ROT == 3 ? TK * 2 * RT : 0;
  static constexpr int NRL = NRU > 0 ? (NRU + NTT - 1) / NTT : 1;
  u4 bv[NBL];
  u4 xv[NXL];
  unsigned r1[NRL];
  u4 r3[NRL];

  __device__ static bool usable(const Geo& g) {
    const bool rot_ok = ROT == 0 || (ROT == 1 ? (g.A % 2) == 0 : (g.J % 2) == 0);
    return (g.r % 8) == 0 && (g.p % 8) == 0 && rot_ok;
  }
  // Work items run over (j,c) fastest: the lanes of a wave then write
  // consecutive (j,c) of one LDS tile column (free of bank conflicts; with
  // the columns fastest, 16 lanes would hit one bank).
  __device__ void load_x(const Geo& g, const bf16* __restrict__ xhat, int nc, int pblk, int bi, int hi, int tid) {
#pragma unroll
    for (int i = 0; i < NXL; i++) {
      const int idx = tid + i * NTT;
      const int k = idx % K, c8 = idx / K;
      const int j = k / CK, ci = k % CK, pos = nc * ELL + slot_tok<PO>(j);
      xv[i] = u4{0u, 0u, 0u, 0u};
      if (idx < NXU && pblk + 8 * c8 < g.p && ci < g.c && pos < g.V)
        xv[i] = *reinterpret_cast<const u4*>(xhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pblk + 8 * c8);
    }
  }
  __device__ void store_x(bf16* xs, int tid) const {
#pragma unroll
    for (int i = 0; i < NXL; i++) {
      const int idx = tid + i * NTT;
      if (idx >= NXU) continue;
      const int k = idx % K, c8 = idx / K;
      const bf16* v = reinterpret_cast<const bf16*>(&xv[i]);
#pragma unroll
      for (int e = 0; e < 8; e++) xs[(8 * c8 + e) * KP + k] = v[e];
    }
  }
  __device__ void load(const Geo& g, const bf16* __restrict__ xhat, const bf16* __restrict__ bhat,
                       const bf16* __restrict__ rot, int nc, int bi, int hi, int tid) {
#pragma unroll
    for (int i = 0; i < NBL; i++) {
      const int idx = tid + i * NTT;
      const int k = idx % K, c8 = idx / K;
      const int j = k / CK, ci = k % CK, pos = nc * ELL + slot_tok<PO>(j);
      bv[i] = u4{0u, 0u, 0u, 0u};
      if (idx < NBU && 8 * c8 < g.r && ci < g.c && pos < g.V)
        bv[i] = *reinterpret_cast<const u4*>(bhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + 8 * c8);
    }
    load_x(g, xhat, nc, 0, bi, hi, tid);
#pragma unroll
    for (int i = 0; i < NRL; i++) {
      const int idx = tid + i * NTT;
      if constexpr (ROT == 1) {
        const int tk = idx / (4 * RT), a2 = idx % (4 * RT), pos = nc * ELL + slot_tok<PO>(T0 + tk);
        r1[i] = 0u;
        if (idx < NRU && 2 * a2 < g.A && pos < g.V)
          r1[i] = *reinterpret_cast<const unsigned*>(rot + (((size_t)bi * g.s + pos) * g.h + hi) * g.RW + 2 * a2);
      } else if constexpr (ROT == 3) {
        const int tk = idx / (2 * RT), e8 = idx % (2 * RT), pos = nc * ELL + slot_tok<PO>(T0 + tk);
        const unsigned one = 0x3f80u;  // bf16 1.0: identity quaternions (1, 0, 0, 0)
        r3[i] = u4{one, 0u, one, 0u};
        if (idx < NRU && 2 * e8 < g.J && pos < g.V)
          r3[i] = *reinterpret_cast<const u4*>(rot + (((size_t)bi * g.s + pos) * g.h + hi) * g.RW + 8 * e8);
      }
    }
  }
  __device__ void store(const Geo& g, bf16* bsT, bf16* bsY, bf16* xs, void* rtv, int tid) const {
#pragma unroll
    for (int i = 0; i < NBL; i++) {
      const int idx = tid + i * NTT;
      if (idx >= NBU) continue;
      const int k = idx % K, c8 = idx / K;
      const bf16* v = reinterpret_cast<const bf16*>(&bv[i]);
      if (!g.half) {
        // internal columns 8c8.. = caller columns: their K-slots in the (j,c)-row
        // tile are two runs of four, 32ks + 8q + 4h + (0..3) for q = c8 % 2 * 2,
        // +1 (columns 16h + 4q.. of K-step ks = c8 / 4, h = c8 / 2 % 2)
#pragma unroll
        for (int e = 0; e < 8; e++) bsT[(8 * c8 + e) * KP + k] = v[e];
        if constexpr (BY) {
          const int s0 = slot_of_col(8 * c8), s1 = slot_of_col(8 * c8 + 4);
          const unsigned lo[2] = {bv[i][0], bv[i][1]}, hi[2] = {bv[i][2], bv[i][3]};
          *reinterpret_cast<unsigned long long*>(bsY + k * SP + s0) = __builtin_bit_cast(unsigned long long, lo);
          *reinterpret_cast<unsigned long long*>(bsY + k * SP + s1) = __builtin_bit_cast(unsigned long long, hi);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int cc = 8 * c8 + e;                           // caller column
          const int col = cc < g.r ? inv_perm_rc(g, cc) : cc;  // internal column
          bsT[col * KP + k] = v[e];
          if constexpr (BY) bsY[k * SP + slot_of_col(col)] = v[e];
        }
      }
    }
    store_x(xs, tid);
#pragma unroll
    for (int i = 0; i < NRL; i++) {
      const int idx = tid + i * NTT;
      if (idx >= NRU) continue;
      if constexpr (ROT == 1) {
        const int tk = idx / (4 * RT), a2 = idx % (4 * RT);
        float s0, c0, s1, c1;
        sincosf(bf16_lo(r1[i]), &s0, &c0);
        sincosf(bf16_hi(r1[i]), &s1, &c1);
        *reinterpret_cast<f4*>((float*)rtv + tk * RTP + 4 * a2) = f4{c0, s0, c1, s1};
      } else if constexpr (ROT == 3) {
        const int tk = idx / (2 * RT), e8 = idx % (2 * RT);
        *reinterpret_cast<u4*>((bf16*)rtv + tk * RTP + 8 * e8) = r3[i];  // two blocks, bf16 as loaded
      }
    }
  }
};

// Four consecutive internal columns 4q.. of a state row (zero past r).
__device__ __forceinline__ f4 load_cols4(const float* row, int r, int col, int R) {
  if (r == R) return *reinterpret_cast<const f4*>(row + col);  // every column present
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
template <int NT, int ROT, int CK, int RT, bool PO = false>
__global__ __launch_bounds__(NTT, 1) void k_bwdt(
    Geo g, const bf16* __restrict__ xhat, const bf16* __restrict__ bhat, const bf16* __restrict__ da,
    const bf16* __restrict__ rot, const float* __restrict__ carry, const float* __restrict__ dm2,
    const float* __restrict__ dm1i, float* Db, bf16* d_xhat, bf16* d_bhat, bf16* d_da, bf16* d_rot) {
  constexpr int R = 16 * NT, K = ELL * CK, SP = cf_pitch(R), KP = cf_pitch(K), GTP = R + 16;
  constexpr int NKT = K / 16;      // (j,c) tiles
  constexpr int KSR = NT / 2;      // K-steps over state columns
  constexpr int KW = NKT < 2 ? NKT : 2;  // d_bhat: waves along (j,c) tiles (2 x 2 tile blocks per wave at K = 64)
  constexpr int CW = NWT / KW;     // d_bhat: waves along column tiles
  constexpr int KH = NKT / KW;     // d_bhat (j,c) tiles per wave
  constexpr int CH = NT / CW;      // d_bhat column tiles per wave
  constexpr int NRC = ROT == 3 ? 4 : 2;  // rotation-gradient values per (t, rotated tile)
  constexpr int RTA = RT > 0 ? RT : 1;
  constexpr int RTP = rt_pitch(16 * RT);  // rotation table floats per token (padded)
  static_assert((ROT == 0) == (RT == 0) && RT <= NT && CH >= 1 && KH >= 1, "tiling");
  using L = LdsT<NT, CK, PO>;
  constexpr int RR = L::RR;  // state rows of a round
  static_assert(!PO || CK == 2, "odd pair tokens: two channels per pair token");
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* Ss = (bf16*)(smem + L::Ss);
  bf16* bsT = (bf16*)(smem + L::bsT);
  bf16* bsY = (bf16*)(smem + L::bsY);
  bf16* xs = (bf16*)(smem + L::xs);
  float* LT = (float*)(smem + L::LT);
  float* s_a = (float*)(smem + L::a);
  float* s_d = (float*)(smem + L::d);
  using RTE = typename std::conditional<ROT == 3, bf16, float>::type;  // rotation table entries
  RTE* rt = (RTE*)(smem + L::rot);
  // four consecutive table entries as floats (a cos/sin pair of two angles, or a quaternion)
  auto rt4 = [&](int idx) -> f4 {
    if constexpr (ROT == 3) {
      const uint2 v = *reinterpret_cast<const uint2*>(rt + idx);
      return f4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
    } else {
      return *reinterpret_cast<const f4*>(rt + idx);
    }
  };
  bf16* Gs = (bf16*)(smem + L::Gs);
  bf16* dXs = (bf16*)(smem + L::dXs);
  float* red = (float*)(smem + L::red);
  f4* LWt = (f4*)(smem + L::lw);          // [LWN][64]
  f4* LYt = LWt + L::LWN * 64;            // [LYN][64]
  float* cst = (float*)(smem + L::cst);   // [carry x2 | d_m1 | D+][row of the round][R]
  float* dxp = (float*)(smem + L::dxp);   // [token half][row of the round][K]

  const int bh = blockIdx.x / g.NGR, gi = blockIdx.x % g.NGR;
  const int bi = bh / g.h, hi = bh % g.h;
  g.V = chain_len(g, bi);  // this sequence's valid length (per-sequence lengths)
  // tid is refreshed through an empty asm at every chunk: the per-thread
  // addresses of the chunk-boundary work are then recomputed per chunk instead
  // of being hoisted out of the chunk loop and held (spilled) across the rounds
  int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform in the wave
  const int lane = tid & 63, n = lane & 15, q = lane >> 4;
  const int u = w & 3, tt = w >> 2;       // row slot of the round, token half
  // PO: every wave works on the odd token slots; the first half takes rows 4..7
  const int t = PO ? 16 + n : 16 * tt + n;  // this lane's token slot in the transposed tiles
  const int rs = PO && tt == 0 ? 4 + u : u;  // this wave's row of the round
  const int tr = PO ? n : t;                 // its row of the rotation table
  const int gsl = PO && tt == 0 ? n : t;     // its slot row in the G block
  const int ptk = slot_tok<PO>(t);         // and its token
  const int kq = w / CW, cq = w % CW;     // d_bhat block of this wave

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

  using WS = WideStage<NT, CK, ROT, RT, true, PO>;
  const bool wide = WS::usable(g);
  WS wst;
  auto stage_x = [&](int nc, int pblk) {
    for (int idx = tid; idx < K * XPB; idx += NTT) {
      const int k = idx / XPB, pl = idx % XPB;
      const int j = k / CK, ci = k % CK;
      const int pos = nc * ELL + slot_tok<PO>(j);
      float v = 0.0f;
      if (pblk + pl < g.p && ci < g.c && pos < g.V)
        v = (float)xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pblk + pl];
      xs[pl * KP + k] = (bf16)v;
    }
  };
  auto flush_dx = [&](int nc, int pblk) {
    if (d_xhat == nullptr) return;
    if (wide) {
      // 16-byte stores of 8 rows p; work items over (j,c) fastest (LDS reads
      // of one row free of bank conflicts)
      constexpr int NXU = K * XPB / 8;
      for (int idx = tid; idx < NXU; idx += NTT) {
        const int k = idx % K, c8 = idx / K;
        const int j = k / CK, ci = k % CK;
        const int pos = nc * ELL + slot_tok<PO>(j);
        if (ci < g.c && pos < g.s && pblk + 8 * c8 < g.p) {
          u4 v;
#pragma unroll
          for (int e = 0; e < 4; e++)
            v[e] = (unsigned)__builtin_bit_cast(unsigned short, dXs[(8 * c8 + 2 * e) * KP + k]) |
                   ((unsigned)__builtin_bit_cast(unsigned short, dXs[(8 * c8 + 2 * e + 1) * KP + k]) << 16);
          *reinterpret_cast<u4*>(d_xhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pblk + 8 * c8) = v;
        }
      }
      return;
    }
    const int rows = g.p - pblk < XPB ? g.p - pblk : XPB;
    for (int idx = tid; idx < K * rows; idx += NTT) {
      const int k = idx / rows, pl = idx % rows;
      const int j = k / CK, ci = k % CK;
      const int pos = nc * ELL + slot_tok<PO>(j);
      if (ci < g.c && pos < g.s)
        d_xhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + pblk + pl] = dXs[pl * KP + k];
    }
  };
  // The carry rows h_-(n)[p][:], the d_m1 rows and the D(n+1) rows of a round
  // (RR state rows) travel through LDS: every thread with a piece loads its float4
  // pieces of them a round ahead and stores them after the round's row work, off
  // the rows' critical path. D(n+1) was written by this workgroup one chunk earlier.
  constexpr int CQA = RR * R / 4;          // float4 pieces of one array per round
  constexpr int CQ = 3 * CQA;              // pieces per round
  constexpr int NPC = (CQ + NTT - 1) / NTT;  // pieces per thread
  static_assert(CQA % 64 == 0, "whole waves per array");
  // This thread's pieces of the round rows are fixed: array farr (uniform in the
  // wave), row frr of the round, columns fcol..; per chunk only the row pointer
  // of round 0 changes, and each round steps it by RR rows.
  struct RowPiece {
    int farr, fidx, frr, fcol;
    bool fthr, fon;
    const float* frow0;
    size_t fstep;
    int flim;
  };
  RowPiece pc[NPC];
#pragma unroll
  for (int k = 0; k < NPC; k++) {
    const int pi = tid + k * NTT;
    pc[k].farr = __builtin_amdgcn_readfirstlane((w * 64 + k * NTT) / CQA);
    pc[k].fidx = pi - pc[k].farr * CQA;
    pc[k].frr = pc[k].fidx / (R / 4);
    pc[k].fcol = 4 * (pc[k].fidx % (R / 4));
    pc[k].fthr = w * 64 + k * NTT < CQ;
    pc[k].frow0 = nullptr;  // set per chunk
    pc[k].fstep = 0;
    pc[k].flim = R;
    pc[k].fon = false;
  }
  struct Pieces {
    f4 v[NPC];
  };
  int fnc = 0;           // chunk of the walk (PO: the pieces' rows are addressed at each fetch)
  bool fnext = false;    // ... and whether D(n+1) comes from it
  auto fetch_round = [&](int round) -> Pieces {
    Pieces r;
#pragma unroll
    for (int k = 0; k < NPC; k++) {
      r.v[k] = f4{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (PO) {
        // two pieces per thread: their row pointers are not held across the round
        const int farr = __builtin_amdgcn_readfirstlane((w * 64 + k * NTT) / CQA);
        const int fidx = tid + k * NTT - farr * CQA;
        const int row = RR * round + fidx / (R / 4), fcol = 4 * (fidx % (R / 4));
        if (w * 64 + k * NTT < CQ && row < g.p) {
          if (farr == 0)
            r.v[k] = load_cols4(carry + (((size_t)bh * g.NK + fnc) * g.p + row) * g.r, g.r, fcol, R);
          else if (farr == 1)
            r.v[k] = load_cols4(dm1i + ((size_t)bh * g.p + row) * R, R, fcol, R);
          else if (fnext)
            r.v[k] = load_cols4(Db + (((size_t)bh * g.NK + fnc + 1) * g.p + row) * g.r, g.r, fcol, R);
        }
      } else {
        if (pc[k].fon && RR * round + pc[k].frr < g.p)
          r.v[k] = load_cols4(pc[k].frow0 + (size_t)round * pc[k].fstep, pc[k].flim, pc[k].fcol, R);
      }
    }
    return r;
  };
  // The carry rows go to the buffer of the round's parity (they are read before
  // the round's first barrier); d_m1 and D+ rows to their single buffers.
  auto store_carry = [&](const Pieces& v, int buf) {
#pragma unroll
    for (int k = 0; k < NPC; k++)
      if (pc[k].fthr && pc[k].farr == 0) reinterpret_cast<f4*>(cst + (size_t)buf * RR * R)[pc[k].fidx] = v.v[k];
  };
  auto store_dmdp = [&](const Pieces& v) {
#pragma unroll
    for (int k = 0; k < NPC; k++)
      if (pc[k].fthr && pc[k].farr > 0)
        reinterpret_cast<f4*>(cst + (size_t)(1 + pc[k].farr) * RR * R)[pc[k].fidx] = v.v[k];
  };

  float dav = 0.0f;
  // the global loads of a chunk's inputs, all issued before the first is used
  auto load_chunk = [&](int ncl) {
    dav = 0.0f;
    if (tid < 32 && ncl * ELL + tid < g.V) dav = (float)da[((size_t)bi * g.s + ncl * ELL + tid) * g.h + hi];
    if (wide) wst.load(g, xhat, bhat, rot, ncl, bi, hi, tid);
  };
  const int n0 = gi * g.G;
  const int nkc = chain_nk(g);  // chunks walked
  const int n1 = (n0 + g.G < nkc) ? n0 + g.G : nkc;
  const int nrounds = (g.p + RR - 1) / RR;
  // ---- d_da of chunk ncs: sum_{t>=s} d_t <G[t], h_-> + sum_{s'<s} (C[s'] - Rw[s']),
  // from the per-wave partials the chunk left in LDS and its s_d, on the last
  // wave (the first wave rewrites s_d only after the staging barrier that
  // follows this scan)
  float* rg = (float*)(smem + L::red);  // [w][q][16] partial <G[t], h_->
  float* rwp = rg + NWT * 4 * 16;       // [w][16] partial row sums Rw
  float* csum = rwp + NWT * 16;         // [rr][(j,c)] partial column sums
  auto dda_scan = [&](int ncs) {
    const int lt = tid - (NTT - 64);  // the last wave's lanes
    if (lt < 0) return;
    // lane t < 32: x = d_t <G[t], h_->, y = C[t] - Rw[t]; then a suffix scan of x
    // and an exclusive prefix scan of y across the lanes (fixed order)
    const int tvs = g.V - ncs * ELL;
    const int tk = lt & 31, sl = tok_slot<PO>(tk), half = sl >> 4;
    float x = 0.0f, y = 0.0f;
    if (lt < ELL) {
      float gt = 0.0f, rw = 0.0f, cj = 0.0f;
      if constexpr (PO) {
        // every wave's partials are at the odd token slots 16..31; the even ones are zero
        if (half == 1) {
#pragma unroll
          for (int w8 = 0; w8 < NWT; w8++) {
#pragma unroll
            for (int qq = 0; qq < 4; qq++) gt += rg[(w8 * 4 + qq) * 16 + (sl & 15)];
            rw += rwp[w8 * 16 + (sl & 15)];
          }
        }
      } else {
#pragma unroll
        for (int uu = 0; uu < 4; uu++) {
#pragma unroll
          for (int qq = 0; qq < 4; qq++) gt += rg[((4 * half + uu) * 4 + qq) * 16 + (sl & 15)];
          rw += rwp[(4 * half + uu) * 16 + (sl & 15)];
        }
      }
      // channels ci >= c hold exact zeros (their xhat is staged as zero)
#pragma unroll
      for (int rr = 0; rr < RR; rr++)
#pragma unroll
        for (int ci = 0; ci < CK; ci++) cj += csum[rr * K + sl * CK + ci];
      x = s_d[sl] * gt;
      y = cj - rw;
    }
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const float xd = __shfl_down(x, off, 32);
      const float yu = __shfl_up(y, off, 32);
      if (tk + off < 32) x += xd;
      if (tk >= off) y += yu;
    }
    const float yex = __shfl_up(y, 1, 32);
    if (lt < ELL && d_da != nullptr) {
      const float pre = tk > 0 ? yex : 0.0f;
      // past valid_len every term vanishes; C - Rw cancels there only up to rounding
      const int pos = ncs * ELL + lt;
      if (pos < g.s) d_da[((size_t)bi * g.s + pos) * g.h + hi] = (bf16)(tk < tvs ? x + pre : 0.0f);
    }
  };
  for (int nc = n1 - 1; nc >= n0; nc--) {
    asm volatile("" : "+v"(tid));
    const bool has_next = nc + 1 < n1;  // D(n+1) comes from this walk; zero at the group's end
    fnc = nc;
    fnext = has_next;
#pragma unroll
    for (int k = 0; k < NPC && !PO; k++) {
      RowPiece& f = pc[k];
      if (f.farr == 0) {
        f.frow0 = carry + (((size_t)bh * g.NK + nc) * g.p + f.frr) * g.r;
        f.fstep = (size_t)RR * g.r;
        f.flim = g.r;
        f.fon = f.fthr;
      } else if (f.farr == 1) {
        f.frow0 = dm1i + ((size_t)bh * g.p + f.frr) * R;
        f.fstep = (size_t)RR * R;
        f.flim = R;
        f.fon = f.fthr;
      } else {
        f.frow0 = Db + (((size_t)bh * g.NK + nc + 1) * g.p + f.frr) * g.r;
        f.fstep = (size_t)RR * g.r;
        f.flim = g.r;
        f.fon = f.fthr && has_next;
      }
    }
    float* dbase = Db + ((size_t)bh * g.NK + nc) * g.p * g.r;  // D(n) rows of this chunk
    __syncthreads();
    if (nc + 1 < n1) dda_scan(nc + 1);  // the previous step's d_da
    load_chunk(nc);
    const Pieces v0 = fetch_round(0);
    // ---- chunk staging
    float dnew = 0.0f;  // d_t of this chunk, lanes 0..31 of the first wave
    if (tid < 64) {
      const int tk = tid & 31;
      float v = dav;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        const float up = __shfl_up(v, off, 32);
        if (tk >= off) v += up;
      }
      if (tid < 32) {
        s_a[tok_slot<PO>(tk)] = v;  // lane tk is token tk of the chunk
        dnew = expf(v);
      }
    }
    if (wide) {
      wst.store(g, bsT, bsY, xs, rt, tid);
    } else {
      for (int idx = tid; idx < K * R; idx += NTT) {
        const int k = idx / R, col = idx % R;
        const int j = k / CK, ci = k % CK;
        const int pos = nc * ELL + slot_tok<PO>(j);
        bf16 v = (bf16)0.0f;
        if (col < g.r && pos < g.V && ci < g.c)
          v = bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + perm_rc(g, col)];
        bsT[col * KP + k] = v;
        bsY[k * SP + slot_of_col(col)] = v;
      }
      if constexpr (ROT == 1) {
        for (int idx = tid; idx < L::RTK * 8 * RT; idx += NTT) {
          const int tk = idx / (8 * RT), a = idx % (8 * RT);
          const int pos = nc * ELL + slot_tok<PO>((PO ? ELL / 2 : 0) + tk);
          float th = 0.0f;
          if (a < g.A && pos < g.V) th = (float)rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + a];
          float sv, cv;
          sincosf(th, &sv, &cv);
          rt[tk * RTP + 2 * a] = cv;
          rt[tk * RTP + 2 * a + 1] = sv;
        }
      } else if constexpr (ROT == 3) {
        for (int idx = tid; idx < L::RTK * 16 * RT; idx += NTT) {
          const int tk = idx / (16 * RT), e = idx % (16 * RT);
          const int pos = nc * ELL + slot_tok<PO>((PO ? ELL / 2 : 0) + tk);
          float v = (e & 3) == 0 ? 1.0f : 0.0f;
          if ((e >> 2) < g.J && pos < g.V) v = (float)rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + e];
          rt[tk * RTP + e] = (RTE)v;
        }
      }
      stage_x(nc, 0);
    }
    store_carry(v0, 0);
    store_dmdp(v0);
    __syncthreads();  // (the last wave's scan of the previous chunk's s_d is done)
    if (tid < 32) s_d[tok_slot<PO>(tid)] = dnew;
    for (int idx = tid; idx < ELL * ELL; idx += NTT) {
      const int j = idx / ELL, tk = idx % ELL;
      LT[j * LTP + tk] = (slot_tok<PO>(j) <= slot_tok<PO>(tk)) ? expf(s_a[tk] - s_a[j]) : 0.0f;
    }
    __syncthreads();

    // ---- per-lane chunk constants: LDS tables of entries per wave lane l =
    // 16 ql + nl, filled by the whole workgroup ----------------------------------
    const int tv = g.V - nc * ELL;  // valid tokens of this chunk (<= 0: none)
    {
      // W factors: L[16h+nl][j of the slots 32ks+8ql..], flattened (h*CK+ks)*(8/CK)+v
      // (PO: the second half h = 1 only, at entries f - 8)
      constexpr int NLW = PO ? 8 : 16;
      for (int idx = tid; idx < NLW * 64; idx += NTT) {
        const int fe = idx >> 6, l = idx & 63, ql = l >> 4, nl = l & 15;
        const int f = PO ? fe + 8 : fe;
        const int hh = f / 8, rest = f % 8, ks = rest / (8 / CK), v = rest % (8 / CK);
        reinterpret_cast<float*>(LWt + (fe >> 2) * 64 + l)[fe & 3] =
            LT[((32 * ks + 8 * ql) / CK + v) * LTP + 16 * hh + nl];
      }
      // d_xhat factors: L[16h+4ql+i][j of (j,c) = 16kt+nl], entry h*NKT+kt (PO: h = 1, entry kt)
      constexpr int NLY = (PO ? 1 : 2) * NKT;
      for (int idx = tid; idx < NLY * 64; idx += NTT) {
        const int e = idx >> 6, l = idx & 63, ql = l >> 4, nl = l & 15;
        const int hh = PO ? 1 : e / NKT, kt = e % NKT;
        f4 v;
#pragma unroll
        for (int i = 0; i < 4; i++) v[i] = LT[((16 * kt + nl) / CK) * LTP + 16 * hh + 4 * ql + i];
        LYt[e * 64 + l] = v;
      }
    }
    __syncthreads();

    f4 dbacc[KH][CH];
#pragma unroll
    for (int a = 0; a < KH; a++)
#pragma unroll
      for (int b = 0; b < CH; b++) dbacc[a][b] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    float racc[RTA][NRC];
#pragma unroll
    for (int ct = 0; ct < RTA; ct++)
#pragma unroll
      for (int v = 0; v < NRC; v++) racc[ct][v] = 0.0f;
    float gcar = 0.0f;  // sum over this wave's rows and columns of G[t] h_- at token t
    f4 rwa = f4{0.0f, 0.0f, 0.0f, 0.0f};  // row sums of E at t = 16tt+4q+i, over this lane's (j,c) and rows
    float cct = 0.0f;   // thread (rr, k) < 4K: sum over the rounds' rows rr of xhat * d_xhat
    const float dtl = s_d[t];

    for (int round = 0; round < nrounds; round++) {
      const int pr0 = RR * round;
      const int pblk = pr0 - pr0 % XPB;
      if (round > 0 && pr0 % XPB == 0) {
        __syncthreads();  // the previous round's d_bhat work read the old block
        flush_dx(nc, pblk - XPB);
        __syncthreads();
        if (wide) {
          if constexpr (!PO) wst.load_x(g, xhat, nc, pblk, bi, hi, tid);  // (PO: loaded a round early)
          wst.store_x(xs, tid);
        } else {
          stage_x(nc, pblk);
        }
        __syncthreads();
      }
      const int p = pr0 + rs;
      const Pieces pf = fetch_round(round + 1);  // next round's rows
      // One state row, all columns, this wave's 16 tokens, in two parts: the
      // states and the packed c^T, then (after a barrier that retires the
      // previous round's reads of the G blocks) everything that writes them.
      // MASK zeroes d_c at tokens >= tv (only the chunk holding valid_len needs
      // it; the PO lanes hold odd pair tokens only).
      const int pl = p - pblk;
      u4 cP[KSR];
      u4 hP[ROT == 3 ? KSR : 1];
      const float* hrow = cst + ((size_t)(round & 1) * RR + rs) * R;
      auto row1 = [&]() {
        // ---- W fragment: W[t][(j,c)] = L[t,j] xhat[(j,c)][p] ----------------
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
            const f4 v = LWt[((PO ? 0 : 2 * tt) + e4) * 64 + lane];
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
        // ---- states h~^T[col][t] one column tile at a time, then the carry, the
        // de-rotation in the lane and the packed c^T (and h~^T) --------------------
        // tokens 0..15 see j <= 15 only: their last K-steps are all zero
        const int nks = tt == 0 && !PO ? (CK + 1) / 2 : CK;

        // bhat^T fragments software-pipelined one column tile ahead
        bf8 bn[CK];
#pragma unroll
        for (int ks = 0; ks < CK; ks++)
          if (ks < nks) bn[ks] = ld_frag(bsT + n * KP + 32 * ks + 8 * q);
        // carry and rotation rows pipelined one column tile ahead as well
        f4 hvn = *reinterpret_cast<const f4*>(hrow + 4 * q);
        f4 rtn = RT > 0 ? rt4(tr * RTP + 4 * q) : f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ct = 0; ct < NT; ct++) {
          __builtin_amdgcn_sched_barrier(0);
          bf8 ba[CK];
#pragma unroll
          for (int ks = 0; ks < CK; ks++) ba[ks] = bn[ks];
          const f4 hv = hvn, rtc = rtn;
          if (ct + 1 < NT) {
#pragma unroll
            for (int ks = 0; ks < CK; ks++)
              if (ks < nks) bn[ks] = ld_frag(bsT + (16 * (ct + 1) + n) * KP + 32 * ks + 8 * q);
            hvn = *reinterpret_cast<const f4*>(hrow + 16 * (ct + 1) + 4 * q);
            if (ct + 1 < RT) rtn = rt4(tr * RTP + 16 * (ct + 1) + 4 * q);
          }
          __builtin_amdgcn_sched_barrier(0);
          f4 hT = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < CK; ks++)
            if (ks < nks) hT = MM<bf16>::mma(ba[ks], as_bf8(Wf[ks]), hT);
          f4 h;
#pragma unroll
          for (int i = 0; i < 4; i++) h[i] = hT[i] + dtl * hv[i];
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
            hP[ROT == 3 ? ct >> 1 : 0][2 * (ct & 1)] = pk_bf16(h[0], h[1]);
            hP[ROT == 3 ? ct >> 1 : 0][2 * (ct & 1) + 1] = pk_bf16(h[2], h[3]);
          }
          cP[ct >> 1][2 * (ct & 1)] = pk_bf16(c[0], c[1]);
          cP[ct >> 1][2 * (ct & 1) + 1] = pk_bf16(c[2], c[3]);
        }
      };
      auto row2 = [&](auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        // ---- d_c^T = S c^T + d_m1, rotation VJP, G, Y = G bhat^T ------------
        const float* dmrow = cst + (2 * RR + rs) * R;
        const float* dprow = cst + (3 * RR + rs) * R;  // D(n+1)[p][:], enters G at the last token
        const float f31 = t == ELL - 1 ? 1.0f : 0.0f;
        f4 Y[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; kt++) Y[kt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        // this lane's piece of its slot row in the G block (PO: block u holds rows u
        // and 4+u of the round at slots 16.. and 0..)
        bf16* Gw = Gs + ((size_t)u * ELL + gsl) * GTP + 4 * gpiece(q, gsl);
        // S fragments are software-pipelined one column tile ahead: tile ct+1's
        // reads are in flight while tile ct runs its MFMAs and rotation work
        bf8 sn[KSR];
#pragma unroll
        for (int ks = 0; ks < KSR; ks++) sn[ks] = ld_frag(Ss + n * SP + 32 * ks + 8 * q);
#pragma unroll
        for (int ky = 0; ky < KSR; ky++) {
          u4 GP;
#pragma unroll
          for (int h2 = 0; h2 < 2; h2++) {
            // keep each column tile's work together (bounds live registers)
            __builtin_amdgcn_sched_barrier(0);
            const int ct = 2 * ky + h2;
            f4 d = *reinterpret_cast<const f4*>(dmrow + 16 * ct + 4 * q);
            bf8 sa[KSR];
#pragma unroll
            for (int ks = 0; ks < KSR; ks++) sa[ks] = sn[ks];
            if (ct + 1 < NT) {
#pragma unroll
              for (int ks = 0; ks < KSR; ks++) sn[ks] = ld_frag(Ss + (16 * (ct + 1) + n) * SP + 32 * ks + 8 * q);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KSR; ks++) d = MM<bf16>::mma(sa[ks], as_bf8(cP[ks]), d);
            if constexpr (MASK) {
              if (ptk >= tv) d = f4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            f4 hc;  // c (complex, none) or h~ (quaternion), from the packed fragments
            {
              const unsigned w0 = ROT == 3 ? hP[ROT == 3 ? ky : 0][2 * h2] : cP[ky][2 * h2];
              const unsigned w1 = ROT == 3 ? hP[ROT == 3 ? ky : 0][2 * h2 + 1] : cP[ky][2 * h2 + 1];
              hc[0] = bf16_lo(w0);
              hc[1] = bf16_hi(w0);
              hc[2] = bf16_lo(w1);
              hc[3] = bf16_hi(w1);
            }
            f4 G = d;
            if constexpr (ROT == 3) {
              if (ct < RT) {
                const f4 Q = rt4(tr * RTP + 16 * ct + 4 * q);
                G[0] = Q[0] * d[0] + Q[1] * d[1] + Q[2] * d[2] + Q[3] * d[3];
                G[1] = Q[0] * d[1] - Q[1] * d[0] - Q[2] * d[3] + Q[3] * d[2];
                G[2] = Q[0] * d[2] + Q[1] * d[3] - Q[2] * d[0] - Q[3] * d[1];
                G[3] = Q[0] * d[3] - Q[1] * d[2] + Q[2] * d[1] - Q[3] * d[0];
                float* ra = racc[ct < RT ? ct : 0];
                ra[0] += d[0] * hc[0] + d[1] * hc[1] + d[2] * hc[2] + d[3] * hc[3];
                ra[1] += -d[0] * hc[1] + d[1] * hc[0] - d[2] * hc[3] + d[3] * hc[2];
                ra[2] += -d[0] * hc[2] + d[1] * hc[3] + d[2] * hc[0] - d[3] * hc[1];
                ra[3] += -d[0] * hc[3] - d[1] * hc[2] + d[2] * hc[1] + d[3] * hc[0];
              }
            } else {
              if constexpr (ROT == 1) {
                if (ct < RT) {
                  const f4 r4 = rt4(tr * RTP + 16 * ct + 4 * q);
                  float* ra = racc[ct < RT ? ct : 0];
                  ra[0] += d[0] * hc[1] - d[1] * hc[0];
                  ra[1] += d[2] * hc[3] - d[3] * hc[2];
                  G[0] = r4[0] * d[0] - r4[1] * d[1];
                  G[1] = r4[1] * d[0] + r4[0] * d[1];
                  G[2] = r4[2] * d[2] - r4[3] * d[3];
                  G[3] = r4[3] * d[2] + r4[2] * d[3];
                }
              }
            }
            if ((PO || tt == 1) && has_next) {
              const f4 dp = *reinterpret_cast<const f4*>(dprow + 16 * ct + 4 * q);
#pragma unroll
              for (int i = 0; i < 4; i++) G[i] += f31 * dp[i];
            }
            {
              const f4 hv = *reinterpret_cast<const f4*>(hrow + 16 * ct + 4 * q);
              gcar += G[0] * hv[0] + G[1] * hv[1] + G[2] * hv[2] + G[3] * hv[3];
            }
            GP[2 * h2] = pk_bf16(G[0], G[1]);
            GP[2 * h2 + 1] = pk_bf16(G[2], G[3]);
          }
          // Y[t][(j,c)] += sum over this K-step's columns of G[t][col] bhat[(j,c)][col]
          bf8 yb[NKT];
#pragma unroll
          for (int kt = 0; kt < NKT; kt++) yb[kt] = ld_frag(bsY + (16 * kt + n) * SP + 32 * ky + 8 * q);
#pragma unroll
          for (int kt = 0; kt < NKT; kt++) Y[kt] = MM<bf16>::mma(as_bf8(GP), yb[kt], Y[kt]);
          // G into the row's block, [token][column]: columns 32ky+4q.. and 32ky+16+4q..
          {
            const unsigned lo[2] = {GP[0], GP[1]}, hi[2] = {GP[2], GP[3]};
            *reinterpret_cast<unsigned long long*>(Gw + 32 * ky) = __builtin_bit_cast(unsigned long long, lo);
            *reinterpret_cast<unsigned long long*>(Gw + 32 * ky + 16) = __builtin_bit_cast(unsigned long long, hi);
          }
        }
        // ---- this half's share of d_xhat[(j,c)][p] = sum_t L[t,j] Y[t][(j,c)] ----
        float* part = dxp + (tt * 4 + u) * K;
        float vq = 0.0f;  // the sum of tile kt = q % NKT, which lane group q stores
#pragma unroll
        for (int kt = 0; kt < NKT; kt++) {
          const f4 ly = LYt[((PO ? 0 : tt * NKT) + kt) * 64 + lane];
          const float xk = (float)xs[pl * KP + 16 * kt + n];
          f4 e;
#pragma unroll
          for (int i = 0; i < 4; i++) e[i] = ly[i] * Y[kt][i];
#pragma unroll
          for (int i = 0; i < 4; i++) rwa[i] += xk * e[i];
          float v = e[0] + e[1] + e[2] + e[3];
          v = col4_sum(v);
          vq = (q % NKT) == kt ? v : vq;
        }
        part[16 * (q % NKT) + n] = vq;
      };
      // (PO: a wave whose row is past p zeroes its G slots, which the d_bhat
      // contraction reads together with the other row of its block)
      if (p < g.p) row1();
      __syncthreads();  // the previous round's d_bhat reads of the G blocks are done
      if (PO && p >= g.p) {
        bf16* Gw = Gs + ((size_t)u * ELL + gsl) * GTP + 4 * gpiece(q, gsl);
#pragma unroll
        for (int ky = 0; ky < KSR; ky++) {
          *reinterpret_cast<unsigned long long*>(Gw + 32 * ky) = 0ull;
          *reinterpret_cast<unsigned long long*>(Gw + 32 * ky + 16) = 0ull;
        }
      }
      if (p < g.p) {
        if (tv >= ELL) row2(std::false_type{});
        else row2(std::true_type{});
      }
      store_carry(pf, (round + 1) & 1);  // its buffer was last read two rounds back
      __syncthreads();  // the round's G blocks and d_xhat partials are complete; next carry rows staged
      store_dmdp(pf);   // the round's d_c work, their only reader, is done
      // (PO: the next xhat block, when the next round starts one, is in flight
      // during this round's d_bhat work)
      if constexpr (PO) {
        if (wide && (RR * (round + 1)) % XPB == 0 && round + 1 < nrounds)
          wst.load_x(g, xhat, nc, RR * (round + 1), bi, hi, tid);
      }
      // ---- d_xhat of the round's rows: the two token halves added (PO: each
      // wave slot tt*4+u holds a whole row, rs = u or 4+u) -----------------------
      if (tid < RR * K) {
        const int rr = tid / K, k = tid % K;
        const int pp = pr0 + rr;
        if (pp < g.p) {
          const float v = PO ? dxp[(rr < 4 ? 4 + rr : rr - 4) * K + k] : dxp[rr * K + k] + dxp[(4 + rr) * K + k];
          const int pl = pp - pblk;
          dXs[pl * KP + k] = (bf16)v;
          cct += v * (float)xs[pl * KP + k];
        }
      }
      // the second token half has the longer row work ahead of it: its waves get
      // issue priority for the d_bhat work, the first half's fills in under their rows
      if (!PO && tt == 1) __builtin_amdgcn_s_setprio(2);
      if constexpr (PO) {
        // ---- d_bhat and local over the odd pair tokens of two rows per block:
        // K-slots 8q+e (e < 4) are block slots 4q+e = row 4+rr at token slot
        // 16+4q+e, K-slots e >= 4 are block slots 16+4q+e-4 = row rr at token
        // slot 16+4q+e-4; so both halves of a K-step take L at the same tokens.
        float LB[KH][4];  // L[16+4q+i][j of (j,c) = 16(kq*KH+kb)+n]
#pragma unroll
        for (int kb = 0; kb < KH; kb++) {
          const f4 l = *reinterpret_cast<const f4*>(LT + ((16 * (kq * KH + kb) + n) / CK) * LTP + 16 + 4 * q);
#pragma unroll
          for (int i = 0; i < 4; i++) LB[kb][i] = l[i];
        }
        bf8 dA;  // A operand of local: row 0 = d_t over row rr's K-slots, row 4 over row 4+rr's
        {
          const f4 d1 = *reinterpret_cast<const f4*>(s_d + 16 + 4 * q);
          const float on0 = n == 0 ? 1.0f : 0.0f, on4 = n == 4 ? 1.0f : 0.0f;
#pragma unroll
          for (int e = 0; e < 4; e++) {
            dA[e] = (bf16)(on4 * d1[e]);
            dA[e + 4] = (bf16)(on0 * d1[e]);
          }
        }
#pragma unroll 1
        for (int rr = 0; rr < 4; rr++) {
          const int pa = pr0 + rr, pb = pr0 + 4 + rr;  // the rows of block rr
          if (pa >= g.p) break;                         // then pb >= p as well
          const bool vb = pb < g.p;
          u4 Ab[KH];
#pragma unroll
          for (int kb = 0; kb < KH; kb++) {
            const int kk = 16 * (kq * KH + kb) + n;
            const float xa = (float)xs[(pa - pblk) * KP + kk];
            const float xb = vb ? (float)xs[(pb - pblk) * KP + kk] : 0.0f;
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              Ab[kb][e / 2] = pk_bf16(LB[kb][e] * xb, LB[kb][e + 1] * xb);
              Ab[kb][2 + e / 2] = pk_bf16(LB[kb][e] * xa, LB[kb][e + 1] * xa);
            }
          }
          const bf16* Gr = Gs + (size_t)rr * ELL * GTP;
          const bool do_local = kq == (rr % KW);  // each (block, column tile) once
#pragma unroll
          for (int cb = 0; cb < CH; cb++) {
            const int ct = cq * CH + cb;
            const bf8 gb = ld_tok_frag<GTP>(Gr, ct, lane);
#pragma unroll
            for (int kb = 0; kb < KH; kb++) dbacc[kb][cb] = MM<bf16>::mma(as_bf8(Ab[kb]), gb, dbacc[kb][cb]);
            if (do_local) {
              const f4 lo = MM<bf16>::mma(dA, gb, f4{0.0f, 0.0f, 0.0f, 0.0f});
              const int col = 16 * ct + n;
              if (col < g.r) {
                if (q == 0) dbase[(size_t)pa * g.r + col] = lo[0];        // row 0 of the output
                if (q == 1 && vb) dbase[(size_t)pb * g.r + col] = lo[0];  // row 4
              }
            }
          }
        }
      } else {
        // ---- d_bhat[(j,c)][col] += sum_t L[t,j] xhat[(j,c)][p] G[t][col]; local ----
        float LB[KH][8];  // L[tslot(8q+e)][j of (j,c) = 16(kq*KH+kb)+n]
  #pragma unroll
        for (int kb = 0; kb < KH; kb++) {
          const float* src = LT + ((16 * (kq * KH + kb) + n) / CK) * LTP + 4 * q;
          const f4 l0 = *reinterpret_cast<const f4*>(src);
          const f4 l1 = *reinterpret_cast<const f4*>(src + 16);
  #pragma unroll
          for (int e = 0; e < 4; e++) {
            LB[kb][e] = l0[e];
            LB[kb][e + 4] = l1[e];
          }
        }
        bf8 dA;  // A operand of local: rows 0, 4, 8, 12 = d_t over the K-slots, t = tslot(8q+e)
        {
          const f4 d0 = *reinterpret_cast<const f4*>(s_d + 4 * q);
          const f4 d1 = *reinterpret_cast<const f4*>(s_d + 16 + 4 * q);
          const float on = (n & 3) == 0 ? 1.0f : 0.0f;
  #pragma unroll
          for (int e = 0; e < 4; e++) {
            dA[e] = (bf16)(on * d0[e]);
            dA[e + 4] = (bf16)(on * d1[e]);
          }
        }
        if (pr0 + 4 <= g.p) {
          // all four rows present: every G^T fragment of the round is loaded up
          // front, so one LDS latency covers the whole phase
          bf8 gbf[4][CH];
  #pragma unroll
          for (int rr = 0; rr < 4; rr++)
  #pragma unroll
            for (int cb = 0; cb < CH; cb++)
              gbf[rr][cb] = ld_tok_frag<GTP>(Gs + (size_t)rr * ELL * GTP, cq * CH + cb, lane);
          u4 Ab[4][KH];
  #pragma unroll
          for (int rr = 0; rr < 4; rr++)
  #pragma unroll
            for (int kb = 0; kb < KH; kb++) {
              const float xk = (float)xs[(pr0 + rr - pblk) * KP + 16 * (kq * KH + kb) + n];
  #pragma unroll
              for (int e = 0; e < 8; e += 2) Ab[rr][kb][e / 2] = pk_bf16(LB[kb][e] * xk, LB[kb][e + 1] * xk);
            }
  #pragma unroll
          for (int rr = 0; rr < 4; rr++)
  #pragma unroll
            for (int cb = 0; cb < CH; cb++)
  #pragma unroll
              for (int kb = 0; kb < KH; kb++)
                dbacc[kb][cb] = MM<bf16>::mma(as_bf8(Ab[rr][kb]), gbf[rr][cb], dbacc[kb][cb]);
          // local of the rows rr with rr % KW == kq (each (row, column tile) once):
          // every lane group holds the row sums (dA repeats d_t in rows 0, 4, 8,
          // 12), and group q stores column tile q % CH
  #pragma unroll
          for (int rr = 0; rr < 4; rr++) {
            if (rr % KW != kq) continue;
            float* dbrow = dbase + (size_t)(pr0 + rr) * g.r;
            float lq = 0.0f;
  #pragma unroll
            for (int cb = 0; cb < CH; cb++) {
              const f4 lo = MM<bf16>::mma(dA, gbf[rr][cb], f4{0.0f, 0.0f, 0.0f, 0.0f});
              lq = (q % CH) == cb ? lo[0] : lq;
            }
            const int col = 16 * (cq * CH + q % CH) + n;
            if (q < CH && col < g.r) dbrow[col] = lq;
          }
        } else {
  #pragma unroll 1
          for (int rr = 0; rr < 4; rr++) {
            const int pp = pr0 + rr;
            if (pp >= g.p) break;
            const int pl = pp - pblk;
            u4 Ab[KH];
  #pragma unroll
            for (int kb = 0; kb < KH; kb++) {
              const float xk = (float)xs[pl * KP + 16 * (kq * KH + kb) + n];
  #pragma unroll
              for (int e = 0; e < 8; e += 2) Ab[kb][e / 2] = pk_bf16(LB[kb][e] * xk, LB[kb][e + 1] * xk);
            }
            const bf16* Gr = Gs + (size_t)rr * ELL * GTP;
            float* dbrow = dbase + (size_t)pp * g.r;
            const bool do_local = kq == (rr % KW);  // each (row, column tile) once
  #pragma unroll
            for (int cb = 0; cb < CH; cb++) {
              const int ct = cq * CH + cb;
              const bf8 gb = ld_tok_frag<GTP>(Gr, ct, lane);
  #pragma unroll
              for (int kb = 0; kb < KH; kb++) dbacc[kb][cb] = MM<bf16>::mma(as_bf8(Ab[kb]), gb, dbacc[kb][cb]);
              if (do_local) {
                const f4 lo = MM<bf16>::mma(dA, gb, f4{0.0f, 0.0f, 0.0f, 0.0f});
                const int col = 16 * ct + n;
                if (q == 0 && col < g.r) dbrow[col] = lo[0];  // every group holds it; group 0 stores
              }
            }
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();  // the last round's d_bhat reads are done
    flush_dx(nc, (nrounds - 1) * RR - ((nrounds - 1) * RR) % XPB);

    // ---- chunk end: d_bhat, the rotation gradient and the d_da partials go
    // through LDS behind one barrier: d_bhat in the G space, the rotation-gradient
    // partials in the (now dead) bhat tiles when they fit there
    constexpr int rw = ROT == 3 ? 16 * RTA : 8 * RTA;
    constexpr size_t RB_FULL = (size_t)NWT * 16 * rw * 4;
    constexpr bool RB_IN_B = RB_FULL <= L::xs - L::bsT;
    // passes over groups of rotated tiles when the partials exceed the G space
    constexpr int NPASS = RB_IN_B || RB_FULL <= L::gsb ? 1 : RB_FULL <= 2 * L::gsb ? 2 : 4;
    static_assert(ROT == 0 || RTA % NPASS == 0, "whole rotated tiles per pass");
    constexpr int rwq = rw / NPASS, CTP = RTA / NPASS;  // columns and rotated tiles per pass
    float* RB = RB_IN_B ? (float*)(smem + L::bsT) : (float*)Gs;  // [w][16 tokens][rwq]
    bf16* DBs = Gs;  // [K][SP]
    if (d_bhat != nullptr) {
#pragma unroll
      for (int kb = 0; kb < KH; kb++)
#pragma unroll
        for (int cb = 0; cb < CH; cb++)
#pragma unroll
          for (int i = 0; i < 4; i++)
            DBs[(16 * (kq * KH + kb) + 4 * q + i) * SP + 16 * (cq * CH + cb) + n] = (bf16)dbacc[kb][cb][i];
    }
    auto rb_write = [&](auto pass_c) {
      constexpr int PS = decltype(pass_c)::value;
#pragma unroll
      for (int c = 0; c < CTP; c++) {
        const int ct = PS * CTP + c;
        float* dst = RB + (w * 16 + n) * rwq;
        if constexpr (ROT == 1) {
          dst[8 * c + 2 * q] = racc[ct][0];
          dst[8 * c + 2 * q + 1] = racc[ct][1];
        } else {
#pragma unroll
          for (int v = 0; v < 4; v++) dst[4 * (4 * c + q) + v] = racc[ct][v];
        }
      }
    };
    // one pass of the fixed-order sum over the waves of a token half
    auto rb_reduce = [&](int pass) {
      for (int idx = tid; idx < ELL * rwq; idx += NTT) {
        const int tk = idx / rwq, el = idx % rwq, e = pass * rwq + el;
        if (e >= g.RW) continue;
        const int half = tk >> 4;
        float s = 0.0f;
        if constexpr (PO) {
          // every wave holds the odd token slots 16..31; the even slots are zero
          if (half == 1) {
#pragma unroll
            for (int w8 = 0; w8 < NWT; w8++) s += RB[(w8 * 16 + (tk & 15)) * rwq + el];
          }
        } else {
#pragma unroll
          for (int uu = 0; uu < 4; uu++) s += RB[((4 * half + uu) * 16 + (tk & 15)) * rwq + el];
        }
        const int pos = nc * ELL + slot_tok<PO>(tk);
        if (pos < g.s) d_rot[(((size_t)bi * g.s + pos) * g.h + hi) * g.RW + e] = (bf16)s;
      }
    };
    if constexpr (ROT != 0 && RB_IN_B) {
      if (d_rot != nullptr) rb_write(IC4<0>{});
    }
    rg[(w * 4 + q) * 16 + n] = gcar;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float r = row16_sum(rwa[i]);
      if (n == 0) rwp[w * 16 + 4 * q + i] = r;
    }
    if (tid < RR * K) csum[tid] = cct;
    // (the d_da partials are scanned at the start of the next step of the walk,
    // behind the barrier there, while the next chunk's loads are in flight)
    __syncthreads();
    if (d_bhat != nullptr) {
      if (wide && !g.half) {
        // internal columns are the caller's: 16-byte pieces of 8 columns, a row's
        // pieces on consecutive lanes
        for (int idx = tid; idx < K * (R / 8); idx += NTT) {
          const int k = idx / (R / 8), c8 = idx % (R / 8);
          const int j = k / CK, ci = k % CK;
          const int pos = nc * ELL + slot_tok<PO>(j);
          if (pos < g.s && ci < g.c && 8 * c8 < g.r)
            *reinterpret_cast<u4*>(d_bhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + 8 * c8) =
                *reinterpret_cast<const u4*>(DBs + k * SP + 8 * c8);
        }
      } else {
        for (int idx = tid; idx < K * g.r; idx += NTT) {
          const int k = idx / g.r, ra = idx - k * g.r;
          const int j = k / CK, ci = k % CK;
          const int pos = nc * ELL + slot_tok<PO>(j);
          if (pos < g.s && ci < g.c)
            d_bhat[((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + ra] = DBs[k * SP + inv_perm_rc(g, ra)];
        }
      }
    }
    // ---- rotation gradient: fixed-order sum over the waves of a token half -----
    if constexpr (ROT != 0) {
      if (d_rot != nullptr) {
        if constexpr (RB_IN_B) {
          rb_reduce(0);
        } else {
          auto one_pass = [&](auto pass_c) {
            __syncthreads();  // the d_bhat reads (or the previous pass) of the shared space are done
            rb_write(pass_c);
            __syncthreads();
            rb_reduce(decltype(pass_c)::value);
          };
          one_pass(IC4<0>{});
          if constexpr (NPASS > 1) one_pass(IC4<1>{});
          if constexpr (NPASS > 2) {
            one_pass(IC4<2>{});
            one_pass(IC4<3>{});
          }
        }
      }
    }
  }
  __syncthreads();
  if (n1 > n0) dda_scan(n0);  // the last chunk's d_da
}

}  // namespace mom

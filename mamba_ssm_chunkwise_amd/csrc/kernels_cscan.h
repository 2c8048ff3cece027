// Boundary carries: one walk per (b,h) chain, or per group of its chunks
// (bf16 inputs).
//
// Source: burn-mamba "backward.rs" source page, boundary_carries: the state
// entering chunk n is h_-(0) = h0 and h_-(n+1) = dec_n h_-(n) + U_n, where
// dec_n = exp(a_last) and U_n[p][col] = sum_{(j,c)} exp(a_last - a_j)
// xhat[j,c,p] bhat[j,c,col] is the chunk's decay-to-chunk-end product.
//
// One workgroup walks one chain from the first chunk to the last (or, in the
// group forms below, one group of chunks). The state rows stay in MFMA
// accumulators for the whole walk (wave w owns row tiles w, w+4): per chunk the
// wave stores h_-(n), scales by dec_n and accumulates U_n on MFMA. Each chunk's
// xhat and bhat are fetched one chunk ahead into registers and stored to LDS in
// their global layouts ([(j,c)][p] and [(j,c)][col]); transposing LDS reads
// build both MFMA operands from there.
// The states are kept in the caller's column order and written to the
// internal order on store.
#pragma once

#include "kernels_bwdt.h"

namespace mom {

constexpr int CSW = 4;           // waves of k_cscan
constexpr int CST = 64 * CSW;    // threads of k_cscan
constexpr int CMT = 2;           // row tiles per wave at most (state rows <= 128)

// Row pitch (bf16) of a staged [(j,c)][row] block with PK rows: the eight rows
// a half wave reads in one transposing read start 8 banks apart.
__host__ __device__ __forceinline__ int cscan_xp(int PK) { return PK + (((PK >> 4) & 1) ? 32 : 16); }

template <int NT, int CK>
struct LdsC {
  static constexpr int R = 16 * NT, K = ELL * CK, BP = R + 16;
  // nb staging buffers (Geo::cnb)
  __host__ __device__ static size_t xs(int, int) { return 0; }                                     // [nb][K][XP]
  __host__ __device__ static size_t bs(int PK, int nb) { return (size_t)nb * K * cscan_xp(PK) * 2; }  // [nb][K][BP]
  __host__ __device__ static size_t wv(int PK, int nb) { return bs(PK, nb) + (size_t)nb * K * BP * 2; }  // [nb][ELL+4]
  __host__ __device__ static size_t total(int PK, int nb) { return wv(PK, nb) + (size_t)nb * (ELL + 4) * 4; }
};

// Operand over K-step ks of a [(j,c)][x] block (pitch P): lane (q, m) gets x =
// x0 + m at K-slots 8q+e, which hold (j,c) = 32ks + 4q + e (e < 4) and
// 32ks + 16 + 4q + e - 4. Lane 4r+s of a group addresses (j,c) 32ks+4q+r
// (+16), x0 + 4s.
__device__ __forceinline__ bf8 ld_kx_frag(const bf16* blk, int P, int ks, int x0, int lane) {
  const bf16* p0 = blk + (32 * ks + 4 * (lane >> 4) + ((lane >> 2) & 3)) * P + x0 + 4 * (lane & 3);
  const s4 a = lds_read_tr16(p0), b = lds_read_tr16(p0 + 16 * P);
  const s4 v[2] = {a, b};
  return __builtin_bit_cast(bf8, v);
}

// 4x4 transpose within each quad of lanes: lane j's v[i] becomes lane i's
// v[j] (two exchanges, lanes j ^ 2 then j ^ 1, through DPP quad permutes).
__device__ __forceinline__ void quad_transpose(f4& v, int j) {
  auto xch = [](float x, int ctrl) {
    return __builtin_bit_cast(float, ctrl == 0x4E ? __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false)
                                                  : __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  };
  {  // 2x2 blocks: lanes 0-1 registers 2-3 <-> lanes 2-3 registers 0-1
    const bool hi = j & 2;
    const float r0 = xch(hi ? v[0] : v[2], 0x4E), r1 = xch(hi ? v[1] : v[3], 0x4E);
    if (hi) { v[0] = r0; v[1] = r1; } else { v[2] = r0; v[3] = r1; }
  }
  {  // within each 2x2 block
    const bool od = j & 1;
    const float r0 = xch(od ? v[0] : v[1], 0xB1), r1 = xch(od ? v[2] : v[3], 0xB1);
    if (od) { v[0] = r0; v[2] = r1; } else { v[1] = r0; v[3] = r1; }
  }
}

// MTW: row tiles per wave (1: state rows <= 64, 2: <= 128).
// GM: 0 walks each chain from h0 and stores every carry. 1 (group summaries):
// workgroup (chain, group gi) walks the group's G chunks from a zero state and
// leaves Z, the state after the group, in the carry rows of chunk gi G + 1 and
// the product D of its chunk decays in dec at that chunk (slots a forward that
// carries its state through each group never reads); k_gentry then forms the
// states entering the groups, and the last group of a chain returns at once.
// 2 (group carries): each group is walked from the state k_gentry left in its
// first chunk's carry rows, storing every carry and decay of the group.
// Staging: chunk nc+1's inputs are loaded during chunk nc's work and go into
// the other of two LDS buffers, or (Geo::cnb = 1) into the one buffer once
// every wave has read chunk nc from it.
template <int NT, int CK, int MTW, int GM = 0>
__global__ __launch_bounds__(CST, 2) void k_cscan(Geo g, int PK, const bf16* __restrict__ xhat,
                                               const bf16* __restrict__ bhat, const bf16* __restrict__ da,
                                               const bf16* __restrict__ h0, float* carry, float* dec) {
  constexpr int R = 16 * NT, K = ELL * CK, BP = R + 16, NKS = K / 32;
  constexpr int XPT = K * 16 / CST;      // xhat pieces (8 rows) per thread, rows <= 128
  constexpr int BPT = K * R / 8 / CST;   // bhat pieces (8 columns) per thread
  static_assert(XPT >= 1 && BPT >= 1, "tiling");
  using L = LdsC<NT, CK>;
  const int XP = cscan_xp(PK);
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* xs = (bf16*)(smem + L::xs(PK, g.cnb));
  bf16* bs = (bf16*)(smem + L::bs(PK, g.cnb));
  float* wv = (float*)(smem + L::wv(PK, g.cnb));  // per buffer: exp(a_last - a_j), j < ELL; then dec
  const int bmask = g.cnb - 1;                   // buffer of the chunk nc: (nc - n0) & bmask

  constexpr bool GS = GM == 1;  // group summaries
  const int bh = GM ? blockIdx.x / g.NGR : blockIdx.x, bi = bh / g.h, hi = bh % g.h;
  const int gi = GM ? blockIdx.x % g.NGR : 0;
  g.V = chain_len(g, bi);  // this sequence's valid length (per-sequence lengths)
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, q = lane >> 4;
  const int MT = PK / 16;
  const int xpr = PK / 8;  // xhat pieces per (j,c)
  const size_t pr = (size_t)g.p * g.r;

  struct Pf {
    u4 x[XPT];
    u4 b[BPT];
    float d;
  };
  auto fetch = [&](int nc) -> Pf {
    Pf f;
#pragma unroll
    for (int i = 0; i < XPT; i++) {
      f.x[i] = u4{0u, 0u, 0u, 0u};
      const int idx = tid + i * CST;
      const int k = idx / xpr, p0 = 8 * (idx % xpr);
      const int j = k / CK, ci = k % CK, pos = nc * ELL + j;
      if (k < K && p0 < g.p && ci < g.c && pos < g.V) {
        const bf16* src = xhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.p + p0;
        if ((g.p & 7) == 0) {
          f.x[i] = *reinterpret_cast<const u4*>(src);
        } else {
          unsigned short v[8];
#pragma unroll
          for (int e = 0; e < 8; e++) v[e] = p0 + e < g.p ? __builtin_bit_cast(unsigned short, src[e]) : 0;
          f.x[i] = __builtin_bit_cast(u4, v);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < BPT; i++) {
      f.b[i] = u4{0u, 0u, 0u, 0u};
      const int idx = tid + i * CST;
      const int k = idx / (R / 8), c0 = 8 * (idx % (R / 8));
      const int j = k / CK, ci = k % CK, pos = nc * ELL + j;
      if (c0 < g.r && ci < g.c && pos < g.V) {
        const bf16* src = bhat + ((((size_t)bi * g.s + pos) * g.c + ci) * g.h + hi) * g.r + c0;
        if ((g.r & 7) == 0) {
          f.b[i] = *reinterpret_cast<const u4*>(src);
        } else {
          unsigned short v[8];
#pragma unroll
          for (int e = 0; e < 8; e++) v[e] = c0 + e < g.r ? __builtin_bit_cast(unsigned short, src[e]) : 0;
          f.b[i] = __builtin_bit_cast(u4, v);
        }
      }
    }
    f.d = 0.0f;
    if (tid < ELL && nc * ELL + tid < g.V) f.d = (float)da[((size_t)bi * g.s + nc * ELL + tid) * g.h + hi];
    return f;
  };
  auto store = [&](const Pf& f, int buf) {
    bf16* xb = xs + (size_t)buf * K * XP;
    bf16* bb = bs + (size_t)buf * K * BP;
#pragma unroll
    for (int i = 0; i < XPT; i++) {
      const int idx = tid + i * CST;
      const int k = idx / xpr, p0 = 8 * (idx % xpr);
      if (k < K) *reinterpret_cast<u4*>(xb + k * XP + p0) = f.x[i];
    }
#pragma unroll
    for (int i = 0; i < BPT; i++) {
      const int idx = tid + i * CST;
      const int k = idx / (R / 8), c0 = 8 * (idx % (R / 8));
      *reinterpret_cast<u4*>(bb + k * BP + c0) = f.b[i];
    }
    if (tid < 64) {  // a_j = cumsum of da over the chunk; weights exp(a_last - a_j), dec = exp(a_last)
      float a = f.d;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        const float up = __shfl_up(a, off, 32);
        if ((tid & 31) >= off) a += up;
      }
      const float al = __shfl(a, 31, 32);
      if (tid < ELL) wv[buf * (ELL + 4) + tid] = expf(al - a);
      if (tid == 0) wv[buf * (ELL + 4) + ELL] = expf(al);
    }
  };

  // h_-(0) = h0, caller's column order
  static_assert(MTW >= 1 && MTW <= CMT, "row tiles per wave");
  f4 acc[MTW][NT];
#pragma unroll
  for (int mi = 0; mi < MTW; mi++)
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = 16 * (w + CSW * mi) + 4 * q + i, col = 16 * nt + m;
        acc[mi][nt][i] = (GM == 0 && h0 != nullptr && row < g.p && col < g.r)
                             ? (float)h0[((size_t)bh * g.p + row) * g.r + col] : 0.0f;
      }
  // 16-byte stores of four consecutive columns when the internal column order
  // is the caller's and the rows hold whole column tiles
  const bool vec_store = !g.half && g.r % 16 == 0;
  // internal position of this lane's columns (half-split interleaves the halves)
  int icol[NT];
#pragma unroll
  for (int nt = 0; nt < NT; nt++) icol[nt] = 16 * nt + m < g.r ? inv_perm_rc(g, 16 * nt + m) : 0;

  const int nkc = chain_nk(g);  // chunks walked (carries past them are not written)
  // chunks n0 .. n1-1: the whole walk, or a group (for summaries, one none of
  // whose chunks is the last)
  const int n0 = GM ? gi * g.G : 0;
  const int n1 = GM ? (n0 + g.G < nkc ? n0 + g.G : nkc) : nkc;
  if (GM && n0 >= nkc) return;
  if (GS && n1 >= nkc) return;
  if constexpr (GM == 2) {
    // the state entering the group, in the carry layout (internal column order)
    const float* in = carry + ((size_t)bh * g.NK + n0) * pr;
#pragma unroll
    for (int mi = 0; mi < MTW; mi++)
#pragma unroll
      for (int nt = 0; nt < NT; nt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int row = 16 * (w + CSW * mi) + 4 * q + i;
          acc[mi][nt][i] = row < g.p && 16 * nt + m < g.r ? in[(size_t)row * g.r + icol[nt]] : 0.0f;
        }
  }
  if (GS || (GM == 2 ? n0 + 1 < nkc : nkc > 1)) store(fetch(n0), 0);
  __syncthreads();
  float dprod = 1.0f;  // GS: product of the group's chunk decays
  for (int nc = n0; nc < n1; nc++) {
    // chunk nc+1 contributes U only if it is not the last (in a summarized
    // group it never is)
    const bool more = GS ? nc + 1 < n1 : (nc + 2 < nkc && nc + 1 < n1);
    Pf pf;
    if (more) pf = fetch(nc + 1);
    float* out = carry + ((size_t)bh * g.NK + nc) * pr;
#pragma unroll
    for (int mi = 0; mi < MTW; mi++) {
      const int mt = w + CSW * mi;
      if (GS || mt >= MT || nc % g.cstride != 0) break;
      if (vec_store) {
        // after a quad transpose lane (q, m) holds columns 16nt + 4(m / 4) ..
        // + 3 of row 16mt + 4q + m % 4: one 16-byte store per tile
        const int row = 16 * mt + 4 * q + (m & 3);
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
          f4 v = acc[mi][nt];
          quad_transpose(v, m & 3);
          if (row < g.p && 16 * nt < g.r)
            *reinterpret_cast<f4*>(out + (size_t)row * g.r + 16 * nt + 4 * (m >> 2)) = v;
        }
        continue;
      }
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        if (16 * nt + m >= g.r) continue;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int row = 16 * mt + 4 * q + i;
          if (row < g.p) out[(size_t)row * g.r + icol[nt]] = acc[mi][nt][i];
        }
      }
    }
    if (GS || nc + 1 < nkc) {
      const int b = (nc - n0) & bmask;
      const float* wb = wv + b * (ELL + 4);
      const float dn = wb[ELL];
      if (GS) dprod *= dn;
      else if (tid == 0) dec[(size_t)bh * g.NK + nc] = dn;
      const bf16* xb = xs + (size_t)b * K * XP;
      const bf16* bb = bs + (size_t)b * K * BP;
#pragma unroll
      for (int mi = 0; mi < MTW; mi++) {
        const int mt = w + CSW * mi;
        if (mt >= MT) break;
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
#pragma unroll
          for (int i = 0; i < 4; i++) acc[mi][nt][i] *= dn;
#pragma unroll
        for (int ks = 0; ks < NKS; ks++) {
          // A: rows of this tile, K-slot e weighted by exp(a_last - a_j) of its (j,c)
          const bf8 xr = ld_kx_frag(xb, XP, ks, 16 * mt, lane);
          bf8 a;
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const int k = 32 * ks + (e < 4 ? 4 * q + e : 16 + 4 * q + e - 4);
            a[e] = (bf16)(wb[k / CK] * (float)xr[e]);
          }
#pragma unroll
          for (int nt = 0; nt < NT; nt++)
            acc[mi][nt] = MM<bf16>::mma(a, ld_kx_frag(bb, BP, ks, 16 * nt, lane), acc[mi][nt]);
        }
      }
    }
    // one buffer: every wave is done reading it before the next chunk goes in
    if (bmask == 0 && more) __syncthreads();
    if (more) store(pf, (nc + 1 - n0) & bmask);
    __syncthreads();
  }
  if constexpr (GS) {
    float* out = carry + ((size_t)bh * g.NK + n0 + 1) * pr;
#pragma unroll
    for (int mi = 0; mi < MTW; mi++) {
      const int mt = w + CSW * mi;
      if (mt >= MT) break;
#pragma unroll
      for (int nt = 0; nt < NT; nt++) {
        if (16 * nt + m >= g.r) continue;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int row = 16 * mt + 4 * q + i;
          if (row < g.p) out[(size_t)row * g.r + icol[nt]] = acc[mi][nt][i];
        }
      }
    }
    if (tid == 0) dec[(size_t)bh * g.NK + n0 + 1] = dprod;
  }
}

// States entering the groups from the group summaries of k_cscan<.., true>:
// E_0 = h0 and E_{g+1} = D_g E_g + Z_g, element by element, written to the carry
// rows of each group's first chunk (carry layout: internal column order).
__global__ __launch_bounds__(NTH) void k_gentry(Geo g, const bf16* __restrict__ h0, float* carry,
                                                const float* __restrict__ dec) {
  const int bh = blockIdx.x, bi = bh / g.h;
  const size_t pr = (size_t)g.p * g.r;
  const size_t e = (size_t)blockIdx.y * NTH + threadIdx.x;
  if (e >= pr) return;
  g.V = chain_len(g, bi);
  const int nkc = chain_nk(g);
  const int row = (int)(e / g.r), ic = (int)(e % g.r);
  float E = h0 != nullptr ? (float)h0[((size_t)bh * g.p + row) * g.r + perm_rc(g, ic)] : 0.0f;
  for (int gi = 0; gi < g.NGR; gi++) {
    const int n0 = gi * g.G;
    if (n0 >= nkc) break;
    carry[((size_t)bh * g.NK + n0) * pr + e] = E;
    if (n0 + g.G >= nkc) break;  // the last group's summary is not formed
    const size_t zs = (size_t)bh * g.NK + n0 + 1;
    E = dec[zs] * E + carry[zs * pr + e];
  }
}

}  // namespace mom

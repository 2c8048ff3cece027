// Shared device helpers for the state-moments kernels (gfx950 / CDNA4).
//
// Notation follows the burn-mamba moments pages ("recalculated.rs" and
// "backward.rs" source pages): a kernel chunk holds ELL tokens t; inside it
// a_t = inclusive cumsum of da, d_t = exp(a_t), L[t,j] = exp(a_t - a_j) for
// j <= t (0 above the diagonal). The write axis (j,c) is folded into one index
// k = j*c + c_i, as the pages fold it for chunk_states.
//
// MFMA tiles are 16x16 with fp32 accumulators. A lane l of a wave64 holds:
//   A operand: row (l % 16), E consecutive K-slots starting at E*(l/16)
//   B operand: col (l % 16), the same K-slots
//   C/D      : col (l % 16), rows 4*(l/16) + i, i = 0..3
// Only the row/col placement matters to this code: every operand of one MFMA
// is loaded with the same slot -> k assignment, so any order of K inside an
// instruction gives the same sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mom {

constexpr int ELL = 32;   // tokens per kernel chunk (two 16-row MFMA tiles)
constexpr int NW = 4;     // waves per workgroup (forward, carry, correction kernels)
constexpr int NTH = 256;  // threads per workgroup (forward, carry, correction kernels)
constexpr int NTHB = 1024; // threads per workgroup of the backward main kernel (16 waves)
constexpr int NCW = 4;     // backward: waves sharing one state row (column quarters)

typedef float f4 __attribute__((ext_vector_type(4)));
template <int V> struct IC4 { static constexpr int value = V; };  // compile-time index tag
typedef __bf16 bf16;
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

template <typename T> struct MM;
template <> struct MM<float> {
  static constexpr int KS = 4;  // K per instruction
  static constexpr int E = 1;   // K-slots per lane
  using frag = float;
  __device__ static inline f4 mma(frag a, frag b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};
template <> struct MM<bf16> {
  static constexpr int KS = 32;
  static constexpr int E = 8;
  using frag = bf8;
  __device__ static inline f4 mma(frag a, frag b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T to_t(float x);
template <> __device__ __forceinline__ float to_t<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 to_t<bf16>(float x) { return (bf16)x; }

// Two floats -> one register of two bf16 (round to nearest even), kept as a
// 32-bit word so packed fragments are built once and reused.
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float fl2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pk_bf16(float lo, float hi) {
  const fl2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf2));
}
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ bf8 as_bf8(u4 v) { return __builtin_bit_cast(bf8, v); }

// Load one operand fragment (E consecutive elements, 4 or 16 bytes aligned).
__device__ __forceinline__ float ld_frag(const float* p) { return *p; }
__device__ __forceinline__ bf8 ld_frag(const bf16* p) { return *reinterpret_cast<const bf8*>(p); }

// Token of a K-slot when K runs over the ELL = 32 tokens of a chunk and the B
// operand comes straight from accumulator registers (rows 4q+i of tile mt):
//   bf16 (one K-step of 32): slot 8q+e -> t = 4q+e (e<4) or 16+4q+(e-4)
//   fp32 (eight K-steps of 4): slot 4s+q -> t = 16*(s/4) + 4q + (s%4)
template <typename T> __host__ __device__ __forceinline__ int tslot(int slot);
template <> __host__ __device__ __forceinline__ int tslot<bf16>(int slot) {
  const int q = slot >> 3, e = slot & 7;
  return e < 4 ? 4 * q + e : 16 + 4 * q + (e - 4);
}
template <> __host__ __device__ __forceinline__ int tslot<float>(int slot) {
  const int s = slot >> 2, q = slot & 3;
  return 16 * (s >> 2) + 4 * q + (s & 3);
}

// B fragment over the 32 tokens from accumulator registers v[mt] (one N tile).
__device__ __forceinline__ bf8 pack_tslots(const f4 (&v)[2], int /*ks*/, bf16) {
  bf8 f;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    f[e] = (bf16)v[0][e];
    f[e + 4] = (bf16)v[1][e];
  }
  return f;
}
__device__ __forceinline__ float pack_tslots(const f4 (&v)[2], int ks, float) { return v[ks >> 2][ks & 3]; }

// DPP lane exchange within a quad (row_mask/bank_mask all lanes).
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_amdgcn_update_dpp(0.0f, v, CTRL, 0xF, 0xF, false);
}
constexpr int QP_SWAP1 = 0xB1;  // quad_perm [1,0,3,2]: lane k gets lane k^1
constexpr int QP_X2 = 0x4E;     // quad_perm [2,3,0,1]: lane k gets lane k^2
constexpr int QP_X3 = 0x1B;     // quad_perm [3,2,1,0]: lane k gets lane k^3
constexpr int QP_B0 = 0x00, QP_B1 = 0x55, QP_B2 = 0xAA, QP_B3 = 0xFF;  // broadcast lane k of quad

constexpr int DPP_ROW_MIRROR = 0x140;       // lane i of a row <- lane 15 - i
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i of a half row <- lane 7 - i

// Sum over the 16 lanes of a row (lanes sharing l/16); every lane gets the sum.
// Quad sums first, then the two quads of each half row, then the two halves.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<QP_SWAP1>(v);
  v += dpp<QP_X2>(v);
  v += dpp<DPP_ROW_HALF_MIRROR>(v);
  v += dpp<DPP_ROW_MIRROR>(v);
  return v;
}
// Sum over the four lane groups (lanes sharing l%16), in registers: the
// gfx950 permlane swaps pair each 16-lane row with its neighbour (l ^ 16), then
// each half wave with the other (l ^ 32); both halves of a swap add the same
// two values, so every lane ends with the same sum.
__device__ __forceinline__ float col4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Order LDS traffic between lanes of one wave without a workgroup barrier.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Everything a kernel needs to know about the problem.
struct Geo {
  int b, s, c, h, p, r;
  int V;         // min(valid_len, s)
  int NK;        // processed kernel chunks: ceil(V / ELL)
  int K;         // ELL * c (folded write axis)
  int KP;        // LDS row length of K-contiguous tiles (elements)
  int RP;        // LDS row length of R-contiguous tiles (elements)
  int PP;        // LDS row length of P-contiguous tiles (elements)
  int P16;       // p rounded up to 16
  int rot_kind;  // 0 none, 1 pairwise, 2 half-split, 3 quaternion
  int A;         // angles per token (complex modes)
  int J;         // quaternion blocks
  int RW;        // last dim of rot per token: A or 4*J
  int G;         // chunks per workgroup (fwd/bwd main kernels)
  int NGR;       // workgroups per (b,h) chain: ceil(NK / G)
  int half;      // half-split: internal state column order interleaves the halves
  int cinv;      // ceil(65536 / c): j = (k * cinv) >> 16 for the folded index k < 65536 / c
  const int* lens;  // per-sequence valid lengths [b] (device), or nullptr: every sequence has V
  int pair;         // backward over token pairs: only odd tokens carry moments (see moments.hip)
  int skip;         // with per-sequence lengths: chunks past a sequence's length are not walked
                    // (set only when every kernel of the call skips them the same way)
  int cstride;      // the carry pass stores the state entering chunk n only for n % cstride == 0
                    // (1: every chunk; a forward that carries its state through each group of
                    // cstride chunks reads only the states entering the groups)
  int cnb;          // chunk staging buffers of the carry walk: 2 (the next chunk is staged
                    // while the current one is read), or 1 (one barrier more per chunk, half
                    // the LDS, so that two workgroups share a CU)
};

// Kernel chunks a sequence walks: all NK, or with `skip` only those holding a
// valid token of the sequence (g.V already holds its length).
__device__ __forceinline__ int chain_nk(const Geo& g) { return g.skip ? (g.V + ELL - 1) / ELL : g.NK; }

// Valid length of sequence bi: lens[bi] clamped to [0, V] (V bounds every
// sequence and sets the chunk count NK that sizes the grids and workspaces).
// Kernels that mask by position replace g.V with it once bi is known; chunks
// past a sequence's length then hold no valid token and contribute exact zeros.
__device__ __forceinline__ int chain_len(const Geo& g, int bi) {
  if (g.lens == nullptr) return g.V;
  const int v = g.lens[bi];
  return v < 0 ? 0 : (v < g.V ? v : g.V);
}

// Internal state-column order. Half-split pairs (i, r/2+i) are stored next to
// each other (internal 2i, 2i+1) so every complex mode rotates adjacent columns.
__device__ __forceinline__ int perm_rc(const Geo& g, int rc) {
  return g.half ? ((rc & 1) ? (g.r >> 1) + (rc >> 1) : (rc >> 1)) : rc;
}
__device__ __forceinline__ int inv_perm_rc(const Geo& g, int ra) {
  if (!g.half) return ra;
  const int hr = g.r >> 1;
  return ra < hr ? 2 * ra : 2 * (ra - hr) + 1;
}

__host__ __device__ __forceinline__ size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace mom

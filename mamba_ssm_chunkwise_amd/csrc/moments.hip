// C ABI of the state-moments library: validation, planning, dispatch.
// The operation and its conventions are stated in include/moments.h.
#include "moments.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <type_traits>
#include <mutex>
#include <vector>

#include "kernels_bwd.h"
#include "kernels_bwdt.h"
#include "kernels_fwdt.h"
#include "kernels_cscan.h"
#include "kernels_fwd4.h"
#include "kernels_reduce.h"
#include "kernels_rot.h"
#include "fwd4_launch.h"

using namespace mom;

// Device scratch of the allocation-free forward (moments_fwd_static): one copy
// per GPU, alive until the process ends. Host code never passes this name to a
// kernel or a copy; it uses the address hipGetSymbolAddress returns for the
// current device (static_scratch below).
__device__ __align__(256) unsigned char scratch[MOMENTS_STATIC_SCRATCH_BYTES];

namespace {

std::atomic<int> g_last_hip{0};

constexpr size_t kLdsLimit = 160 * 1024;
constexpr long kCUs = 256;  // compute units of the part (MI355X)

// ---- optional per-kernel event timing (moments_profile_*) -------------------
enum KernelId {
  KID_CARRY, KID_SCAN, KID_FWD, KID_REDUCE, KID_BWD, KID_DSCAN, KID_FIX, KID_ZERO, KID_PREP, KID_GSCAN, KID_GFIX,
  KID_CSCAN, KID_ROTSEG, KID_ROTCARRY, KID_ROTAPPLY, KID_PAIR, KID_GENTRY, KID_CSUM, KID_CGRP, KID_N
};
const char* const kKernelNames[KID_N] = {"k_carry", "k_scan",      "k_fwd",      "k_reduce", "k_bwd",  "k_dscan",
                                         "k_fix",   "k_zero_tail", "k_prep_dm1", "k_gscan",  "k_gfix",
                                         "k_cscan", "k_rot_seg",   "k_rot_carry", "k_rot_apply",
                                         "k_pair",  "k_gentry",    "k_cscan_sum", "k_cscan_grp"};
struct Prof {
  std::mutex mu;
  bool on = false;
  struct Rec { int kid; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  double ms[KID_N] = {};
  int64_t n[KID_N] = {};
};
Prof& prof() {
  static Prof p;
  return p;
}
hipEvent_t prof_event() {
  Prof& P = prof();
  if (!P.pool.empty()) {
    hipEvent_t e = P.pool.back();
    P.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
// Brackets one launch with events when profiling is on.
struct ProfScope {
  int kid;
  hipStream_t st;
  hipEvent_t a = nullptr;
  ProfScope(int k, hipStream_t s) : kid(k), st(s) {
    Prof& P = prof();
    std::lock_guard<std::mutex> g(P.mu);
    if (P.on && (a = prof_event()) != nullptr) (void)hipEventRecord(a, st);
  }
  ~ProfScope() {
    if (a == nullptr) return;
    Prof& P = prof();
    std::lock_guard<std::mutex> g(P.mu);
    hipEvent_t b = prof_event();
    if (b == nullptr) return;
    (void)hipEventRecord(b, st);
    P.pending.push_back({kid, a, b});
  }
};

template <int V> using IC = std::integral_constant<int, V>;
template <typename T> struct TT { using type = T; };

struct Plan {
  Geo g;
  bool bf;      // bf16 inputs
  int CK;       // channel slots of the folded write axis (c padded to 1, 2 or 4)
  int NT, R;    // state columns padded to R = 16*NT
  int PK;       // state rows padded for MFMA K over rows
  bool bwdt;    // backward main kernel in the transposed layout (bf16, c <= 2)
  bool fwdt;    // forward main kernel in the transposed layout (bf16, c <= 2)
  bool fwdt_inc;  // ... carrying the state rows itself (one group per chain): no carry pass
  bool fwd4;      // forward main kernel in the lane-pair layout (bf16, p <= 128)
  bool fwd4_inc;  // ... carrying the state rows itself
  size_t carry, dec, m2p, m1p, db, dm1i, gdb;  // workspace offsets
  size_t ws_fwd, ws_bwd;
  size_t saved;  // bytes of the saved carries: states [chains][NK][p][r], then decays [chains][NK]
  size_t flag_fwd, flag_bwd;  // the finiteness check's flag (last 256 bytes of each workspace)
  // backward over token pairs (bf16, c == 4): workspace regions after the pair
  // plan's own workspace (pair-token da, rot, their gradients, lengths)
  bool pair;
  bool po;  // ... with every wave on the odd pair tokens (eight state rows a round)
  size_t pr_da2, pr_rot2, pr_dda2, pr_drot2, pr_lens2;
};

int round_nt(int r, bool /*bf*/) {
  int nt = (r + 15) / 16;
  if (nt <= 4) nt = 4;
  else nt = 8;
  return nt;
}

// LDS bytes of k_fwdt for (NT, CK), or 0 when that kernel does not cover the shape.
size_t fwdt_lds(const Geo& g, int NT, int CK) {
  const int RT = rot_tiles(g);
  if (g.p > 128) return 0;  // m1 accumulators cover 32 rounds of 4 rows
  if (NT == 4 && CK == 1) return LdsF<4, 1>::total(RT, g.p);
  if (NT == 4 && CK == 2) return LdsF<4, 2>::total(RT, g.p);
  if (NT == 8 && CK == 1) return LdsF<8, 1>::total(RT, g.p);
  if (NT == 8 && CK == 2) return LdsF<8, 2>::total(RT, g.p);
  return 0;
}

// LDS bytes of k_fwd4 for (NT, CK), or 0 when that kernel does not cover the shape.
size_t fwd4_lds(const Geo& g, int NT, int CK, bool inc) {
  if (g.p > 128) return 0;  // m1 accumulators: 32 rows per wave
  const int RG = rot_groups(g), pp = 4 * ((g.p + 3) / 4), rk = g.rot_kind == 3 ? 3 : 1;
  if (NT == 4 && RG * (rk == 3 ? 4 : 2) > 4) return 0;
  if (NT == 4 && CK == 1) return LdsF4<4, 1>::total(pp, rk, RG, inc);
  if (NT == 4 && CK == 2) return LdsF4<4, 2>::total(pp, rk, RG, inc);
  if (NT == 4 && CK == 4) return LdsF4<4, 4>::total(pp, rk, RG, inc);
  if (NT == 8 && CK == 1) return LdsF4<8, 1>::total(pp, rk, RG, inc);
  if (NT == 8 && CK == 2) return LdsF4<8, 2>::total(pp, rk, RG, inc);
  if (NT == 8 && CK == 4) return LdsF4<8, 4>::total(pp, rk, RG, inc);
  return 0;
}

// LDS bytes of k_bwdt for (NT, CK) (po: the odd-pair-token variant), or 0 when
// that kernel does not cover the shape.
size_t bwdt_lds(const Geo& g, int NT, int CK, bool po = false) {
  const int RT = rot_tiles(g);
  auto one = [&](auto lt) -> size_t {
    using LT = typename decltype(lt)::type;
    return LT::fits(g.rot_kind, RT) ? LT::total(RT, g.rot_kind) : 0;
  };
  if (po) {
    if (NT == 4 && CK == 2) return one(TT<LdsT<4, 2, true>>{});
    if (NT == 8 && CK == 2) return one(TT<LdsT<8, 2, true>>{});
    return 0;
  }
  if (NT == 4 && CK == 1) return one(TT<LdsT<4, 1>>{});
  if (NT == 4 && CK == 2) return one(TT<LdsT<4, 2>>{});
  if (NT == 8 && CK == 1) return one(TT<LdsT<8, 1>>{});
  if (NT == 8 && CK == 2) return one(TT<LdsT<8, 2>>{});
  return 0;
}

int make_plan(const moments_desc* d, Plan* P);

// Plan of the token-pair backward: 2s tokens of two channels each, twice the
// valid length; per-sequence lengths are doubled on the device (lens2).
int make_pair_plan(const moments_desc* d, Plan* Pv) {
  moments_desc v = *d;
  const int64_t V = d->valid_len < d->s ? d->valid_len : d->s;
  v.s = 2 * d->s;
  v.c = 2;
  v.chunk_len = 2 * d->chunk_len;
  v.valid_len = 2 * V;
  v.valid_lens = nullptr;
  const int rc = make_plan(&v, Pv);
  if (rc != MOMENTS_OK) return rc;
  Pv->g.pair = 1;
  // the transposed backward walks token pairs in its odd-pair-token form only
  const size_t lpo = bwdt_lds(Pv->g, Pv->NT, Pv->CK, true);
  Pv->po = Pv->bwdt && lpo > 0 && lpo <= kLdsLimit;
  Pv->bwdt = Pv->po;
  return MOMENTS_OK;
}

int make_plan(const moments_desc* d, Plan* P) {
  if (d == nullptr) return MOMENTS_EINVAL;
  if (d->b < 1 || d->s < 1 || d->c < 1 || d->h < 1 || d->p < 1 || d->r < 1) return MOMENTS_EINVAL;
  if (d->chunk_len < 1 || d->s % d->chunk_len != 0) return MOMENTS_EINVAL;
  if (d->valid_len < 0) return MOMENTS_EINVAL;
  if (d->dtype != MOMENTS_F32 && d->dtype != MOMENTS_BF16) return MOMENTS_EINVAL;
  int A = 0, J = 0, RW = 0;
  switch (d->rot_kind) {
    case MOMENTS_ROT_NONE:
      break;
    case MOMENTS_ROT_COMPLEX_PAIRWISE:
    case MOMENTS_ROT_COMPLEX_HALF:
      if (d->rope_dim < 0 || d->rope_dim % 2 != 0 || d->rope_dim > d->r) return MOMENTS_EINVAL;
      if (d->rot_kind == MOMENTS_ROT_COMPLEX_HALF && d->r % 2 != 0) return MOMENTS_EINVAL;
      A = (int)(d->rope_dim / 2);
      RW = A;
      break;
    case MOMENTS_ROT_QUATERNION:
      if (d->quat_blocks < 0 || 4 * d->quat_blocks > d->r) return MOMENTS_EINVAL;
      J = (int)d->quat_blocks;
      RW = 4 * J;
      break;
    default:
      return MOMENTS_EINVAL;
  }
  if (d->r > 128 || d->c > 4) return MOMENTS_ENOTSUP;
  if (d->s > (int64_t)1 << 30 || d->p > 4096 || d->b * d->h > ((int64_t)1 << 30)) return MOMENTS_ENOTSUP;

  const bool bf = d->dtype == MOMENTS_BF16;
  const int tsz = bf ? 2 : 4, pad = 16 / tsz;
  Geo& g = P->g;
  g = Geo{};
  g.b = (int)d->b; g.s = (int)d->s; g.c = (int)d->c; g.h = (int)d->h; g.p = (int)d->p; g.r = (int)d->r;
  g.V = (int)(d->valid_len < d->s ? d->valid_len : d->s);
  g.NK = (g.V + ELL - 1) / ELL;
  g.cstride = 1;
  g.cnb = 2;
  P->bf = bf;
  P->CK = g.c <= 1 ? 1 : g.c <= 2 ? 2 : 4;
  g.K = ELL * P->CK;
  P->NT = round_nt(g.r, bf);
  if (!bf && P->NT > 4) return MOMENTS_ENOTSUP;  // float32 kernels cover r <= 64
  P->R = 16 * P->NT;
  const int kq = bf ? 32 : 16;
  P->PK = ((g.p + kq - 1) / kq) * kq;
  g.KP = g.K + pad;
  g.RP = P->R + pad;
  g.PP = P->PK + pad;
  g.P16 = P->PK;
  g.rot_kind = d->rot_kind;
  g.A = A; g.J = J; g.RW = RW;
  g.half = d->rot_kind == MOMENTS_ROT_COMPLEX_HALF;
  g.cinv = (65536 + g.c - 1) / g.c;
  g.lens = (const int*)d->valid_lens;
  const int64_t chains = (int64_t)g.b * g.h;
  const int64_t total = chains * g.NK;
  // chunks per workgroup of the main kernels: about 512 workgroups (two per
  // CU at one resident workgroup each), fewer groups meaning fewer partial
  // moments and group fix-ups
  int G = (int)((total + 511) / 512);
  if (G < 1) G = 1;
  if (g.NK > 0 && G > g.NK) G = g.NK;
  g.G = G;
  g.NGR = g.NK > 0 ? (g.NK + G - 1) / G : 0;

  if (lds_fwd(g, P->R, tsz, P->NT).total > kLdsLimit || lds_bwd(g, P->R, tsz, P->NT).total > kLdsLimit ||
      lds_carry(g, P->R, tsz, P->PK).total > kLdsLimit || lds_fix(g, P->R, tsz, P->PK).total > kLdsLimit)
    return MOMENTS_ENOTSUP;

  const size_t pr = (size_t)g.p * g.r;
  size_t o = 0;
  P->carry = o; o = align256(o + chains * (size_t)g.NK * pr * 4);
  P->dec = o; o = align256(o + chains * (size_t)g.NK * 4);
  P->saved = o;  // the same two regions, at the same offsets, in the caller's buffer
  const size_t base = o;
  P->m2p = o; o = align256(o + chains * (size_t)g.NGR * NW4 * P->R * P->R * 4);  // per wave for k_fwd4
  P->m1p = o; o = align256(o + chains * (size_t)g.NGR * g.p * P->R * 4);
  P->flag_fwd = o;
  o += 256;
  P->ws_fwd = o;
  P->db = base;
  o = align256(base + chains * (size_t)g.NK * pr * 4);
  if (bf) {
    const size_t l4 = fwd4_lds(g, P->NT, P->CK, false);
    P->fwd4 = l4 > 0 && l4 <= kLdsLimit;
    P->fwd4_inc = P->fwd4 && g.NGR == 1 && fwd4_lds(g, P->NT, P->CK, true) <= kLdsLimit;
  } else {
    P->fwd4 = false;
    P->fwd4_inc = false;
  }
  if (bf && P->CK <= 2) {
    const size_t lf = fwdt_lds(g, P->NT, P->CK);
    P->fwdt = lf > 0 && lf <= kLdsLimit;
    P->fwdt_inc = P->fwdt && g.NGR == 1 && lf + (size_t)g.p * P->R * 4 <= kLdsLimit;
  } else {
    P->fwdt = false;
    P->fwdt_inc = false;
  }
  P->po = false;
  if (bf && P->CK <= 2) {
    const size_t lb = bwdt_lds(g, P->NT, P->CK);
    P->bwdt = lb > 0 && lb <= kLdsLimit;
  } else {
    P->bwdt = false;
  }
  P->dm1i = o;
  if (P->bwdt) o = align256(o + chains * (size_t)g.p * P->R * 4);
  P->gdb = o;  // per-group boundary cotangents of the transposed backward
  if (P->bwdt) o = align256(o + chains * (size_t)g.NGR * pr * 4);
  P->flag_bwd = o;
  o += 256;
  P->ws_bwd = o;
  P->pair = false;
  if (bf && d->c == 4) {
    // four channels: the backward walks token pairs of two channels each with the
    // transposed kernel (the general kernel's registers do not hold four channels)
    Plan Pv;
    if (make_pair_plan(d, &Pv) == MOMENTS_OK && Pv.bwdt) {
      const size_t tok = (size_t)g.b * g.s;
      size_t q = align256(Pv.ws_bwd);
      P->pr_da2 = q; q = align256(q + 2 * tok * g.h * 2);
      P->pr_rot2 = q; q = align256(q + 2 * tok * g.h * g.RW * 2);
      P->pr_dda2 = q; q = align256(q + 2 * tok * g.h * 2);
      P->pr_drot2 = q; q = align256(q + 2 * tok * g.h * g.RW * 2);
      P->pr_lens2 = q; q = align256(q + (size_t)g.b * 4);
      P->flag_bwd = q;
      P->ws_bwd = q + 256;
      P->pair = true;
    }
  }
  return MOMENTS_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int hip_fail(hipError_t e) {
  g_last_hip.store((int)e);
  return MOMENTS_EHIP;
}

template <typename K>
int set_lds(K kernel, size_t bytes) {
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  return e == hipSuccess ? 0 : hip_fail(e);
}

int check_launch() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : hip_fail(e);
}

#define MOM_TRY(x)          \
  do {                      \
    const int _rc = (x);    \
    if (_rc != 0) return _rc; \
  } while (0)

// The carry walk's group forms with `grid` workgroups: one staging buffer when
// that lets two workgroups share a CU where two double-buffered ones would not
// fit, and the grid has more workgroups than one per CU (the long-context shape:
// 148 KB double-buffered, 74 KB single).
template <int NT, int CK>
Geo cscan_geo(const Plan& P, long grid) {
  Geo g = P.g;
  const size_t l2 = LdsC<NT, CK>::total(P.PK, 2), l1 = LdsC<NT, CK>::total(P.PK, 1);
  g.cnb = (2 * l2 > kLdsLimit && 2 * l1 <= kLdsLimit && grid > kCUs) ? 1 : 2;
  return g;
}

// The states entering each group: per-group walks from a zero state (k_cscan
// in its group-summary form, in parallel over the groups) and a scan over the
// groups (k_gentry), into each group's first carry rows. Needs groups of two
// chunks or more; returns MOMENTS_ENOTSUP when k_cscan does not cover the shape.
template <int NT, int CK>
int launch_group_entries(const Plan& P, const bf16* xhat, const bf16* bhat, const bf16* da, const bf16* h0,
                         float* carry, float* dec, hipStream_t st) {
  const int chains = P.g.b * P.g.h;
  const Geo g = cscan_geo<NT, CK>(P, (long)chains * P.g.NGR);
  const size_t lds = LdsC<NT, CK>::total(P.PK, g.cnb);
  if (g.G < 2 || g.NGR < 2 || P.PK > 16 * CSW * CMT || lds > kLdsLimit) return MOMENTS_ENOTSUP;
  auto launch = [&](auto mtw_c) -> int {
    constexpr int MTW = decltype(mtw_c)::value;
    MOM_TRY(set_lds(k_cscan<NT, CK, MTW, 1>, lds));
    ProfScope ps(KID_CSUM, st);
    hipLaunchKernelGGL((k_cscan<NT, CK, MTW, 1>), dim3(chains * g.NGR), dim3(CST), lds, st, g, P.PK, xhat, bhat,
                       da, h0, carry, dec);
    return check_launch();
  };
  MOM_TRY(P.PK <= 16 * CSW ? launch(IC<1>{}) : launch(IC<2>{}));
  const size_t pr = (size_t)g.p * g.r;
  ProfScope ps(KID_GENTRY, st);
  hipLaunchKernelGGL(k_gentry, dim3(chains, (unsigned)((pr + NTH - 1) / NTH)), dim3(NTH), 0, st, g, h0, carry,
                     (const float*)dec);
  return check_launch();
}

// The carry pass: states entering every kernel chunk (carry) and chunk decays
// (dec), into the workspace or the caller's saved-carry buffer.
template <typename T, int NT, int CK>
int launch_carry_scan(const Plan& P, const T* xhat, const T* bhat, const T* da, const T* h0,
                      float* carry, float* dec, hipStream_t st) {
  const Geo& g = P.g;
  const int chains = g.b * g.h;
  if constexpr (std::is_same<T, bf16>::value) {
    const size_t lds = LdsC<NT, CK>::total(P.PK, g.cnb);
    // with groups of two chunks or more: the states entering the groups, then
    // every group walked from its entering state, in parallel over the groups
    if (g.cstride == 1 && g.NK >= 1) {
      const int rc = launch_group_entries<NT, CK>(P, xhat, bhat, da, h0, carry, dec, st);
      if (rc != MOMENTS_ENOTSUP) {
        MOM_TRY(rc);
        const Geo gg = cscan_geo<NT, CK>(P, (long)chains * g.NGR);
        const size_t lg = LdsC<NT, CK>::total(P.PK, gg.cnb);
        auto launch = [&](auto mtw_c) -> int {
          constexpr int MTW = decltype(mtw_c)::value;
          MOM_TRY(set_lds(k_cscan<NT, CK, MTW, 2>, lg));
          ProfScope ps(KID_CGRP, st);
          hipLaunchKernelGGL((k_cscan<NT, CK, MTW, 2>), dim3(chains * g.NGR), dim3(CST), lg, st, gg, P.PK, xhat,
                             bhat, da, h0, carry, dec);
          return check_launch();
        };
        return P.PK <= 16 * CSW ? launch(IC<1>{}) : launch(IC<2>{});
      }
    }
    // one sequential walk per chain when there are enough chains to fill the
    // chip (or the chains are short); otherwise the chunk-parallel pair below
    if (g.NK >= 1 && P.PK <= 16 * CSW * CMT && lds <= kLdsLimit && (chains >= 64 || g.NK <= 32)) {
      auto launch = [&](auto mtw_c) -> int {
        constexpr int MTW = decltype(mtw_c)::value;
        MOM_TRY(set_lds(k_cscan<NT, CK, MTW>, lds));
        ProfScope ps(KID_CSCAN, st);
        hipLaunchKernelGGL((k_cscan<NT, CK, MTW>), dim3(chains), dim3(CST), lds, st, g, P.PK, xhat, bhat, da, h0,
                           carry, dec);
        return check_launch();
      };
      return P.PK <= 16 * CSW ? launch(IC<1>{}) : launch(IC<2>{});
    }
  }
  if (g.NK >= 2) {
    const size_t lds = lds_carry(g, P.R, sizeof(T), P.PK).total;
    MOM_TRY(set_lds(k_carry<T, NT, CK>, lds));
    ProfScope ps(KID_CARRY, st);
    hipLaunchKernelGGL((k_carry<T, NT, CK>), dim3(chains * (g.NK - 1)), dim3(NTH), lds, st, g, P.PK, xhat,
                       bhat, da, carry, dec);
    MOM_TRY(check_launch());
  }
  if (g.NK >= 1) {
    const int pr = g.p * g.r;
    ProfScope ps(KID_SCAN, st);
    if (pr % 4 == 0)
      hipLaunchKernelGGL((k_scan4<T>), dim3(chains, (pr / 4 + NTH - 1) / NTH), dim3(NTH), 0, st, g, h0, carry,
                         dec);
    else
      hipLaunchKernelGGL((k_scan<T>), dim3(chains, (pr + NTH - 1) / NTH), dim3(NTH), 0, st, g, h0, carry,
                         dec);
    MOM_TRY(check_launch());
  }
  return 0;
}

// saved != nullptr: also leave the carries and chunk decays in the caller's
// buffer (the carrying kernels write them; otherwise the carry pass writes there).
template <typename T, int NT, int ROT, int CK>
int run_fwd(const Plan& P0, const void* xhat, const void* bhat, const void* da, const void* rot,
            const void* h0, float* m2, float* m1, unsigned char* ws, unsigned char* saved, hipStream_t st) {
  // with per-sequence lengths the lane-pair forward and its carry pass skip the
  // chunks past each sequence (a saved buffer then holds only the walked chunks,
  // which only the transposed backward reads alike)
  Plan P = P0;
  P.g.skip = P.g.lens != nullptr && std::is_same<T, bf16>::value && P.fwd4 && (saved == nullptr || P.bwdt);
  const Geo& g = P.g;
  unsigned char* cbase = saved != nullptr ? saved : ws;
  float* carry = (float*)(cbase + P.carry);
  float* dec = (float*)(cbase + P.dec);
  const T* X = (const T*)xhat;
  const T* B = (const T*)bhat;
  const T* D = (const T*)da;
  const T* Rt = (const T*)rot;
  float* m2p = (float*)(ws + P.m2p);
  float* m1p = (float*)(ws + P.m1p);
  const int chains = g.b * g.h;
  if constexpr (std::is_same<T, bf16>::value) {
    if (P.fwd4) {
      // A forward over several groups per chain, with no saved buffer, carries
      // its state rows through each group in LDS when they fit there; its carry
      // pass then stores only the states entering the groups.
      const bool grp_inc =
          !P.fwd4_inc && saved == nullptr && g.NGR > 1 && fwd4_lds(g, P.NT, P.CK, true) <= kLdsLimit;
      if (!P.fwd4_inc) {
        // the group entries from per-group summaries where they apply, else a
        // carry pass that stores only those entries (or, without grp_inc, all)
        const int rc = grp_inc ? launch_group_entries<NT, CK>(P, X, B, D, (const T*)h0, carry, dec, st)
                               : MOMENTS_ENOTSUP;
        if (rc == MOMENTS_ENOTSUP) {
          Plan Pc = P;
          if (grp_inc) Pc.g.cstride = g.G;
          MOM_TRY((launch_carry_scan<T, NT, CK>(Pc, X, B, D, (const T*)h0, carry, dec, st)));
        } else {
          MOM_TRY(rc);
        }
      }
      const int RG = rot_groups(g);
      auto launch = [&](auto rot_c, auto rg_c) -> int {
        constexpr int RO = decltype(rot_c)::value, RGc = decltype(rg_c)::value;
        if constexpr (RGc * (RO == 3 ? 4 : 2) > NT) {
          return MOMENTS_ENOTSUP;
        } else {
          const size_t lds = fwd4_lds(g, NT, CK, P.fwd4_inc || grp_inc);
          if (g.NK >= 1) {
            auto go = [&](auto m1t_c, auto inc_c) -> int {
              constexpr int M1 = decltype(m1t_c)::value;
              constexpr int INC = decltype(inc_c)::value;
              ProfScope ps(KID_FWD, st);
              const hipError_t e = launch_fwd4<NT, RO, CK, RGc, M1, INC>(
                  g, lds, (unsigned)(chains * g.NGR), st, X, B, D, Rt,
                  INC == 0 || INC == 3 ? (const float*)carry : nullptr,
                  (const T*)h0, m2p, m1p, INC == 2 ? carry : nullptr, INC == 2 ? dec : nullptr);
              return e == hipSuccess ? 0 : hip_fail(e);
            };
            if (P.fwd4_inc && saved != nullptr) MOM_TRY(g.p <= 64 ? go(IC<1>{}, IC<2>{}) : go(IC<2>{}, IC<2>{}));
            else if (P.fwd4_inc) MOM_TRY(g.p <= 64 ? go(IC<1>{}, IC<1>{}) : go(IC<2>{}, IC<1>{}));
            else if (grp_inc) MOM_TRY(g.p <= 64 ? go(IC<1>{}, IC<3>{}) : go(IC<2>{}, IC<3>{}));
            else MOM_TRY(g.p <= 64 ? go(IC<1>{}, IC<0>{}) : go(IC<2>{}, IC<0>{}));
          }
          const int nout = P.R * P.R + g.p * P.R;
          ProfScope ps(KID_REDUCE, st);
          hipLaunchKernelGGL(k_reduce4, dim3(chains, (nout + NTH - 1) / NTH), dim3(NTH), 0, st, g, P.R,
                             RGc > 0 ? RO : 0, (const float*)m2p, (const float*)m1p, m2, m1);
          return check_launch();
        }
      };
      if constexpr (ROT == 0) {
        return launch(IC<0>{}, IC<0>{});
      } else {
        if (RG == 0) return launch(IC<0>{}, IC<0>{});
        if (RG == 1) return launch(IC<ROT>{}, IC<1>{});
        if (RG == 2) return launch(IC<ROT>{}, IC<2>{});
        if (RG == 4) return launch(IC<ROT>{}, IC<4>{});
        return MOMENTS_ENOTSUP;
      }
    }
  }
  // the transposed carrying forward keeps no carries: with `saved` the carry pass runs
  const bool fwdt_inc = P.fwdt_inc && saved == nullptr;
  if (!fwdt_inc) MOM_TRY((launch_carry_scan<T, NT, CK>(P, X, B, D, (const T*)h0, carry, dec, st)));
  bool done = false;
  if constexpr (std::is_same<T, bf16>::value && CK <= 2) {
    if (P.fwdt && g.NK >= 1) {
      const int RT = rot_tiles(g);
      auto launch = [&](auto rot_c, auto rt_c) -> int {
        constexpr int RO = decltype(rot_c)::value, RTc = decltype(rt_c)::value;
        const size_t lds = fwdt_inc ? LdsF<NT, CK>::total_inc(RTc, g.p) : LdsF<NT, CK>::total(RTc, g.p);
        MOM_TRY(set_lds(k_fwdt<NT, RO, CK, RTc>, lds));
        ProfScope ps(KID_FWD, st);
        hipLaunchKernelGGL((k_fwdt<NT, RO, CK, RTc>), dim3(chains * g.NGR), dim3(NTT), lds, st, g, X, B, D, Rt,
                           fwdt_inc ? nullptr : (const float*)carry, (const T*)h0, m2p, m1p);
        return check_launch();
      };
      int rc = MOMENTS_ENOTSUP;
      if constexpr (ROT == 0) {
        rc = launch(IC<0>{}, IC<0>{});
      } else {
        if (RT == 0) rc = launch(IC<0>{}, IC<0>{});
        else if (RT == 1) rc = launch(IC<ROT>{}, IC<1>{});
        else if (RT == 2) rc = launch(IC<ROT>{}, IC<2>{});
        else if (RT == 4) rc = launch(IC<ROT>{}, IC<4>{});
        else if (RT == 8) {
          if constexpr (NT >= 8) rc = launch(IC<ROT>{}, IC<8>{});
        }
      }
      MOM_TRY(rc);
      done = true;
    }
  }
  if (!done && g.NK >= 1) {
    const size_t lds = lds_fwd(g, P.R, sizeof(T), P.NT).total;
    MOM_TRY(set_lds(k_fwd<T, NT, ROT, CK>, lds));
    ProfScope ps(KID_FWD, st);
    hipLaunchKernelGGL((k_fwd<T, NT, ROT, CK>), dim3(chains * g.NGR), dim3(NTH), lds, st, g, X, B, D, Rt,
                       (const float*)carry, m2p, m1p);
    MOM_TRY(check_launch());
  }
  {
    const int nout = g.r * g.r + g.p * g.r;
    ProfScope ps(KID_REDUCE, st);
    hipLaunchKernelGGL(k_reduce, dim3(chains, (nout + NTH - 1) / NTH), dim3(NTH), 0, st, g, P.R,
                       (const float*)m2p, (const float*)m1p, m2, m1);
  }
  return check_launch();
}

template <typename T, int NT, int ROT, int CK>
int run_bwd(const Plan& P0, const void* xhat, const void* bhat, const void* da, const void* rot,
            const void* h0, const float* dm2, const float* dm1, void* dx, void* db, void* dda,
            void* drot, void* dh0, unsigned char* ws, const unsigned char* saved, hipStream_t st) {
  // with per-sequence lengths the transposed path (carry pass, walk, group
  // fix-ups, zero fill) skips the chunks past each sequence
  Plan P = P0;
  P.g.skip = P.g.lens != nullptr && std::is_same<T, bf16>::value && CK <= 2 && P.bwdt && P.g.NK >= 1;
  const Geo& g = P.g;
  const T* X = (const T*)xhat;
  const T* B = (const T*)bhat;
  const T* D = (const T*)da;
  const T* Rt = (const T*)rot;
  // the carries come from the caller's saved buffer, or from the carry pass
  float* carry = saved != nullptr ? (float*)(saved + P.carry) : (float*)(ws + P.carry);
  float* dec = saved != nullptr ? (float*)(saved + P.dec) : (float*)(ws + P.dec);
  if (saved == nullptr) MOM_TRY((launch_carry_scan<T, NT, CK>(P, X, B, D, (const T*)h0, carry, dec, st)));
  float* Db = (float*)(ws + P.db);
  const int chains = g.b * g.h;
  bool done = false;
  if constexpr (std::is_same<T, bf16>::value && CK <= 2) {
    if (P.bwdt && g.NK >= 1) {
      float* dm1i = (float*)(ws + P.dm1i);
      {
        const size_t total = (size_t)chains * g.p * P.R;
        ProfScope ps(KID_PREP, st);
        hipLaunchKernelGGL(k_prep_dm1, dim3((unsigned)((total + NTH - 1) / NTH)), dim3(NTH), 0, st, g, P.R, dm1,
                           dm1i);
        MOM_TRY(check_launch());
      }
      const int RT = rot_tiles(g);
      auto launch = [&](auto rot_c, auto rt_c) -> int {
        constexpr int RO = decltype(rot_c)::value, RTc = decltype(rt_c)::value;
        if constexpr (CK == 2) {
          if (P.po) {  // token pairs: every wave on the odd pair tokens
            const size_t lds = LdsT<NT, CK, true>::total(RTc, RO);
            MOM_TRY(set_lds(k_bwdt<NT, RO, CK, RTc, true>, lds));
            ProfScope ps(KID_BWD, st);
            hipLaunchKernelGGL((k_bwdt<NT, RO, CK, RTc, true>), dim3(chains * g.NGR), dim3(NTT), lds, st, g, X, B, D,
                               Rt, (const float*)carry, dm2, (const float*)dm1i, Db, (T*)dx, (T*)db, (T*)dda, (T*)drot);
            return check_launch();
          }
        }
        if (P.g.pair) return MOMENTS_ENOTSUP;  // token pairs run the odd-pair-token form above
        const size_t lds = LdsT<NT, CK>::total(RTc, RO);
        MOM_TRY(set_lds(k_bwdt<NT, RO, CK, RTc>, lds));
        ProfScope ps(KID_BWD, st);
        hipLaunchKernelGGL((k_bwdt<NT, RO, CK, RTc>), dim3(chains * g.NGR), dim3(NTT), lds, st, g, X, B, D, Rt,
                           (const float*)carry, dm2, (const float*)dm1i, Db, (T*)dx, (T*)db, (T*)dda, (T*)drot);
        return check_launch();
      };
      int rc = MOMENTS_ENOTSUP;
      if constexpr (ROT == 0) {
        rc = launch(IC<0>{}, IC<0>{});
      } else {
        if (RT == 0) rc = launch(IC<0>{}, IC<0>{});
        else if (RT == 1) rc = launch(IC<ROT>{}, IC<1>{});
        else if (RT == 2) rc = launch(IC<ROT>{}, IC<2>{});
        else if (RT == 4) rc = launch(IC<ROT>{}, IC<4>{});
        else if (RT == 8) {
          if constexpr (NT >= 8) rc = launch(IC<ROT>{}, IC<8>{});
        }
      }
      MOM_TRY(rc);
      done = true;
    }
  }
  if (!done && g.NK >= 1) {
    const size_t lds = lds_bwd(g, P.R, sizeof(T), P.NT).total;
    MOM_TRY(set_lds(k_bwd<T, NT, ROT, CK>, lds));
    ProfScope ps(KID_BWD, st);
    hipLaunchKernelGGL((k_bwd<T, NT, ROT, CK>), dim3(chains * g.NGR), dim3(NTHB), lds, st, g, X, B, D, Rt,
                       (const float*)carry, dm2, dm1, Db, (T*)dx, (T*)db, (T*)dda, (T*)drot);
    MOM_TRY(check_launch());
  }
  const int pr = g.p * g.r;
  if (done) {
    // the transposed kernel walked each group backward; add what enters at the group ends
    float* gdb = (float*)(ws + P.gdb);
    {
      ProfScope ps(KID_GSCAN, st);
      hipLaunchKernelGGL((k_gscan<T>), dim3(chains, (pr + NTH - 1) / NTH), dim3(NTH), 0, st, g,
                         (const float*)Db, (const float*)dec, gdb, (T*)dh0);
      MOM_TRY(check_launch());
    }
    if (g.NGR > 1 && (dx != nullptr || db != nullptr || dda != nullptr)) {
      const size_t lds = lds_fix(g, P.R, sizeof(T), P.PK).total;
      MOM_TRY(set_lds(k_gfix<T, NT, CK>, lds));
      ProfScope ps(KID_GFIX, st);
      hipLaunchKernelGGL((k_gfix<T, NT, CK>), dim3(chains * (g.NGR - 1)), dim3(NTH), lds, st, g, P.PK, X, B, D,
                         (const float*)carry, (const float*)dec, (const float*)gdb, (T*)dx, (T*)db, (T*)dda);
      MOM_TRY(check_launch());
    }
  } else {
    {
      ProfScope ps(KID_DSCAN, st);
      hipLaunchKernelGGL((k_dscan<T>), dim3(chains, (pr + NTH - 1) / NTH), dim3(NTH), 0, st, g, Db,
                         (const float*)dec, (T*)dh0);
    }
    MOM_TRY(check_launch());
  }
  if (!done && g.NK >= 2 && (dx != nullptr || db != nullptr || dda != nullptr)) {
    const size_t lds = lds_fix(g, P.R, sizeof(T), P.PK).total;
    MOM_TRY(set_lds(k_fix<T, NT, CK>, lds));
    ProfScope ps(KID_FIX, st);
    hipLaunchKernelGGL((k_fix<T, NT, CK>), dim3(chains * (g.NK - 1)), dim3(NTH), lds, st, g, P.PK, X, B, D,
                       (const float*)carry, (const float*)Db, (T*)dx, (T*)db, (T*)dda);
    MOM_TRY(check_launch());
  }
  const int z0 = g.NK * ELL;
  if (z0 < g.s || g.skip) {
    ProfScope ps(KID_ZERO, st);
    hipLaunchKernelGGL((k_zero_tail<T>), dim3(g.skip ? 256 : 1024, g.skip ? std::min(g.b, 65535) : 1), dim3(NTH), 0,
                       st, g, z0,
                       (T*)dx, (T*)db, (T*)dda, (T*)drot);
    MOM_TRY(check_launch());
  }
  return 0;
}

// Debug finiteness check (the pages' san() on the outputs), on when the
// environment variable MOMENTS_CHECK_FINITE is set to anything but "" or "0".
// It waits for the stream and returns MOMENTS_ENONFINITE if any listed output
// holds a NaN or an infinity.
bool check_finite_on() {
  const char* e = getenv("MOMENTS_CHECK_FINITE");
  return e != nullptr && e[0] != 0 && !(e[0] == '0' && e[1] == 0);
}

struct OutSpan {
  const void* p;
  size_t n;
  bool f32;
};

int check_finite(const OutSpan* outs, int nout, unsigned char* flag_mem, hipStream_t st) {
  int* flag = (int*)flag_mem;
  hipLaunchKernelGGL(k_flag_clear, dim3(1), dim3(NTH), 0, st, flag);
  MOM_TRY(check_launch());
  for (int i = 0; i < nout; i++) {
    if (outs[i].p == nullptr || outs[i].n == 0) continue;
    const unsigned blocks = (unsigned)std::min<size_t>((outs[i].n + NTH - 1) / NTH, 2048);
    if (outs[i].f32)
      hipLaunchKernelGGL(k_check_finite<float>, dim3(blocks), dim3(NTH), 0, st, (const float*)outs[i].p, outs[i].n,
                         flag);
    else
      hipLaunchKernelGGL(k_check_finite<bf16>, dim3(blocks), dim3(NTH), 0, st, (const bf16*)outs[i].p, outs[i].n,
                         flag);
    MOM_TRY(check_launch());
  }
  int host = 0;
  hipError_t e = hipMemcpyAsync(&host, flag, sizeof(int), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e);
  return host ? MOMENTS_ENONFINITE : 0;
}

// Calls f(TT<T>, IC<NT>, IC<ROT>, IC<CK>) for the compiled variant matching the plan.
template <class F>
int with_variant(const Plan& P, F&& f) {
  auto by_ck = [&](auto tt, auto nt, auto rot) -> int {
    switch (P.CK) {
      case 1: return f(tt, nt, rot, IC<1>{});
      case 2: return f(tt, nt, rot, IC<2>{});
      case 4: return f(tt, nt, rot, IC<4>{});
    }
    return MOMENTS_ENOTSUP;
  };
  auto by_rot = [&](auto tt, auto nt) -> int {
    switch (P.g.rot_kind) {
      case MOMENTS_ROT_NONE: return by_ck(tt, nt, IC<0>{});
      case MOMENTS_ROT_COMPLEX_PAIRWISE:
      case MOMENTS_ROT_COMPLEX_HALF: return by_ck(tt, nt, IC<1>{});
      case MOMENTS_ROT_QUATERNION: return by_ck(tt, nt, IC<3>{});
    }
    return MOMENTS_EINVAL;
  };
  if (P.bf) {
    if (P.NT == 4) return by_rot(TT<bf16>{}, IC<4>{});
    if (P.NT == 8) return by_rot(TT<bf16>{}, IC<8>{});
  } else {
    if (P.NT == 4) return by_rot(TT<float>{}, IC<4>{});
  }
  return MOMENTS_ENOTSUP;
}

// ---- rotation-sequence producer ---------------------------------------------
struct RotPlan {
  RotGeo g;
  bool bf, quat, empty;
  int V;                // chains per thread of the streaming passes
  size_t tot, aux, ws_fwd, ws_bwd;  // workspace offsets and bytes
};

// Reads b, s, h, dtype, rot_kind, rope_dim / quat_blocks of the descriptor.
int make_rot_plan(const moments_desc* d, RotPlan* P) {
  if (d == nullptr) return MOMENTS_EINVAL;
  if (d->b < 0 || d->s < 0 || d->h < 0) return MOMENTS_EINVAL;
  if (d->dtype != MOMENTS_F32 && d->dtype != MOMENTS_BF16) return MOMENTS_EINVAL;
  int64_t per_h = 0;
  if (d->rot_kind == MOMENTS_ROT_COMPLEX_PAIRWISE || d->rot_kind == MOMENTS_ROT_COMPLEX_HALF) {
    if (d->rope_dim < 2 || d->rope_dim % 2 != 0) return MOMENTS_EINVAL;
    per_h = d->rope_dim / 2;
    P->quat = false;
  } else if (d->rot_kind == MOMENTS_ROT_QUATERNION) {
    if (d->quat_blocks < 1) return MOMENTS_EINVAL;
    per_h = d->quat_blocks;
    P->quat = true;
  } else {
    return MOMENTS_EINVAL;
  }
  const int64_t C = d->h * per_h;
  if (C > (1 << 24) || d->s > (1ll << 30) || d->b > 65535 || d->b * C > (1ll << 30)) return MOMENTS_ENOTSUP;
  P->bf = d->dtype == MOMENTS_BF16;
  P->empty = d->b == 0 || d->s == 0 || C == 0;
  RotGeo& g = P->g;
  g.b = (int)d->b;
  g.s = (int)d->s;
  g.C = (int)C;
  // chains per thread: up to 16 bytes of one token row per load, C divisible by it
  const int width = (P->quat ? 4 : 1) * (P->bf ? 2 : 4);
  P->V = 1;
  while (P->V * 2 * width <= 16 && g.C % (P->V * 2) == 0) P->V *= 2;
  // segments long enough that every walk amortises its entering value, short
  // enough that (segments x chain groups) fills the chip with ~128K threads
  int64_t seg = 16;
  const int64_t work = (int64_t)g.b * g.s * (g.C / P->V);
  while (seg < 1024 && work / (2 * seg) >= (1 << 17)) seg *= 2;
  while (g.s > 0 && (g.s + seg - 1) / seg > 65535) seg *= 2;
  g.seg = (int)seg;
  g.nseg = g.s == 0 ? 0 : (int)((g.s + seg - 1) / seg);
  const size_t n = (size_t)g.b * g.nseg * g.C * (P->quat ? 4 : 1) * sizeof(float);
  P->tot = 0;
  P->aux = (n + 255) / 256 * 256;
  P->ws_fwd = n;
  P->ws_bwd = P->quat ? P->aux + n : n;
  return 0;
}

template <typename T, bool QUAT, bool BWD, int V>
int run_rot(const RotPlan& P, const void* inc, const void* dout, void* out, unsigned char* ws, hipStream_t st) {
  const RotGeo& g = P.g;
  float* tot = (float*)(ws + P.tot);
  float* aux = QUAT && BWD ? (float*)(ws + P.aux) : nullptr;
  const int groups = g.C / V;
  const dim3 grid((groups + ROT_TPB - 1) / ROT_TPB, g.nseg, g.b);
  {
    ProfScope ps(KID_ROTSEG, st);
    hipLaunchKernelGGL((k_rot_seg<T, QUAT, BWD, V>), grid, dim3(ROT_TPB), 0, st, g, (const T*)inc,
                       (const T*)dout, tot, aux);
    MOM_TRY(check_launch());
  }
  {
    ProfScope ps(KID_ROTCARRY, st);
    const int n = g.b * g.C;
    hipLaunchKernelGGL((k_rot_carry<QUAT, BWD>), dim3((n + ROT_TPB - 1) / ROT_TPB), dim3(ROT_TPB), 0, st, g,
                       tot, aux);
    MOM_TRY(check_launch());
  }
  ProfScope ps(KID_ROTAPPLY, st);
  hipLaunchKernelGGL((k_rot_apply<T, QUAT, BWD, V>), grid, dim3(ROT_TPB), 0, st, g, (const T*)inc,
                     (const T*)dout, tot, aux, (T*)out);
  return check_launch();
}

int rot_entry(const moments_desc* desc, bool bwd, const void* inc, const void* dout, void* out, void* workspace,
              size_t workspace_bytes, void* stream) {
  RotPlan P;
  MOM_TRY(make_rot_plan(desc, &P));
  if (P.empty) return 0;
  if (!inc || !out || (bwd && !dout)) return MOMENTS_EINVAL;
  const void* ptrs[] = {inc, dout, out, workspace};
  for (const void* p : ptrs)
    if (p != nullptr && !aligned16(p)) return MOMENTS_EINVAL;
  const size_t need = bwd ? P.ws_bwd : P.ws_fwd;
  if (workspace_bytes < need || workspace == nullptr) return MOMENTS_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  unsigned char* ws = (unsigned char*)workspace;
  // V = 1, 2, 4 or 8 chains per thread (8 only for bf16 angles)
  auto go = [&](auto tt, auto vv) -> int {
    using T = typename decltype(tt)::type;
    constexpr int V = decltype(vv)::value;
    if constexpr (V <= 2) {
      if (P.quat) return bwd ? run_rot<T, true, true, V>(P, inc, dout, out, ws, st)
                             : run_rot<T, true, false, V>(P, inc, dout, out, ws, st);
    } else {
      if (P.quat) return MOMENTS_ENOTSUP;  // the plan never gives quaternions more than 2
    }
    return bwd ? run_rot<T, false, true, V>(P, inc, dout, out, ws, st)
               : run_rot<T, false, false, V>(P, inc, dout, out, ws, st);
  };
  auto by_v = [&](auto tt) -> int {
    switch (P.V) {
      case 1: return go(tt, IC<1>{});
      case 2: return go(tt, IC<2>{});
      case 4: return go(tt, IC<4>{});
    }
    if constexpr (std::is_same<typename decltype(tt)::type, bf16>::value) return go(tt, IC<8>{});
    return MOMENTS_ENOTSUP;
  };
  return P.bf ? by_v(TT<bf16>{}) : by_v(TT<float>{});
}

// Address of this device's copy of `scratch`, looked up once per device with
// that device current; nullptr (and the HIP error recorded) on failure.
void* static_scratch() {
  static std::mutex mu;
  static std::vector<void*> ptrs;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_fail(e);
    return nullptr;
  }
  std::lock_guard<std::mutex> g(mu);
  if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      hip_fail(e);
      return nullptr;
    }
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace

// Backward over token pairs (see k_pair_prep): pair-token da and rot are built
// in the workspace, the transposed backward runs on the pair plan (d_xhat and
// d_bhat land in place: the layouts coincide), and d_da, d_rot are taken back.
static int run_pair_bwd(const Plan& P, const moments_desc* desc, const void* xhat, const void* bhat, const void* da,
                        const void* rot, const void* h0, const float* d_m2, const float* d_m1, void* d_xhat,
                        void* d_bhat, void* d_da, void* d_rot, void* d_h0, unsigned char* ws, hipStream_t st) {
  Plan Pv;
  MOM_TRY(make_pair_plan(desc, &Pv));
  const Geo& g = P.g;
  bf16* da2 = (bf16*)(ws + P.pr_da2);
  bf16* rot2 = (bf16*)(ws + P.pr_rot2);
  bf16* dda2 = (bf16*)(ws + P.pr_dda2);
  bf16* drot2 = (bf16*)(ws + P.pr_drot2);
  int* lens2 = g.lens != nullptr ? (int*)(ws + P.pr_lens2) : nullptr;
  Pv.g.lens = lens2;
  const size_t row_bytes = (size_t)g.h * g.RW * sizeof(bf16);
  const bool wide = row_bytes % 16 == 0;
  const int units = (int)(wide ? row_bytes / 16 : (size_t)g.h * g.RW);
  const size_t work = (size_t)g.b * g.s * (size_t)(units > g.h ? units : g.h);
  const unsigned blocks = (unsigned)std::min<size_t>((work + NTH - 1) / NTH, 8192);
  {
    ProfScope ps(KID_PAIR, st);
    if (wide)
      hipLaunchKernelGGL((k_pair_prep<bf16, uint4>), dim3(blocks), dim3(NTH), 0, st, g, (const bf16*)da,
                         (const uint4*)rot, units, da2, (uint4*)rot2, lens2);
    else
      hipLaunchKernelGGL((k_pair_prep<bf16, bf16>), dim3(blocks), dim3(NTH), 0, st, g, (const bf16*)da,
                         (const bf16*)rot, units, da2, rot2, lens2);
    MOM_TRY(check_launch());
  }
  unsigned char* wsv = ws;  // the pair plan's workspace is the first Pv.ws_bwd bytes
  MOM_TRY(with_variant(Pv, [&](auto tt, auto nt, auto rk, auto ck) {
    using T = typename decltype(tt)::type;
    constexpr int CK = decltype(ck)::value;
    if constexpr (!std::is_same<T, bf16>::value || CK != 2) {
      return MOMENTS_ENOTSUP;
    } else {
      return run_bwd<T, decltype(nt)::value, decltype(rk)::value, CK>(
          Pv, xhat, bhat, da2, rot != nullptr ? rot2 : nullptr, h0, d_m2, d_m1, d_xhat, d_bhat,
          d_da != nullptr ? dda2 : nullptr, d_rot != nullptr ? drot2 : nullptr, d_h0, wsv, nullptr, st);
    }
  }));
  if (d_da != nullptr || d_rot != nullptr) {
    ProfScope ps(KID_PAIR, st);
    if (wide)
      hipLaunchKernelGGL((k_pair_post<bf16, uint4>), dim3(blocks), dim3(NTH), 0, st, g, (const bf16*)dda2,
                         (const uint4*)drot2, units, (bf16*)d_da, (uint4*)d_rot);
    else
      hipLaunchKernelGGL((k_pair_post<bf16, bf16>), dim3(blocks), dim3(NTH), 0, st, g, (const bf16*)dda2,
                         (const bf16*)drot2, units, (bf16*)d_da, (bf16*)d_rot);
    MOM_TRY(check_launch());
  }
  return 0;
}

// Shared bodies of the forward and backward entry points; `saved` (optional)
// is the caller's saved-carry buffer of `saved_bytes`.
static int fwd_impl(const moments_desc* desc, const void* xhat, const void* bhat, const void* da, const void* rot,
                    const void* h0, float* m2, float* m1, void* saved, size_t saved_bytes, bool want_saved,
                    void* workspace, size_t workspace_bytes, void* stream) {
  Plan P;
  MOM_TRY(make_plan(desc, &P));
  if (!xhat || !bhat || !da || !m2 || !m1) return MOMENTS_EINVAL;
  if (desc->rot_kind != MOMENTS_ROT_NONE && rot == nullptr) return MOMENTS_EINVAL;
  if (want_saved && P.saved > 0 && saved == nullptr) return MOMENTS_EINVAL;
  if (want_saved && saved_bytes < P.saved) return MOMENTS_EWORKSPACE;
  const void* ptrs[] = {xhat, bhat, da, rot, h0, m2, m1, workspace, saved};
  for (const void* p : ptrs)
    if (p != nullptr && !aligned16(p)) return MOMENTS_EINVAL;
  if (workspace_bytes < P.ws_fwd || (P.ws_fwd > 0 && workspace == nullptr)) return MOMENTS_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  unsigned char* ws = (unsigned char*)workspace;
  unsigned char* sv = want_saved && P.saved > 0 ? (unsigned char*)saved : nullptr;
  MOM_TRY(with_variant(P, [&](auto tt, auto nt, auto rk, auto ck) {
    using T = typename decltype(tt)::type;
    return run_fwd<T, decltype(nt)::value, decltype(rk)::value, decltype(ck)::value>(
        P, xhat, bhat, da, rot, h0, m2, m1, ws, sv, st);
  }));
  if (check_finite_on()) {
    const size_t bh = (size_t)P.g.b * P.g.h;
    const OutSpan outs[] = {{m2, bh * P.g.r * P.g.r, true}, {m1, bh * P.g.p * P.g.r, true}};
    return check_finite(outs, 2, ws + P.flag_fwd, st);
  }
  return 0;
}

static int bwd_impl(const moments_desc* desc, const void* xhat, const void* bhat, const void* da, const void* rot,
                    const void* h0, const void* saved, size_t saved_bytes, bool use_saved, const float* d_m2,
                    const float* d_m1, void* d_xhat, void* d_bhat, void* d_da, void* d_rot, void* d_h0,
                    void* workspace, size_t workspace_bytes, void* stream) {
  Plan P;
  MOM_TRY(make_plan(desc, &P));
  if (!xhat || !bhat || !da || !d_m2 || !d_m1) return MOMENTS_EINVAL;
  if (desc->rot_kind != MOMENTS_ROT_NONE && rot == nullptr) return MOMENTS_EINVAL;
  if (desc->rot_kind == MOMENTS_ROT_NONE && d_rot != nullptr) return MOMENTS_EINVAL;
  if (use_saved && P.saved > 0 && saved == nullptr) return MOMENTS_EINVAL;
  if (use_saved && saved_bytes < P.saved) return MOMENTS_EWORKSPACE;
  const void* ptrs[] = {xhat, bhat, da, rot, h0, d_m2, d_m1, d_xhat, d_bhat, d_da, d_rot, d_h0, workspace, saved};
  for (const void* p : ptrs)
    if (p != nullptr && !aligned16(p)) return MOMENTS_EINVAL;
  if (workspace_bytes < P.ws_bwd || (P.ws_bwd > 0 && workspace == nullptr)) return MOMENTS_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  unsigned char* ws = (unsigned char*)workspace;
  const unsigned char* sv = use_saved && P.saved > 0 ? (const unsigned char*)saved : nullptr;
  if (P.pair) {
    // the token-pair walk computes its own carries (at its chunk boundaries), so
    // a saved buffer is not read here
    MOM_TRY(run_pair_bwd(P, desc, xhat, bhat, da, rot, h0, d_m2, d_m1, d_xhat, d_bhat, d_da, d_rot, d_h0, ws, st));
  } else {
    MOM_TRY(with_variant(P, [&](auto tt, auto nt, auto rk, auto ck) {
      using T = typename decltype(tt)::type;
      return run_bwd<T, decltype(nt)::value, decltype(rk)::value, decltype(ck)::value>(
          P, xhat, bhat, da, rot, h0, d_m2, d_m1, d_xhat, d_bhat, d_da, d_rot, d_h0, ws, sv, st);
    }));
  }
  if (check_finite_on()) {
    const Geo& g = P.g;
    const size_t tok = (size_t)g.b * g.s;
    const OutSpan outs[] = {{d_xhat, tok * g.c * g.h * g.p, !P.bf}, {d_bhat, tok * g.c * g.h * g.r, !P.bf},
                            {d_da, tok * g.h, !P.bf}, {d_rot, tok * g.h * g.RW, !P.bf},
                            {d_h0, (size_t)g.b * g.h * g.p * g.r, !P.bf}};
    return check_finite(outs, 5, ws + P.flag_bwd, st);
  }
  return 0;
}

extern "C" {

int moments_validate(const moments_desc* desc) {
  Plan P;
  return make_plan(desc, &P);
}

int64_t moments_workspace_size(const moments_desc* desc, int is_bwd) {
  Plan P;
  const int rc = make_plan(desc, &P);
  if (rc != 0) return rc;
  return (int64_t)(is_bwd ? P.ws_bwd : P.ws_fwd);
}

int moments_fwd(const moments_desc* desc, const void* xhat, const void* bhat, const void* da,
                const void* rot, const void* h0, float* m2, float* m1, void* workspace,
                size_t workspace_bytes, void* stream) {
  return fwd_impl(desc, xhat, bhat, da, rot, h0, m2, m1, nullptr, 0, false, workspace, workspace_bytes, stream);
}

int64_t moments_saved_size(const moments_desc* desc) {
  Plan P;
  const int rc = make_plan(desc, &P);
  if (rc != 0) return rc;
  return (int64_t)P.saved;
}

int moments_fwd_save(const moments_desc* desc, const void* xhat, const void* bhat, const void* da,
                     const void* rot, const void* h0, float* m2, float* m1, void* saved, size_t saved_bytes,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(desc, xhat, bhat, da, rot, h0, m2, m1, saved, saved_bytes, true, workspace, workspace_bytes,
                  stream);
}

int moments_fwd_static(const moments_desc* desc, const void* xhat, const void* bhat, const void* da,
                       const void* rot, const void* h0, float* m2, float* m1, void* stream) {
  Plan P;
  MOM_TRY(make_plan(desc, &P));
  if (P.ws_fwd > (size_t)MOMENTS_STATIC_SCRATCH_BYTES) return MOMENTS_ESCRATCH;
  void* ws = static_scratch();
  if (ws == nullptr) return MOMENTS_EHIP;
  // every region the forward reads is written earlier in the same call (carries
  // by the carry pass, partial moments by the main kernel), so nothing is cleared
  return moments_fwd(desc, xhat, bhat, da, rot, h0, m2, m1, ws, MOMENTS_STATIC_SCRATCH_BYTES, stream);
}

int moments_bwd(const moments_desc* desc, const void* xhat, const void* bhat, const void* da,
                const void* rot, const void* h0, const float* d_m2, const float* d_m1, void* d_xhat,
                void* d_bhat, void* d_da, void* d_rot, void* d_h0, void* workspace,
                size_t workspace_bytes, void* stream) {
  return bwd_impl(desc, xhat, bhat, da, rot, h0, nullptr, 0, false, d_m2, d_m1, d_xhat, d_bhat, d_da, d_rot, d_h0,
                  workspace, workspace_bytes, stream);
}

int moments_bwd_saved(const moments_desc* desc, const void* xhat, const void* bhat, const void* da,
                      const void* rot, const void* h0, const void* saved, size_t saved_bytes, const float* d_m2,
                      const float* d_m1, void* d_xhat, void* d_bhat, void* d_da, void* d_rot, void* d_h0,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(desc, xhat, bhat, da, rot, h0, saved, saved_bytes, true, d_m2, d_m1, d_xhat, d_bhat, d_da, d_rot,
                  d_h0, workspace, workspace_bytes, stream);
}

int64_t moments_rot_workspace_size(const moments_desc* desc, int is_bwd) {
  RotPlan P;
  const int rc = make_rot_plan(desc, &P);
  if (rc != 0) return rc;
  return P.empty ? 0 : (int64_t)(is_bwd ? P.ws_bwd : P.ws_fwd);
}

int moments_rot_fwd(const moments_desc* desc, const void* inc, void* rot, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return rot_entry(desc, false, inc, nullptr, rot, workspace, workspace_bytes, stream);
}

int moments_rot_bwd(const moments_desc* desc, const void* inc, const void* d_rot, void* d_inc, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return rot_entry(desc, true, inc, d_rot, d_inc, workspace, workspace_bytes, stream);
}

const char* moments_strerror(int code) {
  switch (code) {
    case MOMENTS_OK: return "ok";
    case MOMENTS_EINVAL: return "invalid argument (descriptor, NULL pointer or misalignment)";
    case MOMENTS_ENOTSUP: return "shape not covered by the compiled kernels";
    case MOMENTS_EWORKSPACE: return "workspace too small";
    case MOMENTS_EHIP: return "HIP runtime error (see moments_last_hip_error)";
    case MOMENTS_ESCRATCH: return "problem needs more than the static scratch of moments_fwd_static";
    case MOMENTS_ENONFINITE: return "an output holds a NaN or an infinity (MOMENTS_CHECK_FINITE is set)";
  }
  return "unknown error";
}

int moments_last_hip_error(void) { return g_last_hip.load(); }

int64_t moments_kernel_chunk_len(void) { return ELL; }

int moments_profile_enable(int on) {
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  const int was = P.on ? 1 : 0;
  P.on = on != 0;
  return was;
}

int moments_profile_read(int id, const char** name, int64_t* launches, double* total_ms) {
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  for (const auto& r : P.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess) return hip_fail(hipGetLastError());
    if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      P.ms[r.kid] += ms;
      P.n[r.kid] += 1;
    }
    P.pool.push_back(r.a);
    P.pool.push_back(r.b);
  }
  P.pending.clear();
  if (id < 0 || id >= KID_N) return MOMENTS_EINVAL;
  if (name) *name = kKernelNames[id];
  if (launches) *launches = P.n[id];
  if (total_ms) *total_ms = P.ms[id];
  return KID_N;
}

void moments_profile_reset(void) {
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  for (auto& r : P.pending) {
    (void)hipEventSynchronize(r.b);
    P.pool.push_back(r.a);
    P.pool.push_back(r.b);
  }
  P.pending.clear();
  for (int i = 0; i < KID_N; i++) {
    P.ms[i] = 0.0;
    P.n[i] = 0;
  }
}

}  // extern "C"

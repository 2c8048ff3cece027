// The lane-pair forward's launches and every instance the dispatcher can ask
// for (the library is linked with no undefined symbols, so a missing instance
// fails the build). This file is compiled twice: with MOM_FWD4_SAVE = 0, the
// instances that do not save carries, with the ILP scheduling strategy (see
// fwd4_launch.h); with MOM_FWD4_SAVE = 1, those that also save the carries
// (INC = 2), with the default strategy, which measured faster for them.
#include "fwd4_launch.h"

#include "kernels_fwd4.h"

#ifndef MOM_FWD4_SAVE
#error "compile with -DMOM_FWD4_SAVE=0 or 1"
#endif

namespace mom {

template <int NT, int ROT, int CK, int RG, int M1T, int INC>
hipError_t launch_fwd4(const Geo& g, size_t lds, unsigned grid, hipStream_t st, const bf16* xhat,
                       const bf16* bhat, const bf16* da, const bf16* rot, const float* carry, const bf16* h0,
                       float* m2part, float* m1part, float* save, float* save_dec) {
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_fwd4<NT, ROT, CK, RG, M1T, INC>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_fwd4<NT, ROT, CK, RG, M1T, INC>), dim3(grid), dim3(NT4), lds, st, g, xhat, bhat, da, rot,
                     carry, h0, m2part, m1part, save, save_dec);
  return hipGetLastError();
}

// Instances: column tiles NT in {4, 8}; (rotation, rotated column groups) with
// RG * (2 for complex pairs, 4 for quaternions) <= NT; channel steps CK in
// {1, 2, 4}; m1 row tiles M1T in {1, 2}; INC 0 (carries from the carry pass),
// 1 (carried in LDS), 2 (carried in LDS and saved), 3 (carried in LDS through
// each group from the carry pass's group-entry state).
#define MOM_FWD4_ONE(NT, RO, CK, RG, M1, INC)                                                                \
  template hipError_t launch_fwd4<NT, RO, CK, RG, M1, INC>(                                                  \
      const Geo&, size_t, unsigned, hipStream_t, const bf16*, const bf16*, const bf16*, const bf16*,         \
      const float*, const bf16*, float*, float*, float*, float*);
#if MOM_FWD4_SAVE
#define MOM_FWD4_INC(NT, RO, CK, RG, M1) MOM_FWD4_ONE(NT, RO, CK, RG, M1, 2)
#else
#define MOM_FWD4_INC(NT, RO, CK, RG, M1) \
  MOM_FWD4_ONE(NT, RO, CK, RG, M1, 0) MOM_FWD4_ONE(NT, RO, CK, RG, M1, 1) MOM_FWD4_ONE(NT, RO, CK, RG, M1, 3)
#endif
#define MOM_FWD4_M1(NT, RO, CK, RG) MOM_FWD4_INC(NT, RO, CK, RG, 1) MOM_FWD4_INC(NT, RO, CK, RG, 2)
#define MOM_FWD4_CK(NT, RO, RG) MOM_FWD4_M1(NT, RO, 1, RG) MOM_FWD4_M1(NT, RO, 2, RG) MOM_FWD4_M1(NT, RO, 4, RG)

MOM_FWD4_CK(4, 0, 0)
MOM_FWD4_CK(4, 1, 1)
MOM_FWD4_CK(4, 1, 2)
MOM_FWD4_CK(4, 3, 1)
MOM_FWD4_CK(8, 0, 0)
MOM_FWD4_CK(8, 1, 1)
MOM_FWD4_CK(8, 1, 2)
MOM_FWD4_CK(8, 1, 4)
MOM_FWD4_CK(8, 3, 1)
MOM_FWD4_CK(8, 3, 2)

}  // namespace mom

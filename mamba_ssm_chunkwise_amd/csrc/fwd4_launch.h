// Launch of the lane-pair forward kernel k_fwd4. Its instances are compiled in
// translation units of their own (fwd4.hip), those that do not save carries
// with the machine scheduler's ILP strategy: k_fwd4 runs one wave per SIMD,
// which overlaps its MFMAs with its own VALU work only as far as its
// instruction stream interleaves them, and that strategy interleaves them
// better than the default. The backward kernels measured slower with it, so
// the rest of the library keeps the default.
#pragma once

#include "common.h"

namespace mom {

// Sets k_fwd4<...>'s dynamic LDS size and launches `grid` workgroups on `st`;
// returns the first HIP error. Arguments as k_fwd4 takes them.
template <int NT, int ROT, int CK, int RG, int M1T, int INC>
hipError_t launch_fwd4(const Geo& g, size_t lds, unsigned grid, hipStream_t st, const bf16* xhat,
                       const bf16* bhat, const bf16* da, const bf16* rot, const float* carry, const bf16* h0,
                       float* m2part, float* m1part, float* save, float* save_dec);

}  // namespace mom

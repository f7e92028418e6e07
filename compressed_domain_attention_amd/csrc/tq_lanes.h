// Lane exchanges inside a 64-lane wave, shared by the HIP sources.
#pragma once

#include <hip/hip_runtime.h>

namespace tq {
namespace {

// The value of lane `lane ^ m` (m a power of two below 64).  Inside a 16-lane row the
// exchange is a DPP lane move (quad permutes for 1 and 2, a shift left or right by 4, a
// rotation by 8), with no round trip through the LDS crossbar; 16 and 32 cross rows with a
// bpermute.  m is a constant after unrolling, so the branches fold.
__device__ __forceinline__ float lane_xor(float x, int m, int lane) {
  const int v = __builtin_bit_cast(int, x);
  if (m == 1) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  if (m == 2) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  if (m == 4) {
    const int from_above = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false);  // row_shl:4, lane i + 4
    const int from_below = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4, lane i - 4
    return __builtin_bit_cast(float, (lane & 4) ? from_below : from_above);
  }
  if (m == 8) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
  return __shfl_xor(x, m);
}

}  // namespace
}  // namespace tq

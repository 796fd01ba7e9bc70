// xlane.hpp -- cross-lane exchanges within a 64-lane wavefront on gfx950.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

// Value of lane (lane ^ M) for a 32-bit word, M a power of two below 64.
// VALU operations only: DPP inside a 16-lane row for masks 1, 2, 4, 8 and the
// gfx950 permlane swaps for masks 16 and 32 (no LDS round trip).
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const int lane = threadIdx.x & 63;
  if constexpr (M == 1) {
    return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    // banks 1, 3 (lanes 4-7, 12-15 of a row) read lane - 4; banks 0, 2 read lane + 4
    const uint32_t r = __builtin_amdgcn_update_dpp(v, v, 0x114, 0xF, 0xA, false);
    return __builtin_amdgcn_update_dpp(r, v, 0x104, 0xF, 0x5, false);
  } else if constexpr (M == 8) {
    // banks 2, 3 (lanes 8-15 of a row) read lane - 8; banks 0, 1 read lane + 8
    const uint32_t r = __builtin_amdgcn_update_dpp(v, v, 0x118, 0xF, 0xC, false);
    return __builtin_amdgcn_update_dpp(r, v, 0x108, 0xF, 0x3, false);
  } else if constexpr (M == 16) {
    // swap odd rows of the first copy with even rows of the second
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? p[0] : p[1];
  } else {
    static_assert(M == 32, "lane mask");
    // swap the upper half of the first copy with the lower half of the second
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? p[0] : p[1];
  }
}

template <int M>
__device__ __forceinline__ float xor_lane_f32(float x) {
  return __builtin_bit_cast(float, xor_lane<M>(__builtin_bit_cast(uint32_t, x)));
}

}  // namespace tq

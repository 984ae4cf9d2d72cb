// Butterflies of the 128-wide Hadamard (FORMAT F8) on a block held by 16 lanes, 8
// consecutive values each (sub = the lane's index within the block, the block a row of 16
// lanes): strides 1, 2, 4 run inside the lane, strides 8 .. 64 pair lane l with lane
// l ^ 1, 2, 4, 8. Every stage is the fp32 pair map (a, b) -> (a + b, a - b) with a the lower
// index. All lanes of the wave must take part (the cross-lane moves read every lane).
#pragma once

#include "tq_device.h"

namespace tq {

// The value of lane l ^ D within each row of 16 lanes, by DPP (no LDS traffic): quad
// permutations for D = 1, 2, a quad reversal then a half-row mirror for 4, a rotation of
// the row by 8 for 8.
template <int D>
__device__ __forceinline__ float row_xor(float v) {
  int x = __float_as_int(v);
  if constexpr (D == 1) {
    x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);   // quad_perm [1, 0, 3, 2]
  } else if constexpr (D == 2) {
    x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);   // quad_perm [2, 3, 0, 1]
  } else if constexpr (D == 4) {
    x = __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, true);   // quad_perm [3, 2, 1, 0]
    x = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);  // row_half_mirror
  } else {
    static_assert(D == 8, "row_xor: D is 1, 2, 4 or 8");
    x = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true);  // row_ror:8
  }
  return __int_as_float(x);
}

// One cross-lane stage (stride 8 D between values): the lower lane of a pair takes a + b,
// the upper lane a - b, a the lower lane's value.
template <int D>
__device__ __forceinline__ void cross_lane8(float v[8], int sub) {
  const bool upper = (sub & D) != 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float other = row_xor<D>(v[j]);
    v[j] = upper ? other - v[j] : v[j] + other;
  }
}

__device__ __forceinline__ void fwht128_lane8(float v[8], int sub) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((j & h) == 0) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
  cross_lane8<1>(v, sub);
  cross_lane8<2>(v, sub);
  cross_lane8<4>(v, sub);
  cross_lane8<8>(v, sub);
}

}  // namespace tq

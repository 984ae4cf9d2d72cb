// Butterflies of the 128-wide Hadamard (FORMAT F8) on a block held by 16 lanes, 8
// consecutive values each (sub = the lane's index within the block): strides 1, 2, 4 run
// inside the lane, strides 8 .. 64 pair lane l with lane l ^ 1, 2, 4, 8. Every stage is the
// fp32 pair map (a, b) -> (a + b, a - b) with a the lower index. All lanes of the wave must
// take part (the cross-lane moves read every lane).
#pragma once

#include "tq_device.h"

namespace tq {

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
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
    const bool upper = (sub & d) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float other = __shfl_xor(v[j], d, 64);
      v[j] = upper ? other - v[j] : v[j] + other;
    }
  }
}

}  // namespace tq

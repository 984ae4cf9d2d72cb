// Lane-level access to trellis tile columns, shared by the kernels that decode one tile
// column per lane (a wave takes a run of 4 consecutive tiles of one strip: lane (g, n)
// decodes column n of tile g of the run, as in trellis_decode.h).
#pragma once

#include "gemv_wave.h"
#include "trellis_decode.h"

namespace tq {

// ---- code words --------------------------------------------------------------------------
// Words of one tile column a lane loads (see trellis_decode.h): K = 2 word n, K = 4 words
// 2n and 2n + 1, K = 3 the two words of k3_column_words. The word after them (which the
// last states' windows reach) is the next lane's first word, taken by a row rotation: a
// further load would cost more than the two instructions of the rotation.
template <int K>
struct ColWords {
  uint32_t w[K == 2 ? 1 : 2];
};

// Per-lane word offsets inside the wave's run of 4 consecutive tiles.
template <int K>
struct LaneOffsets {
  int o[2];
  uint32_t sel3;
  __device__ LaneOffsets(int g, int n) {
    constexpr int TW = 8 * K;
    o[0] = o[1] = 0;
    sel3 = 0;
    if constexpr (K == 2) {
      o[0] = g * TW + n;
    } else if constexpr (K == 4) {
      o[0] = g * TW + 2 * n;
    } else {
      int a, b;
      k3_column_words(n, &a, &b, &sel3);
      o[0] = g * TW + a;
      o[1] = g * TW + b;
    }
  }
};

template <int K>
__device__ __forceinline__ void load_col(const uint32_t* __restrict__ run,
                                         const LaneOffsets<K>& lo, ColWords<K>& cw) {
  if constexpr (K == 2) {
    cw.w[0] = run[lo.o[0]];
  } else if constexpr (K == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(run + lo.o[0]);
    cw.w[0] = v.x;
    cw.w[1] = v.y;
  } else {
    cw.w[0] = run[lo.o[0]];
    cw.w[1] = run[lo.o[1]];
  }
}

template <int K>
__device__ __forceinline__ void decode_col(const ColWords<K>& cw, uint32_t sel3, uint32_t M[8]) {
  if constexpr (K == 2)
    col_mpairs_k2(cw.w[0], row_next(cw.w[0]), M);
  else if constexpr (K == 4)
    col_mpairs_k4(cw.w[0], cw.w[1], row_next(cw.w[0]), M);
  else
    col_mpairs_k3(cw.w[0], cw.w[1], row_next(cw.w[0]), sel3, M);
}

// ---- buffer loads ------------------------------------------------------------------------
template <int K>
__device__ __forceinline__ void load_col_buf(Rsrc r, const uint32_t vo[2], uint32_t so,
                                             ColWords<K>& cw) {
  if constexpr (K == 2) {
    cw.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, vo[0], so, 0);
  } else if constexpr (K == 4) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, vo[0], so, 0);
    cw.w[0] = v.x;
    cw.w[1] = v.y;
  } else {
    // words p and p + 1 (k3_column_words: p <= 22, so they are adjacent): one 8-byte load
    // (4-byte aligned; a load's cost is set by its lanes, not its bytes)
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, vo[0], so, 0);
    cw.w[0] = v.x;
    cw.w[1] = v.y;
  }
}

}  // namespace tq

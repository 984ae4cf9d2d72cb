// Shared device pieces of the E8M0-scaled stores (MXFP4, fp8b32): scale and code
// conversions and the unit geometry (store order and the GEMV's read order).
#pragma once

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

// E8M0 byte -> fp32 scale 2^(b-127): the byte is the fp32 exponent field; b = 0 is the
// subnormal 2^-127, b = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  uint32_t bits = b << 23;
  bits = (b == 0u) ? 0x00400000u : bits;
  bits = (b == 255u) ? 0x7FC00000u : bits;
  return __uint_as_float(bits);
}

// 8 codes (inputs 8j .. 8j+7, low nibble first) -> 4 dwords of bf16 pairs, natural order.
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t codes, float scale, uint32_t out[4]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
}

// 4 E4M3 codes (inputs 4j .. 4j+3, lowest byte first) -> 2 dwords of bf16 pairs.
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t codes, float scale, uint32_t* out) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, false));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, true));
}

// Unit geometry of the two stores.
template <int FMT>
struct MxUnit {
  static constexpr bool kFp8 = FMT == MX_FP8B32;
  // code bytes of one row (output channel)
  __device__ __host__ static uint32_t row_bytes(int in) { return kFp8 ? (uint32_t)in : (uint32_t)in / 2; }
  __device__ __host__ static size_t code_bytes(int out, int in) { return (size_t)out * row_bytes(in); }
  __device__ __host__ static size_t unit_bytes(int out, int in) {
    return code_bytes(out, in) + (kFp8 ? (size_t)(out / 32) * (in / 32) : (size_t)out * (in / 32));
  }
  // byte offset of the scale of output o, 32-input block kb
  __device__ __host__ static uint32_t scale_at(int out, int in, int o, int kb) {
    return (uint32_t)(code_bytes(out, in) + (kFp8 ? (size_t)(o / 32) * (in / 32) : (size_t)o * (in / 32)) + kb);
  }
  // code bytes of one row and 32-input block
  static constexpr uint32_t kCB = kFp8 ? 32u : 16u;
  // Repacked codes (layout 1, the GEMV's read order): per group of 128 rows, per 128-input
  // step, per strip of 16 rows, the strip's 16 rows x 4 blocks of kCB bytes (row-major)
  // are one contiguous chunk of 64 kCB bytes; a group's steps follow each other with its
  // ns strips each (ns = 8 but in a last, partial group). Scales keep their store order.
  __device__ __host__ static uint32_t group_strips(int out, int grp) {
    const int ns = out / 16 - grp * 8;
    return (uint32_t)(ns < 8 ? ns : 8);
  }
  __device__ __host__ static uint32_t packed_at(int out, int in, int o, int kb) {
    const int grp = o / 128, s8 = (o % 128) / 16, n = o % 16, st = kb / 4, g = kb % 4;
    const size_t S = (size_t)in / 128;
    return (uint32_t)(((size_t)grp * S * 8 + (size_t)st * group_strips(out, grp) + s8) * 64 * kCB +
                      (size_t)n * 4 * kCB + (size_t)g * kCB);
  }
  // store order: byte offset of output o's codes of block kb
  __device__ __host__ static uint32_t stored_at(int in, int o, int kb) {
    return (uint32_t)((size_t)o * row_bytes(in) + (size_t)kb * kCB);
  }
};

}  // namespace tq

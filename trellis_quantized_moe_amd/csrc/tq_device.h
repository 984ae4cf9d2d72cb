// Device-side helpers shared by the gfx950 kernels: operand types, the 16x16x32 matrix-core
// instructions, cross-lane moves and bit conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// D = A * B + C on a 16 x 16 output with K = 32 (one wave). Lane l holds A[m = l % 16]
// [k = 8 (l / 16) .. +7], B[k = 8 (l / 16) .. +7][n = l % 16] and D[m = 4 (l / 16) + i]
// [n = l % 16], i = 0..3. Operands are passed as four 32-bit registers (8 halves).
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
// 16 x 16 x 64 int8 products, int32 accumulation: lane l supplies bytes k = 16 (l / 16) ..
// + 15 of row l % 16 of A and of column l % 16 of B.
__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                               __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Value of the lane one to the right within each row of 16 lanes, wrapping (row_ror:15).
__device__ __forceinline__ uint32_t row_next(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x12F, 0xF, 0xF, true);
}

// Low 32 bits of ({hi, lo} >> s), s in 0..31.
__device__ __forceinline__ uint32_t funnel(uint32_t hi, uint32_t lo, uint32_t s) {
  return __builtin_amdgcn_alignbit(hi, lo, s);
}

// Byte permute: bytes 0-3 of `lo`, 4-7 of `hi`, 12 = 0x00 (v_perm_b32).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// bf16 round-to-nearest-even of an fp32 value (NaN kept quiet with its sign).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t qnan = ((u >> 16) & 0x8000u) | 0x7FC0u;
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? qnan : rounded;  // a select, not a branch
}

// Rounds N fp32 values (N even) to bf16, nearest-even, and returns them as fp32 values: one
// v_cvt_pk_bf16_f32 per pair (finite values round as f32_to_bf16_rne does; a NaN stays a
// NaN, its payload and sign are not kept).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <int N>
__device__ __forceinline__ void round_bf16_pairs(float f[N]) {
#pragma unroll
  for (int j = 0; j < N; j += 2) {
    const bf16x2 h = __builtin_convertvector((f32x2){f[j], f[j + 1]}, bf16x2);
    const uint32_t u = __builtin_bit_cast(uint32_t, h);
    f[j] = __uint_as_float(u << 16);
    f[j + 1] = __uint_as_float(u & 0xFFFF0000u);
  }
}

// f16 bits of an fp32 value, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(unsigned short, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

// Workgroup barrier that orders LDS only. __syncthreads() is also a fence for global
// memory, so each wave first waits for all of its outstanding global loads and stores; a
// kernel that keeps streaming loads in flight, or has just issued result stores, across a
// barrier would stall on them. These fences cover the LDS address space only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workspace status word: sticky error bits (relaxed device-scope OR).
constexpr uint32_t STATUS_BAD_EXPERT = 1u;  // an id outside [-1, E)
constexpr uint32_t STATUS_BAD_UNIT = 2u;    // width byte not in {2,3,4} or misaligned unit
__device__ __forceinline__ void set_status(uint32_t* status, uint32_t bits) {
  __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace tq

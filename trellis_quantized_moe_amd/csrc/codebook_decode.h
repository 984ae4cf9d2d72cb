// Lane-level decoders of the exlr8 codebooks mul1 and pmcgx into FP8 E4M3 operands
// (FORMAT F20, F21; DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores", the paragraph under the
// table). Both read the same tile-column words as the T16 decoders (trellis_cols.h): lane
// (g, n) of a run decodes column n of tile g, the 16 positions of one output channel,
// whose stream bits start at bit 16 K n of the tile.
//   mul1:  position j takes the 16-bit window at column bit K j; m = state * 0x83DCD12D mod
//          2^32, q = (sum of m's bytes) - 510; the operand is E4M3(q / 2) (the GEMM's
//          weight block scale 2^1 restores the factor 2).
//   pmcgx: pair jj (positions 2 jj, 2 jj + 1) takes the 20-bit window at column bit 2 K jj;
//          with c0 = 0xCBAC1FED for the first weight and c1 = 0xBCA14C51 for the second,
//          x = (state * c mod 2^32 & 0x8FFF8FFF) ^ 0x3B603B60, the weight is the E4M3
//          rounding of the sum of x's fp16 halves (exact in fp32).
// The codes come out in the activations' chunk order of the FP8 GEMM (trellis_fp8.hip):
// D[d] holds positions 2d + 8, 2d, 2d + 9, 2d + 1 (bytes 0..3).
#pragma once

#include "trellis_cols.h"

namespace tq {

constexpr uint32_t MUL1_MULT = 0x83DCD12Du;
constexpr uint32_t PMCGX_C0 = 0xCBAC1FEDu;
constexpr uint32_t PMCGX_C1 = 0xBCA14C51u;
constexpr uint32_t PMCGX_MASK = 0x8FFF8FFFu;
constexpr uint32_t PMCGX_XOR = 0x3B603B60u;

constexpr int CB_T16 = 0;
constexpr int CB_MUL1 = 1;
constexpr int CB_PMCGX = 2;

// The column's stream bits: c[0] = bits 0..31, c[1] = 32..63, c[2] = 64..95 (K = 4).
template <int K>
__device__ __forceinline__ void col_bits(const ColWords<K>& cw, uint32_t sel3, uint32_t c[3]) {
  if constexpr (K == 2) {
    c[0] = cw.w[0];
    c[1] = row_next(cw.w[0]);
    c[2] = 0;
  } else if constexpr (K == 3) {
    const uint32_t x2 = row_next(cw.w[0]);
    c[0] = perm(cw.w[0], cw.w[1], sel3);
    c[1] = perm(cw.w[1], x2, sel3);
    c[2] = 0;
  } else {
    c[0] = cw.w[0];
    c[1] = cw.w[1];
    c[2] = row_next(cw.w[0]);
  }
}

// The W-bit window that starts at column bit b (b + W <= 96; b compile-time in the loops).
template <int W>
__device__ __forceinline__ uint32_t col_window(const uint32_t c[3], int b) {
  const int i = b >> 5;
  const uint64_t v = ((uint64_t)c[i] << 32) | (i + 1 < 3 ? c[i + 1] : 0u);
  return (uint32_t)(v >> (64 - W - (b & 31))) & ((1u << W) - 1u);
}

template <int K>
__device__ __forceinline__ void mul1_col(const ColWords<K>& cw, uint32_t sel3, uint32_t D[4]) {
  uint32_t c[3];
  col_bits<K>(cw, sel3, c);
  float h[16];  // q / 2, exact
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t m = col_window<16>(c, K * j) * MUL1_MULT;
    const uint32_t sum = __builtin_amdgcn_udot4(m, 0x01010101u, 0u, false);
    h[j] = __builtin_fmaf((float)sum, 0.5f, -255.0f);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(h[2 * d + 8], h[2 * d], 0, false);
    D[d] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(h[2 * d + 9], h[2 * d + 1], lo, true);
  }
}

__device__ __forceinline__ float pmcgx_sum(uint32_t state, uint32_t mult) {
  const uint32_t x = ((state * mult) & PMCGX_MASK) ^ PMCGX_XOR;
  return f16_bits_to_f32(x & 0xFFFFu) + f16_bits_to_f32(x >> 16);
}

template <int K>
__device__ __forceinline__ void pmcgx_col(const ColWords<K>& cw, uint32_t sel3, uint32_t D[4]) {
  uint32_t c[3];
  col_bits<K>(cw, sel3, c);
  float a[8], b[8];  // first and second weight of pair jj
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const uint32_t s = col_window<20>(c, 2 * K * jj);
    a[jj] = pmcgx_sum(s, PMCGX_C0);
    b[jj] = pmcgx_sum(s, PMCGX_C1);
  }
  // positions 2d, 2d + 1 are pair d; positions 2d + 8, 2d + 9 are pair d + 4
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a[d + 4], a[d], 0, false);
    D[d] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(b[d + 4], b[d], lo, true);
  }
}

}  // namespace tq

// Lane-level T16 trellis decoders for gfx950.
//
// A tile is 16 x 16 weights stored as 8*K uint32 words; its bit stream is read most
// significant bit first and position p (input p % 16 of output channel p / 16 of the tile)
// takes the 16-bit window starting at bit p*K, circularly within the tile. The value is
// q = lo8(m) + hi8(m) - 255 with m = state * 0x3A2F mod 2^16 (DeepSeek-V4.1-Flash-1017
// · dsx T16 page, "How T16 works", items 1 and 2).
//
// One lane decodes one tile column: the 16 consecutive positions of one output channel.
// It gathers the column's bits into at most three registers, cuts the 16 states out
// pairwise (two states per 32-bit register, so one packed 16-bit multiply serves both),
// and multiplies. The result is eight "m-pairs": register r holds the product of the
// state for input IH(r) in its high half and for input IL(r) in its low half.
//   K = 2, 3:  IH(r) = r,      IL(r) = r + 8
//   K = 4:     IH(r) = J(r),   IL(r) = J(r) + 4, with J(r) = r (r < 4) or r + 4 (r >= 4)
// For K = 2 and 4, the two states of a pair sit 16 bits apart in the stream, so a single
// funnel shift yields both; K = 3 needs two funnel shifts and a bit-field merge per pair.
#pragma once

#include "tq_device.h"

namespace tq {

constexpr uint32_t T16_MULT2 = 0x3A2F3A2Fu;

// ---- unit layouts ---------------------------------------------------------------------------
// A unit is out / 16 strips of in / 16 tiles; the kernels read it in runs: the 4 tiles of
// one strip that one 64-input step covers (tile columns 4 st .. 4 st + 3, 128 K bytes).
//   layout 0 (FORMAT F2, TQ_LAYOUT_STORE): a strip's runs follow each other;
//   layout 1 (TQ_LAYOUT_GEMV, written once by trellis_repack): the runs of one group of 8
//            strips (128 output channels) are step-major, so the runs a step of a group
//            needs are contiguous, and so are a group's steps;
//   layout 2 (FORMAT F2b, TQ_LAYOUT_UNIT128): units of 128 inputs (2 steps), each
//            strip-major over its own 8 tile columns.
// Word offset of run (strip t, step st) within the unit, S = in / 64 steps, n_strips =
// out / 16, TW = 8 K words per tile. For every layout, the offset between two strips does
// not depend on the step.
__device__ __forceinline__ uint32_t run_word(int layout, int t, int st, int S, int n_strips,
                                             int TW) {
  if (layout == 0) return (uint32_t)((t * S + st) * 4 * TW);
  if (layout == 2)
    return (uint32_t)((st >> 1) * n_strips * 8 * TW + (t * 2 + (st & 1)) * 4 * TW);
  const int g = t >> 3, ns = min(8, n_strips - 8 * g);
  return (uint32_t)(((g * S * 8) + st * ns + (t & 7)) * 4 * TW);
}

template <int K>
__device__ __forceinline__ int pair_ih(int r) {
  return K == 4 ? (r < 4 ? r : r + 4) : r;
}
template <int K>
__device__ __forceinline__ int pair_il(int r) {
  return K == 4 ? pair_ih<K>(r) + 4 : r + 8;
}

// Word offsets (within a tile) a lane loads for column n.
// K = 2: word n (the window of the column's last states continues into word n+1, which
//        the lane takes from its right neighbour).
// K = 4: words 2n, 2n+1 (word 2n+2 comes from the right neighbour).
// K = 3: the column starts at bit 48n: word p = floor(3n / 2), at bit 0 (n even) or bit 16
//        (n odd). The lane loads words p and p+1; the 61 bits of an odd lane's column run
//        into word p+2, which is the first word of the right neighbour (column n+1 starts
//        at word p+2), taken from it. A byte selector aligns the column start: u0 = the
//        column's bits 0..31, u1 = bits 32..63, one byte permutation each.
__device__ __forceinline__ void k3_column_words(int n, int* w0, int* w1, uint32_t* sel) {
  const int p = (3 * n) >> 1;
  *w0 = p % 24;
  *w1 = (p + 1) % 24;
  *sel = (n & 1) ? 0x05040302u : 0x07060504u;  // {lo16(a), hi16(b)} or a
}

// Eight m-pairs of a K = 2 column. w = word n of the tile, wn = word n + 1 (mod 16).
__device__ __forceinline__ void col_mpairs_k2(uint32_t w, uint32_t wn, uint32_t M[8]) {
  uint32_t R[8];
  R[0] = w;
#pragma unroll
  for (int j = 1; j < 8; ++j) R[j] = funnel(w, wn, 32 - 2 * j);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u16x2 v = __builtin_bit_cast(u16x2, R[j]) * __builtin_bit_cast(u16x2, T16_MULT2);
    M[j] = __builtin_bit_cast(uint32_t, v);
  }
}

// K = 4 column: w0, w1 = words 2n, 2n+1, w2 = word 2n+2 (mod 32).
__device__ __forceinline__ void col_mpairs_k4(uint32_t w0, uint32_t w1, uint32_t w2,
                                              uint32_t M[8]) {
  uint32_t R[8];
  R[0] = w0;
  R[4] = w1;
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    R[j] = funnel(w0, w1, 32 - 4 * j);
    R[4 + j] = funnel(w1, w2, 32 - 4 * j);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u16x2 v = __builtin_bit_cast(u16x2, R[j]) * __builtin_bit_cast(u16x2, T16_MULT2);
    M[j] = __builtin_bit_cast(uint32_t, v);
  }
}

// K = 3 column: x0, x1 = words p, p+1 and x2 = the right neighbour's x0 (see
// k3_column_words).
__device__ __forceinline__ void col_mpairs_k3(uint32_t x0, uint32_t x1, uint32_t x2,
                                              uint32_t sel, uint32_t M[8]) {
  const uint32_t u0 = perm(x0, x1, sel);
  const uint32_t u1 = perm(x1, x2, sel);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t r1 = j == 0 ? u0 : funnel(u0, u1, 32 - 3 * j);  // high half: state j
    uint32_t r2 = funnel(u0, u1, 24 - 3 * j);                 // low half: state j + 8
    uint32_t r = (r1 & 0xFFFF0000u) | (r2 & 0x0000FFFFu);
    u16x2 v = __builtin_bit_cast(u16x2, r) * __builtin_bit_cast(u16x2, T16_MULT2);
    M[j] = __builtin_bit_cast(uint32_t, v);
  }
}

// Half h (pairs 4 h .. 4 h + 3) of the eight m-pairs of a K = 2 column: the pairs of the
// column's first (h = 0) or second (h = 1) matrix-core product.
__device__ __forceinline__ void half_mpairs_k2(uint32_t w, uint32_t wn, int h, uint32_t M[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int jj = 4 * h + j;
    const uint32_t r = jj == 0 ? w : funnel(w, wn, 32 - 2 * jj);
    u16x2 v = __builtin_bit_cast(u16x2, r) * __builtin_bit_cast(u16x2, T16_MULT2);
    M[j] = __builtin_bit_cast(uint32_t, v);
  }
}

// Half h of the eight m-pairs of a K = 3 column (x0..x2, sel as for col_mpairs_k3).
__device__ __forceinline__ void half_mpairs_k3(uint32_t x0, uint32_t x1, uint32_t x2,
                                               uint32_t sel, int h, uint32_t M[4]) {
  const uint32_t u0 = perm(x0, x1, sel);
  const uint32_t u1 = perm(x1, x2, sel);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int jj = 4 * h + j;
    const uint32_t r1 = jj == 0 ? u0 : funnel(u0, u1, 32 - 3 * jj);
    const uint32_t r2 = funnel(u0, u1, 24 - 3 * jj);
    const uint32_t r = (r1 & 0xFFFF0000u) | (r2 & 0x0000FFFFu);
    u16x2 v = __builtin_bit_cast(u16x2, r) * __builtin_bit_cast(u16x2, T16_MULT2);
    M[j] = __builtin_bit_cast(uint32_t, v);
  }
}

// ---- prefill operands: byte sums as f16 subnormals ----------------------------------------
// The matrix cores take v = lo8(m) + hi8(m) = q + 255 (0..510) as the bits of an f16 with a
// zero exponent field, i.e. the subnormal v * 2^-24, exact (the matrix cores keep subnormal
// inputs). A 16-bit lane computes v = m - 255 * (m >> 8) with one packed shift and one
// packed multiply-add. The accumulator then holds 2^-24 * sum x * (q + 255); the epilogue
// multiplies by 2^24 (exact) and removes 255 * sum(x).
//
// The activations use one layout for every K: word r (r = 0..7) of a tile column holds
// [lo: x[r + 8], hi: x[r]], and byte_sums returns the weights in the same layout:
// V[r] = [lo: v[r + 8], hi: v[r]].
constexpr float BYTE_SUM_OFFSET = 255.0f;
constexpr float BYTE_SUM_SCALE = 16777216.0f;  // 2^24

__device__ __forceinline__ uint32_t byte_sum_pair(uint32_t M) {
  u16x2 m = __builtin_bit_cast(u16x2, M);
  u16x2 h = m >> (u16x2){8, 8};
  u16x2 v = m + h * (u16x2){0xFF01, 0xFF01};  // m - 255 * h (mod 2^16)
  return __builtin_bit_cast(uint32_t, v);
}

template <int K>
__device__ __forceinline__ void byte_sums(const uint32_t M[8], uint32_t V[8]) {
  if constexpr (K == 4) {
    // M[r] (r < 4) = [hi: m[r], lo: m[r + 4]]; M[r] (r >= 4) = [hi: m[r + 4], lo: m[r + 8]]
    uint32_t W[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) W[r] = byte_sum_pair(M[r]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      V[r] = perm(W[r], W[r + 4], 0x07060302u);      // [hi: v[r], lo: v[r + 8]]
      V[r + 4] = perm(W[r], W[r + 4], 0x05040100u);  // [hi: v[r + 4], lo: v[r + 12]]
    }
  } else {
    // M[r] = [hi: m[r], lo: m[r + 8]]
#pragma unroll
    for (int r = 0; r < 8; ++r) V[r] = byte_sum_pair(M[r]);
  }
}

// The prefill GEMM's operands of one tile column, in the layout above (register r holds
// [hi: v[r], lo: v[r + 8]]), split into the two halves that feed the step's two products:
// half h is registers 4 h .. 4 h + 3. w0, w1: the column's loaded words (w1 unused at
// K = 2), wn: the right neighbour's first word, sel3: the K = 3 byte selector.
// K = 2, 3 decode each half on its own (only its four m-pairs).
template <int K>
__device__ __forceinline__ void prefill_half(uint32_t w0, uint32_t w1, uint32_t wn,
                                             uint32_t sel3, int h, uint32_t B[4]) {
  static_assert(K == 2 || K == 3, "prefill_half: K = 2 or 3");
  uint32_t M[4];
  if constexpr (K == 2)
    half_mpairs_k2(w0, wn, h, M);
  else
    half_mpairs_k3(w0, w1, wn, sel3, h, M);
#pragma unroll
  for (int r = 0; r < 4; ++r) B[r] = byte_sum_pair(M[r]);
}

// Both halves at once (K = 4 pairs its states across the halves, so it always takes this).
template <int K>
__device__ __forceinline__ void prefill_full(uint32_t w0, uint32_t w1, uint32_t wn,
                                             uint32_t sel3, uint32_t B0[4], uint32_t B1[4]) {
  uint32_t M[8], V[8];
  if constexpr (K == 2)
    col_mpairs_k2(w0, wn, M);
  else if constexpr (K == 4)
    col_mpairs_k4(w0, w1, wn, M);
  else
    col_mpairs_k3(w0, w1, wn, sel3, M);
  byte_sums<K>(M, V);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    B0[r] = V[r];
    B1[r] = V[4 + r];
  }
}

// ---- decode-batch operands: signed bytes ----------------------------------------------
// The int8 matrix-core operation takes the two bytes of m as two separate k positions,
// each against the same activation, so the sum over a weight's two positions is
// x * (lo8(m) + hi8(m)). One xor with 0x80 per byte makes the bytes signed: (lo8 - 128) +
// (hi8 - 128) = q - 1, and the epilogue adds sum(x) back. A register of m-pairs becomes one
// operand register with a single xor.
//
// The activations use one layout for every K: bytes 0..3 of operand register r of a tile
// column hold [x[r + 8], x[r + 8], x[r], x[r]], and i8_operands returns the weights in the
// matching layout: register r = [lo8, hi8 of m[r + 8] | lo8, hi8 of m[r]], each byte - 128.
__device__ __forceinline__ uint32_t signed_bytes(uint32_t M) { return M ^ 0x80808080u; }

template <int K>
__device__ __forceinline__ void i8_operands(const uint32_t M[8], uint32_t B[8]) {
  if constexpr (K == 4) {
    // M[r] (r < 4) = [hi: m[r], lo: m[r + 4]]; M[r] (r >= 4) = [hi: m[r + 4], lo: m[r + 8]]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      B[r] = signed_bytes(perm(M[r], M[r + 4], 0x07060302u));      // [hi: m[r], lo: m[r + 8]]
      B[r + 4] = signed_bytes(perm(M[r], M[r + 4], 0x05040100u));  // [hi: m[r + 4], lo: m[r + 12]]
    }
  } else {
    // M[r] = [hi: m[r], lo: m[r + 8]]
#pragma unroll
    for (int r = 0; r < 8; ++r) B[r] = signed_bytes(M[r]);
  }
}

}  // namespace tq

// Decode-batch grouped GEMV over trellis-coded experts (gfx950).
//
// One wave is one worker of the plan (see gemv_plan.h): the grid is single-wave workgroups,
// and wave w streams the one piece the plan gave it, steps s0 .. s1 - 1 of one group of one
// expert, on its own: no LDS and no barrier, so a wave that waits for memory never holds
// up another, and its load stream never restarts. A step is 4 tile columns (64 inputs) of
// the group's 8 strips (128 output channels). Per step and strip, each lane decodes one
// tile column (16 weights of one output channel) and the wave feeds two 16 x 16 x 64 int8
// matrix-core operations: the weights as signed bytes (two k positions per weight, see
// trellis_decode.h), the activations as the high and the low int8 halves of each token's
// 16-bit integers (rows 0..7: high halves of up to 8 routed tokens, rows 8..15: their low
// halves; rows past the expert's count are zero). The accumulators are exact int32.
//
// Code words are requested D = 2 steps ahead, held in D register sets used in turn, so
// that several steps of loads are in flight per wave, and so are the activations (prepared
// once per call). The load of a strip's next words is issued right after its current words
// are decoded.
//
// A wave takes one chunk of up to 8 of its expert's routed tokens (the plan gives each
// chunk its own waves). At the end it joins each token's two halves (256 hi + lo) and
// stores the piece's partial sums; the reduction launch adds the pieces in order and
// applies the epilogue.
#include "gemv_wave.h"
#include "tq_internal.h"
#include "trellis_decode.h"

namespace tq {

namespace {

constexpr int GEMV_THREADS = 64;         // one wave per workgroup
constexpr int GEMV_WAVES_PER_SIMD = 3;  // register budget: 168 per lane

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
    cw.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, vo[0], so, 0);
    cw.w[1] = __builtin_amdgcn_raw_buffer_load_b32(r, vo[1], so, 0);
  }
}

__device__ __forceinline__ void load_x(Rsrc r, uint32_t vo, uint32_t so, u32x4& xa, u32x4& xb) {
  xa = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0);
  xb = __builtin_amdgcn_raw_buffer_load_b128(r, vo + 16, so, 0);
}

// ---- one step: 4 tile columns of 8 strips ---------------------------------------------
// cw: this step's code words and xa, xb: its activations; with RELOAD they are reloaded
// with those D steps later (scalar offsets cso + strip offset, and xso).
template <int K, bool RELOAD>
__device__ __forceinline__ void step_body(ColWords<K> (&cw)[8], u32x4& xa, u32x4& xb, Rsrc rc,
                                          const uint32_t cvo[2], uint32_t cso,
                                          const uint32_t sso[8], uint32_t sel3, Rsrc rx,
                                          uint32_t xvo, uint32_t xso, i32x4 acc[8]) {
  // Every reload goes into the registers of the value it replaces, after that value's last
  // use (the scheduling barriers keep the compiler from hoisting it), so the loop carries
  // its registers without copies, and a copy would wait for the load in flight.
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) {
    uint32_t M[8], B[8];
    decode_col<K>(cw[s8], sel3, M);
    __builtin_amdgcn_sched_barrier(0);
    if (RELOAD) load_col_buf<K>(rc, cvo, cso + sso[s8], cw[s8]);
    i8_operands<K>(M, B);
    acc[s8] = mfma_i8(xa, (u32x4){B[0], B[1], B[2], B[3]}, acc[s8]);  // pairs 0..3
    acc[s8] = mfma_i8(xb, (u32x4){B[4], B[5], B[6], B[7]}, acc[s8]);  // pairs 4..7
  }
  __builtin_amdgcn_sched_barrier(0);
  if (RELOAD) load_x(rx, xvo, xso, xa, xb);
}

// Steps s0 .. s1 - 1 of output group grp: step st covers tile columns 4 st .. 4 st + 3 (lane
// group g = lane / 16 takes column 4 st + g) of each of the group's strips. tok = this
// lane's token, or -1 (zero row: its activation offset lies past the end of the buffer,
// where buffer loads return 0); half = 0 (high int8 halves) or 1 (low).
template <int K>
__device__ __forceinline__ void stream(const TrellisGemvArgs& a, const uint32_t* __restrict__ unit,
                                       int tok, int half, int grp, int ns, int s0, int s1,
                                       i32x4 acc[8]) {
  constexpr int TW = 8 * K;  // words per tile
  constexpr int D = 2;
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int n_ti = a.in / 16;
  const int steps = s1 - s0, last = steps - 1;
  const LaneOffsets<K> lo(g, n);
  const Rsrc rc = make_rsrc(unit, (uint32_t)((size_t)a.out * a.in * K / 8));
  const uint32_t cvo[2] = {4u * lo.o[0], 4u * lo.o[1]};
  const uint32_t c0 = 4u * (uint32_t)(((size_t)grp * 8 * n_ti + 4 * s0) * TW);
  constexpr uint32_t cstep = 4u * 4 * TW;  // bytes per step and strip (4 tile columns)
  uint32_t sso[8];
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) sso[s8] = 4u * (uint32_t)((s8 < ns ? s8 : ns - 1) * n_ti * TW);
  const Rsrc rx = make_rsrc(a.xq, a.x_bytes);
  const uint32_t xvo = tok >= 0 ? 32u * (uint32_t)((2 * tok + half) * n_ti + g) : 0x80000000u;
  const uint32_t x0 = 128u * (uint32_t)s0;
  // scalar offsets of step st, clamped to the last step (whose words are read again)
  auto cso = [&](int st) { return c0 + (uint32_t)(st < last ? st : last) * cstep; };
  auto xso = [&](int st) { return x0 + (uint32_t)(st < last ? st : last) * 128u; };

  // The prologue issues every code word load first (they need only the plan), then the
  // activations (which wait for this lane's token), so the token lookup delays no code
  // load. In the loop, a step's reloads follow its use, so loads complete in the order
  // they are needed.
  ColWords<K> cw[D][8];
  u32x4 xa[D], xb[D];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) load_col_buf<K>(rc, cvo, cso(d) + sso[s8], cw[d][s8]);
#pragma unroll
  for (int d = 0; d < D; ++d) load_x(rx, xvo, xso(d), xa[d], xb[d]);
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) acc[s8] = (i32x4){0, 0, 0, 0};
  int st = 0;
  for (; st + D <= steps; st += D) {
#pragma unroll
    for (int d = 0; d < D; ++d)
      step_body<K, true>(cw[d], xa[d], xb[d], rc, cvo, cso(st + d + D), sso, lo.sel3, rx, xvo,
                         xso(st + d + D), acc);
  }
  const int rem = steps - st;
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (d < rem)
      step_body<K, false>(cw[d], xa[d], xb[d], rc, cvo, 0, sso, lo.sel3, rx, xvo, 0, acc);
}

// One piece: expert record r, steps s0 .. s1 - 1 of group grp for chunk `chunk` of the
// expert's slot list (up to 8 routed tokens); sums to partial[piece].
template <int K>
__device__ __forceinline__ void run_piece(const TrellisGemvArgs& a, const PlanRec& r, int grp,
                                          int chunk, int s0, int s1, int piece) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int j = n & 7, half = n >> 3;  // this lane's A row: token j of the chunk, its half
  const int ns = min(8, a.out / 16 - grp * 8);
  const uint32_t* unit = a.codes + r.off / 4;
  float* dst = a.partial + (size_t)piece * a.N * a.out + grp * 128 + n;
  {
    const int c0 = 8 * chunk;
    const int rows = min(8, r.cnt - c0);
    // lanes with j = m hold the slot of token m of the chunk
    const int slot = j < rows ? a.list[r.start + c0 + j] : -1;
    i32x4 acc[8];
    stream<K>(a, unit, slot >= 0 ? slot / a.topk : -1, half, grp, ns, s0, s1, acc);
    // accumulator element i of lane (g, n) is row 4 g + i: for g < 2 the high half of token
    // 4 g + i, whose low half is in lane + 32
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      const int sm = __shfl(slot, m & 7);
      float v[8];
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8)
        v[s8] = 256.0f * (float)acc[s8][i] + (float)__shfl_xor(acc[s8][i], 32, 64);
      if (g < 2 && m < rows) {
        float* row = dst + (size_t)sm * a.out;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8)
          if (s8 < ns) row[s8 * 16] = v[s8];
      }
    }
  }
}

__global__ __launch_bounds__(GEMV_THREADS, GEMV_WAVES_PER_SIMD) void trellis_gemv_kernel(TrellisGemvArgs a) {
  Piece pc;
  if (!load_piece(a.desc, blockIdx.x, pc)) return;
  const PlanRec r = load_rec(a.rec, pc.ai);
  if (r.k == 2)
    run_piece<2>(a, r, pc.grp, pc.chunk, pc.s0, pc.s1, pc.idx);
  else if (r.k == 3)
    run_piece<3>(a, r, pc.grp, pc.chunk, pc.s0, pc.s1, pc.idx);
  else
    run_piece<4>(a, r, pc.grp, pc.chunk, pc.s0, pc.s1, pc.idx);
}

// ---- decode hook ------------------------------------------------------------------------
// One wave per (strip, 4 tile columns); lane (g, n) decodes column n of tile column
// 4 * blk + g with the decode-batch GEMV's (path 0: signed bytes) or the prefill GEMM's
// (path 1: byte sums as f16 subnormals) operand conversion, and writes q[out][in] as int16
// recovered from those operands.
template <int K>
__global__ __launch_bounds__(256) void trellis_decode_kernel(const uint32_t* __restrict__ codes,
                                                             int out, int in,
                                                             int16_t* __restrict__ q, int path) {
  constexpr int TW = 8 * K;
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int n_ti = in / 16;
  const int groups_per_strip = n_ti / 4;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= (out / 16) * groups_per_strip) return;  // whole wave exits together
  const int strip = wave / groups_per_strip;
  const int ti0 = (wave % groups_per_strip) * 4;
  const LaneOffsets<K> lo(g, n);
  ColWords<K> cw;
  load_col<K>(codes + (size_t)(strip * n_ti + ti0) * TW, lo, cw);
  uint32_t M[8];
  decode_col<K>(cw, lo.sel3, M);
  int16_t* row = q + (size_t)(strip * 16 + n) * in + (ti0 + g) * 16;
  if (path == 0) {
    // operand register r: bytes [lo8 - 128, hi8 - 128] of input r + 8, then of input r;
    // q = (lo8 - 128) + (hi8 - 128) + 1
    uint32_t B[8];
    i8_operands<K>(M, B);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int8_t b0 = (int8_t)(B[r] & 0xFF), b1 = (int8_t)((B[r] >> 8) & 0xFF);
      const int8_t b2 = (int8_t)((B[r] >> 16) & 0xFF), b3 = (int8_t)(B[r] >> 24);
      row[r] = (int16_t)(b2 + b3 + 1);
      row[r + 8] = (int16_t)(b0 + b1 + 1);
    }
  } else {
    // V[r] holds inputs r (high half) and r + 8 (low half) as the f16 subnormals
    // (q + 255) * 2^-24
    uint32_t V[8];
    byte_sums<K>(M, V);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      row[r] = (int16_t)(f16_bits_to_f32(V[r] >> 16) * BYTE_SUM_SCALE - BYTE_SUM_OFFSET);
      row[r + 8] = (int16_t)(f16_bits_to_f32(V[r]) * BYTE_SUM_SCALE - BYTE_SUM_OFFSET);
    }
  }
}

}  // namespace

int trellis_gemv_grid() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[dev]) return cache[dev];
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, trellis_gemv_kernel, GEMV_THREADS, 0) !=
      hipSuccess)
    return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  int g = std::min(per_cu, GEMV_TARGET_PER_CU) * cus;
  if (g > GEMV_MAX_G) g = GEMV_MAX_G;
  if (g < 1) g = 1;
  if (dev >= 0 && dev < 64) cache[dev] = g;
  return g;
}

hipError_t launch_trellis_gemv(const TrellisGemvArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(trellis_gemv_kernel, dim3(a.G), dim3(GEMV_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_trellis_decode(const uint32_t* codes, int K, int out, int in, int16_t* q,
                                 int path, hipStream_t s) {
  const int waves = (out / 16) * (in / 64);
  const int blocks = (waves + 3) / 4;
  if (K == 2)
    hipLaunchKernelGGL(trellis_decode_kernel<2>, dim3(blocks), dim3(256), 0, s, codes, out, in, q, path);
  else if (K == 3)
    hipLaunchKernelGGL(trellis_decode_kernel<3>, dim3(blocks), dim3(256), 0, s, codes, out, in, q, path);
  else
    hipLaunchKernelGGL(trellis_decode_kernel<4>, dim3(blocks), dim3(256), 0, s, codes, out, in, q, path);
  return hipGetLastError();
}

}  // namespace tq

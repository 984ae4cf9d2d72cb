// Decode-batch grouped GEMV over trellis-coded experts (gfx950).
//
// One wave is one worker of the plan (see gemv_plan.h): the grid is single-wave workgroups,
// and wave w streams the one piece the plan gave it, steps s0 .. s1 - 1 of one group of one
// expert, on its own: no LDS and no barrier, so a wave that waits for memory never holds
// up another, and its load stream never restarts. A plan group is 8 strips (128 output
// channels), and a wave takes NS = 4 of them: wave 2 q + h takes strips 4 h .. 4 h + 3 of
// piece q. The decode is bound by instruction issue, and a SIMD issues VALU and
// matrix-core instructions faster with four waves to choose from than with two, so the
// pieces are shared by twice the waves (the same pieces, so the same partial sums). A step
// is 4 tile columns (64 inputs) of the wave's strips. Per step and strip, each lane decodes one
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
// chunk its own waves). At the end it joins each token's two halves (256 hi + lo, exact in
// int64) and stores the piece's exact integer sums; the reduction launch adds the pieces
// (exactly, so the split never changes a result) and applies the epilogue.
#include "gemv_wave.h"
#include "tq_internal.h"
#include "trellis_cols.h"
#include "trellis_decode.h"

namespace tq {

namespace {

// Waves per workgroup. The waves of a workgroup are independent (no LDS, no barrier); a
// workgroup of 4 puts one wave on each SIMD of its compute unit, so the waves are spread
// evenly over the SIMDs, which single-wave workgroups leave to the dispatcher.
constexpr int GEMV_WG_WAVES = 1;
constexpr int GEMV_THREADS = 64 * GEMV_WG_WAVES;
constexpr int GEMV_WAVES_PER_SIMD = 4;  // register budget: 128 per lane
constexpr int GEMV_NS = 4;              // strips per wave (two waves per piece)

__device__ __forceinline__ void load_x(Rsrc r, uint32_t vo, uint32_t so, u32x4& xa, u32x4& xb) {
  xa = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0);
  xb = __builtin_amdgcn_raw_buffer_load_b128(r, vo + 16, so, 0);
}

// ---- one step: 4 tile columns of NS strips ----------------------------------------------
// cw: this step's code words and xa, xb: its activations; with RELOAD they are reloaded
// with those D steps later (scalar offsets cso + strip offset, and xso).
template <int K, int NS, bool RELOAD>
__device__ __forceinline__ void step_body(ColWords<K> (&cw)[NS], u32x4& xa, u32x4& xb, Rsrc rc,
                                          const uint32_t cvo[2], uint32_t cso,
                                          const uint32_t sso[NS], uint32_t sel3, Rsrc rx,
                                          uint32_t xvo, uint32_t xso, i32x4 acc[NS]) {
  // Every reload goes into the registers of the value it replaces, after that value's last
  // use (the scheduling barriers keep the compiler from hoisting it), so the loop carries
  // its registers without copies, and a copy would wait for the load in flight.
#pragma unroll
  for (int s8 = 0; s8 < NS; ++s8) {
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

// Steps s0 .. s1 - 1 of strips t0 .. t0 + ns - 1: step st covers tile columns 4 st .. 4 st + 3
// (lane group g = lane / 16 takes column 4 st + g) of each strip. tok = this lane's token, or -1 (zero row: its activation offset lies
// past the end of the buffer, where buffer loads return 0); half = 0 (high int8 halves) or
// 1 (low).
template <int K, int NS>
__device__ __forceinline__ void stream(const TrellisGemvArgs& a, const uint32_t* __restrict__ unit,
                                       int tok, int half, int t0, int ns, int s0, int s1,
                                       i32x4 acc[NS]) {
  constexpr int TW = 8 * K;  // words per tile
  constexpr int D = 2;
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int n_ti = a.in / 16;
  const int steps = s1 - s0, last = steps - 1;
  const LaneOffsets<K> lo(g, n);
  const Rsrc rc = make_rsrc(unit, (uint32_t)((size_t)a.out * a.in * K / 8));
  const uint32_t cvo[2] = {4u * lo.o[0], 4u * lo.o[1]};
  // byte offsets: run (strip t0 + s8, step s0 + st) at cso(st) + sso[s8] (run_word)
  const int S = n_ti / 4, nst = a.out / 16;
  uint32_t sso[NS];
#pragma unroll
  for (int s8 = 0; s8 < NS; ++s8)
    sso[s8] = 4u * (run_word(a.layout, t0 + (s8 < ns ? s8 : ns - 1), s0, S, nst, TW) -
                    run_word(a.layout, t0, s0, S, nst, TW));
  const Rsrc rx = make_rsrc(a.xq, a.x_bytes);
  const uint32_t xvo = tok >= 0 ? 32u * (uint32_t)((2 * tok + half) * n_ti + g) : 0x80000000u;
  const uint32_t x0 = 128u * (uint32_t)s0;
  // scalar offsets of step st, clamped to the last step (whose words are read again)
  auto cso = [&](int st) {
    return 4u * run_word(a.layout, t0, s0 + (st < last ? st : last), S, nst, TW);
  };
  auto xso = [&](int st) { return x0 + (uint32_t)(st < last ? st : last) * 128u; };

  // The prologue issues every code word load first (they need only the plan), then the
  // activations (which wait for this lane's token), so the token lookup delays no code
  // load. In the loop, a step's reloads follow its use, so loads complete in the order
  // they are needed.
  ColWords<K> cw[D][NS];
  u32x4 xa[D], xb[D];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int s8 = 0; s8 < NS; ++s8) load_col_buf<K>(rc, cvo, cso(d) + sso[s8], cw[d][s8]);
#pragma unroll
  for (int d = 0; d < D; ++d) load_x(rx, xvo, xso(d), xa[d], xb[d]);
#pragma unroll
  for (int s8 = 0; s8 < NS; ++s8) acc[s8] = (i32x4){0, 0, 0, 0};
  // A SIMD issues for its oldest wave first, so the waves that share it would finish one by
  // one, the last ones alone and bound by their load latency. The wave's priority drops by
  // one level per quarter of its piece, so the waves behind get the issue slots and all of
  // them stream together to the end.
  const int q1 = steps >> 2, q2 = steps >> 1, q3 = (3 * steps) >> 2;
  __builtin_amdgcn_s_setprio(3);
  int st = 0;
  for (; st + D <= steps; st += D) {
    if (st >= q1 && st < q1 + D) __builtin_amdgcn_s_setprio(2);
    if (st >= q2 && st < q2 + D) __builtin_amdgcn_s_setprio(1);
    if (st >= q3 && st < q3 + D) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int d = 0; d < D; ++d)
      step_body<K, NS, true>(cw[d], xa[d], xb[d], rc, cvo, cso(st + d + D), sso, lo.sel3, rx,
                             xvo, xso(st + d + D), acc);
  }
  const int rem = steps - st;
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (d < rem)
      step_body<K, NS, false>(cw[d], xa[d], xb[d], rc, cvo, 0, sso, lo.sel3, rx, xvo, 0, acc);
}

// One piece: expert record r, steps s0 .. s1 - 1 of strips t0 .. t0 + ns - 1 (ns >= 1) for
// chunk `chunk` of the expert's slot list (up to 8 routed tokens); exact int64 sums to
// partial[piece].
template <int K, int NS>
__device__ __forceinline__ void run_piece(const TrellisGemvArgs& a, const PlanRec& r, int t0,
                                          int ns, int chunk, int s0, int s1, int piece) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int j = n & 7, half = n >> 3;  // this lane's A row: token j of the chunk, its half
  const uint32_t* unit = a.codes + r.off / 4;
  int64_t* dst = a.partial + (size_t)piece * a.N * a.out + t0 * 16 + n;
  {
    const int c0 = 8 * chunk;
    const int rows = min(8, r.cnt - c0);
    // lanes with j = m hold the slot of token m of the chunk
    const int slot = j < rows ? a.list[r.start + c0 + j] : -1;
    i32x4 acc[NS];
    stream<K, NS>(a, unit, slot >= 0 ? slot / a.topk : -1, half, t0, ns, s0, s1, acc);
    // accumulator element i of lane (g, n) is row 4 g + i: for g < 2 the high half of token
    // 4 g + i, whose low half is in lane + 32
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      const int sm = __shfl(slot, m & 7);
      int64_t v[NS];
#pragma unroll
      for (int s8 = 0; s8 < NS; ++s8)
        v[s8] = (int64_t)acc[s8][i] * 256 + (int64_t)__shfl_xor(acc[s8][i], 32, 64);
      if (g < 2 && m < rows) {
        int64_t* row = dst + (size_t)sm * a.out;
#pragma unroll
        for (int s8 = 0; s8 < NS; ++s8)
          if (s8 < ns) row[s8 * 16] = v[s8];
      }
    }
  }
}

__global__ __launch_bounds__(GEMV_THREADS, GEMV_WAVES_PER_SIMD) void trellis_gemv_kernel(TrellisGemvArgs a) {
  constexpr int NS = GEMV_NS, SUB = 8 / NS;  // waves per piece
  Piece pc;
  const int w = blockIdx.x * GEMV_WG_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = w / SUB;
  if (q >= a.G || !load_piece(a.desc, q, pc)) return;  // whole wave
  const int t0 = 8 * pc.grp + NS * (w % SUB);              // first strip
  const int ns = min(NS, a.out / 16 - t0);
  if (ns <= 0) return;  // whole wave: past the last strip of a short group
  const PlanRec r = load_rec(a.rec, pc.ai);
  if (r.k == 2)
    run_piece<2, NS>(a, r, t0, ns, pc.chunk, pc.s0, pc.s1, pc.idx);
  else if (r.k == 3)
    run_piece<3, NS>(a, r, t0, ns, pc.chunk, pc.s0, pc.s1, pc.idx);
  else
    run_piece<4, NS>(a, r, t0, ns, pc.chunk, pc.s0, pc.s1, pc.idx);
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
  int16_t* row = q + (size_t)(strip * 16 + n) * in + (ti0 + g) * 16;
  if (path == 0) {
    uint32_t M[8];
    decode_col<K>(cw, lo.sel3, M);
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
    // the prefill GEMM's operands (prefill_half for K = 2, 3, as its main loop decodes
    // them; prefill_full for K = 4): V[r] holds inputs r (high half) and r + 8 (low half)
    // as the f16 subnormals (q + 255) * 2^-24
    uint32_t V[8];
    const uint32_t w1 = cw.w[K == 2 ? 0 : 1], wn = row_next(cw.w[0]);
    if constexpr (K == 4) {
      prefill_full<K>(cw.w[0], w1, wn, lo.sel3, V, V + 4);
    } else {
      prefill_half<K>(cw.w[0], w1, wn, lo.sel3, 0, V);
      prefill_half<K>(cw.w[0], w1, wn, lo.sel3, 1, V + 4);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      row[r] = (int16_t)(f16_bits_to_f32(V[r] >> 16) * BYTE_SUM_SCALE - BYTE_SUM_OFFSET);
      row[r + 8] = (int16_t)(f16_bits_to_f32(V[r]) * BYTE_SUM_SCALE - BYTE_SUM_OFFSET);
    }
  }
}

// ---- repack into the read order ---------------------------------------------------------
// Thread i of grid row e copies 16-byte chunk i of unit e from its run in the store order
// `from` (layout 0 or 2) to the same run in read order (run_word). Chunk i belongs to run
// r = i / (8 K), taken as strip r / S, step r % S (every run is found once). A unit is out / 16 strips x S runs of 128 K bytes; bad
// units (width not 2..4, misaligned, not inside codes) are skipped.
__global__ __launch_bounds__(256) void trellis_repack_kernel(const uint8_t* __restrict__ bits,
                                                             const int64_t* __restrict__ code_off,
                                                             const uint32_t* __restrict__ codes,
                                                             int64_t codes_bytes, int out, int in,
                                                             int from, uint32_t* __restrict__ dst) {
  const int e = blockIdx.y;
  const int K = bits[e];
  const int64_t off = code_off[e];
  const int64_t ub = (int64_t)out * in / 8 * K;
  if (K < 2 || K > 4 || (off & 15) || off < 0 || off > codes_bytes - ub) return;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= ub / 16) return;
  const int TW = 8 * K, S = in / 64, nst = out / 16;
  const int per_run = 8 * K;  // 16-byte chunks per run (128 K bytes)
  const int r = (int)(i / per_run), c = (int)(i % per_run);
  const int t = r / S, st = r % S;
  const uint4* src = reinterpret_cast<const uint4*>(codes + off / 4 + run_word(from, t, st, S, nst, TW));
  uint4* to = reinterpret_cast<uint4*>(dst + off / 4 + run_word(1, t, st, S, nst, TW));
  to[c] = src[c];
}

}  // namespace

hipError_t launch_trellis_repack(const uint8_t* bits, const int64_t* code_off,
                                 const uint32_t* codes, int64_t codes_bytes, int E, int out,
                                 int in, int from, uint32_t* dst, hipStream_t s) {
  const int64_t chunks = (int64_t)out * in / 8 * 4 / 16;  // of the widest unit
  const dim3 grid((unsigned)((chunks + 255) / 256), (unsigned)E);
  hipLaunchKernelGGL(trellis_repack_kernel, grid, dim3(256), 0, s, bits, code_off, codes,
                     codes_bytes, out, in, from, dst);
  return hipGetLastError();
}

int trellis_gemv_grid() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[dev]) return cache[dev];
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, trellis_gemv_kernel, GEMV_THREADS, 0) !=
      hipSuccess)
    return 0;
  per_cu *= GEMV_WG_WAVES;  // waves
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  // pieces: two waves each, up to 4 waves per SIMD
  int g = std::min(per_cu, 2 * GEMV_TARGET_PER_CU) * cus / (8 / GEMV_NS);
  if (g > GEMV_MAX_G) g = GEMV_MAX_G;
  if (g < 1) g = 1;
  if (dev >= 0 && dev < 64) cache[dev] = g;
  return g;
}

hipError_t launch_trellis_gemv(const TrellisGemvArgs& a, hipStream_t s) {
  const int waves = a.G * (8 / GEMV_NS);
  return launch_timed(trellis_gemv_kernel, dim3((waves + GEMV_WG_WAVES - 1) / GEMV_WG_WAVES),
                      dim3(GEMV_THREADS), s, a);
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

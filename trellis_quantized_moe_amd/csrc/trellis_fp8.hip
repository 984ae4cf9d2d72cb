// FP8 variant of the trellis prefill (FORMAT F19; DeepSeek-V4.1-Flash-1017 TrellisMX K2 Mix
// page, "Credits": the trellis decoded straight into FP8 E4M3 tensor-core operands).
//
// 1. tf8_prep_kernel: the activations, optionally rotated first (F8, bf16 result), become
//    MXFP8 (F18): per 32 inputs an E8M0 byte b with max|x| / 2^(b - 127) in [128, 256) and
//    E4M3 codes of x 2^(127 - b). A 128-block is held by 16 lanes, 8 inputs each; the 4
//    lanes of a 32-block share its largest magnitude by two cross-lane steps. The codes of
//    each 16-input chunk are stored in the order the weight decoder produces them (below):
//    dword d of the chunk holds the inputs 2d + 8, 2d, 2d + 9, 2d + 1 (bytes 0..3). The
//    matrix cores pair byte j of the activations with byte j of the weights, so any order
//    applied to both gives the same sum, and the 32-input scale blocks are untouched.
// 2. tf8_gemm_kernel: a work item is up to 128 routed rows of one expert times one group of
//    128 output channels, in steps of 128 inputs, on four waves: wave w owns strips 2w and
//    2w + 1 (32 channels) for all rows, so no weight is decoded twice and none passes
//    through LDS.
//      - weights: lane (q, n) decodes, for each of its strips, column n of tiles 8 kk + q and
//        8 kk + 4 + q: 32 E4M3 codes, the operand of inputs 16 q .. 16 q + 15 and
//        64 + 16 q .. 64 + 16 q + 15 of channel n (the fp8 operand layout of
//        v_mfma_scale_f32_16x16x128_f8f6f4). A tile column's m-pairs (trellis_decode.h) give
//        the byte sums v = q + 255 as 16-bit integers; 0x6400 + v is the f16 1024 + v, one
//        packed f16 subtraction of 1279 gives q exactly, and the hardware conversion rounds
//        two f16 values to E4M3 (nearest, ties to even) per instruction. Code words are
//        loaded two steps ahead into registers.
//      - activations: the item's gathered MXFP8 rows are loaded into a 4-stage LDS ring two
//        steps ahead by buffer loads that write LDS (16-byte chunk c of row r at position
//        c ^ (r % 8)), with each row's 4 block scales.
//    Per step and wave: 8 x 2 products (weight block scales 2^0), fp32 accumulation. The
//    epilogue applies the channel's fp16 scale and the gate and writes each output once.
//    Layers with the exlr8 codebooks (F20 mul1, F21 pmcgx; codebook_decode.h) run the same
//    kernel with their decoder in place of T16's; mul1's operand is E4M3(q / 2) with the
//    weight block scale 2^1.
// 3. tf8_decode_kernel: the decode hook's paths 2 (T16), 3 (mul1) and 4 (pmcgx), the E4M3
//    codes of a unit through the same decoders, in natural order.
#include "gemm_core.h"
#include "hadamard_lane.h"
#include "codebook_decode.h"
#include "trellis_cols.h"

namespace tq {

namespace {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

// ---- activations ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tf8_prep_kernel(const uint16_t* __restrict__ x,
                                                       int64_t nblocks, int n, int rotate,
                                                       const int8_t* __restrict__ signs,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int64_t gtid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gtid >> 4;
  const int sub = threadIdx.x & 15;
  const bool active = blk < nblocks;
  const int64_t bpr = n / 128;
  const int64_t row = active ? blk / bpr : 0;
  const int col0 = active ? (int)(blk % bpr) * 128 + 8 * sub : 0;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (active) {
    const uint4 w = *reinterpret_cast<const uint4*>(x + row * n + col0);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[2 * t] = bf16_lo_to_f32(ww[t]);
      v[2 * t + 1] = bf16_hi_to_f32(ww[t]);
    }
    if (rotate && signs) {
      const uint2 sg = *reinterpret_cast<const uint2*>(signs + col0);
      const uint32_t s2[2] = {sg.x, sg.y};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((int8_t)((s2[j >> 2] >> (8 * (j & 3))) & 0xFF) < 0) v[j] = -v[j];
    }
  }
  if (rotate) {  // F8: fp32 butterflies, x 0x3DB504F3, bf16 nearest-even
    fwht128_lane8(v, sub);
    const float scale = __uint_as_float(0x3DB504F3u);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * scale;
    round_bf16_pairs<8>(v);
  }
  // the 32-block's largest magnitude (an infinity or NaN makes it +inf): lanes 4c .. 4c + 3
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float m = fabsf(v[j]);
    amax = fmaxf(amax, m <= 3.4e38f ? m : __builtin_inff());
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  int b = 127;
  if (!(amax <= 3.4e38f)) {
    b = 255;
  } else if (amax > 0.0f) {
    int ex;
    (void)frexpf(amax, &ex);  // amax in [2^(ex - 1), 2^ex)
    b = min(max(ex - 1 - 7 + 127, 0), 254);
  }
  const float mul = b == 255 ? 0.0f : ldexpf(1.0f, 127 - b);
  // P[d] = codes of inputs 2d, 2d + 1 of this lane's 8; own01 = P[0], P[1]; own23 = P[2], P[3]
  const uint32_t p01 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[0] * mul, v[1] * mul, 0, false);
  const uint32_t own01 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2] * mul, v[3] * mul, (int)p01, true);
  const uint32_t p23 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4] * mul, v[5] * mul, 0, false);
  const uint32_t own23 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[6] * mul, v[7] * mul, (int)p23, true);
  // a 16-input chunk is lanes 2c (inputs 0..7) and 2c + 1 (inputs 8..15); the low lane
  // writes dwords 0, 1 of the chunk, the high lane dwords 2, 3
  const bool low = (sub & 1) == 0;
  const uint32_t recv = (uint32_t)__shfl_xor((int)(low ? own23 : own01), 1, 64);
  uint32_t d0, d1;
  if (low) {  // own = inputs 0..3, recv = inputs 8..11
    d0 = perm(recv, own01, 0x01050004u);  // [x8, x0, x9, x1]
    d1 = perm(recv, own01, 0x03070206u);  // [x10, x2, x11, x3]
  } else {    // own = inputs 12..15, recv = inputs 4..7
    d0 = perm(recv, own23, 0x05010400u);  // [x12, x4, x13, x5]
    d1 = perm(recv, own23, 0x07030602u);  // [x14, x6, x15, x7]
  }
  if (!active) return;
  *reinterpret_cast<uint2*>(codes + row * n + col0) = make_uint2(d0, d1);
  if ((sub & 3) == 0) scales[row * (n / 32) + col0 / 32] = (uint8_t)b;
}

// ---- weights ----------------------------------------------------------------------------------
// E4M3 codes of two T16 values from their m-pair M ([hi: m_a, lo: m_b]), into half `hi` of
// `old`: byte 0 of the half is m_b's code, byte 1 m_a's.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t M, uint32_t old) {
  const uint32_t v = byte_sum_pair(M);                      // q + 255, two 16-bit lanes
  const u16x2 f = __builtin_bit_cast(u16x2, v) + (u16x2){0x6400, 0x6400};  // f16 1024 + v
  const h16x2 q = __builtin_bit_cast(h16x2, f) - (h16x2){(_Float16)1279.0f, (_Float16)1279.0f};
  const i16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(__builtin_bit_cast(i16x2, old), q, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// The 16 E4M3 codes of a tile column in the activations' chunk order: D[d] holds inputs
// 2d + 8, 2d, 2d + 9, 2d + 1.
template <int K>
__device__ __forceinline__ void e4m3_col(const uint32_t M[8], uint32_t D[4]) {
  if constexpr (K == 4) {
    // M[r] (r < 4) = [hi: m(r), lo: m(r + 4)]; M[r] (r >= 4) = [hi: m(r + 4), lo: m(r + 8)]
    const uint32_t w01 = e4m3_pair<true>(M[1], e4m3_pair<false>(M[0], 0));  // [q4, q0, q5, q1]
    const uint32_t w23 = e4m3_pair<true>(M[3], e4m3_pair<false>(M[2], 0));  // [q6, q2, q7, q3]
    const uint32_t w45 = e4m3_pair<true>(M[5], e4m3_pair<false>(M[4], 0));  // [q12, q8, q13, q9]
    const uint32_t w67 = e4m3_pair<true>(M[7], e4m3_pair<false>(M[6], 0));  // [q14, q10, q15, q11]
    D[0] = perm(w45, w01, 0x03070105u);
    D[1] = perm(w67, w23, 0x03070105u);
    D[2] = perm(w45, w01, 0x02060004u);
    D[3] = perm(w67, w23, 0x02060004u);
  } else {
    // M[r] = [hi: m(r), lo: m(r + 8)]
#pragma unroll
    for (int d = 0; d < 4; ++d) D[d] = e4m3_pair<true>(M[2 * d + 1], e4m3_pair<false>(M[2 * d], 0));
  }
}

// ---- the GEMM ---------------------------------------------------------------------------------
constexpr int TF_THREADS = 256;
constexpr int TF_STAGES = 4;  // a stage refilled at step kk was last read at step kk - 2
constexpr int TF_ROW = 128;  // bytes of one row per step (128 inputs)

struct TfShared {
  alignas(16) uint8_t a[TF_STAGES][GEMM_MT * TF_ROW];
  alignas(16) uint32_t s[TF_STAGES][GEMM_MT];  // the row's 4 block scales of the step
  int slot[GEMM_MT];
  float gate[GEMM_MT];
};

// Vector-memory instructions a wave issues per step: 4 activation chunks, the scale row
// (waves 0 and 1), the code words (2 strips x 2 runs, one load each).
template <int K, bool SCALES>
constexpr int tf_step_loads() {
  return 4 + (SCALES ? 1 : 0) + 4;
}

// The 16 E4M3 operand codes of one tile column (in the activations' chunk order) with
// codebook CB.
template <int K, int CB>
__device__ __forceinline__ void fp8_col(const ColWords<K>& cw, uint32_t sel3, uint32_t D[4]) {
  if constexpr (CB == CB_MUL1) {
    mul1_col<K>(cw, sel3, D);
  } else if constexpr (CB == CB_PMCGX) {
    pmcgx_col<K>(cw, sel3, D);
  } else {
    uint32_t M[8];
    decode_col<K>(cw, sel3, M);
    e4m3_col<K>(M, D);
  }
}

template <int K, int CB>
__device__ void tf_item(const TrellisFp8GemmArgs& a, TfShared& sh, const uint32_t* unit, int e,
                        int grp, int nrows, int ns) {
  constexpr int BSCALE = CB == CB_MUL1 ? 128 : 127;  // E8M0 of the weight operand
  constexpr int TW = 8 * K;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nsteps = a.in / 128;  // even
  const bool scale_loader = w < 2;

  // activation chunks: instruction j of wave w fills rows 32 w + 8 j .. + 7 of a stage
  const GemmRsrc ra = gemm_rsrc(a.xa, a.xa_bytes);
  uint32_t avo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * w + 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    avo[j] = r < nrows ? (uint32_t)((sh.slot[r] / a.topk) * a.in) + 16u * c : 0x80000000u;
  }
  const GemmRsrc rs = gemm_rsrc(a.xs, a.xs_bytes);
  const int srow = 64 * (w & 1) + lane;
  const uint32_t svo = srow < nrows ? (uint32_t)((sh.slot[srow] / a.topk) * (a.in / 32)) : 0x80000000u;
  auto load_a = [&](int st, int kk) {
    uint8_t* base = sh.a[st] + 32 * w * TF_ROW;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LdsPtr)(base + 8 * j * TF_ROW), 16, avo[j],
                                               (uint32_t)(TF_ROW * kk), 0, 0);
    if (scale_loader)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LdsPtr)(&sh.s[st][64 * w]), 4, svo,
                                               (uint32_t)(4 * kk), 0, 0);
  };

  // code words: strip 8 grp + 2 w + s (clamped to the group's last strip), runs 2 kk and
  // 2 kk + 1 (tile columns 8 kk .. 8 kk + 3 and 8 kk + 4 .. 8 kk + 7); lane (q, n) takes
  // column n of tile q of each run
  const int S = a.in / 64, nst = a.out / 16;
  const LaneOffsets<K> lo(q, n);
  const Rsrc rc = make_rsrc(unit, (uint32_t)((size_t)a.out * a.in * K / 8));
  const uint32_t cvo[2] = {4u * lo.o[0], 4u * lo.o[1]};
  uint32_t sso[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int t = min(2 * w + s, ns - 1);
    sso[s] = 4u * (run_word(a.layout, 8 * grp + t, 0, S, nst, TW) -
                   run_word(a.layout, 8 * grp, 0, S, nst, TW));
  }
  auto cso = [&](int run) { return 4u * run_word(a.layout, 8 * grp, run, S, nst, TW); };
  ColWords<K> cw[2][2][2];  // [slot][strip][run]
  auto load_b = [&](int d, int kk) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) load_col_buf<K>(rc, cvo, cso(2 * kk + h) + sso[s], cw[d][s][h]);
  };

  f32x4 acc[8][2];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int s = 0; s < 2; ++s) acc[mb][s] = (f32x4){0.f, 0.f, 0.f, 0.f};
  int mblocks = (nrows + 15) / 16;
  mblocks = mblocks > 8 ? 8 : mblocks;

  load_a(0, 0);
  load_b(0, 0);
  load_a(1, 1);
  load_b(1, 1);

  auto step = [&](int kk, int d) {
    // this wave's loads of step kk have landed (those of kk + 1 may be in flight); after the
    // barrier every wave's have, and every wave is done with the stage refilled below
    if (scale_loader)
      wait_vmcnt<tf_step_loads<K, true>()>();
    else
      wait_vmcnt<tf_step_loads<K, false>()>();
    bare_barrier();
    const int nxt = kk + 2 < nsteps ? kk + 2 : nsteps - 1;
    load_a((kk + 2) % TF_STAGES, nxt);
    uint32_t B[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) fp8_col<K, CB>(cw[d][s][h], lo.sel3, B[s] + 4 * h);
    load_b(d, nxt);  // the registers just decoded, for step kk + 2
    const uint8_t* st = sh.a[kk % TF_STAGES];
    const uint32_t* ss = sh.s[kk % TF_STAGES];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      if (mb < mblocks) {
        const int r = 16 * mb + n;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(st + r * TF_ROW + 16 * (q ^ (r & 7)));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(st + r * TF_ROW + 16 * ((4 + q) ^ (r & 7)));
        const int sa = (int)((ss[r] >> (8 * q)) & 0xFFu);
        const i32x8 av = (i32x8){(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                 (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const i32x8 bv = (i32x8){(int)B[s][0], (int)B[s][1], (int)B[s][2], (int)B[s][3],
                                   (int)B[s][4], (int)B[s][5], (int)B[s][6], (int)B[s][7]};
          acc[mb][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mb][s], 0, 0,
                                                                        0, sa, 0, BSCALE);
        }
      }
    }
  };
  for (int kk = 0; kk < nsteps; kk += 2) {
    step(kk, 0);
    step(kk + 1, 1);
  }
  // no load may still be writing this workgroup's LDS when it ends
  wait_vmcnt<0>();

#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int t = 2 * w + s;
    if (t < ns) {
      const int o = grp * 128 + 16 * t + n;
      const float sc = f16_bits_to_f32(a.scales[(size_t)e * a.out + o]);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * mb + 4 * q + i;
          if (row < nrows) a.y[(size_t)sh.slot[row] * a.out + o] = acc[mb][s][i] * sc * sh.gate[row];
        }
      }
    }
  }
}

template <int CB>
__global__ __launch_bounds__(TF_THREADS, 2) void tf8_gemm_kernel(TrellisFp8GemmArgs a) {
  __shared__ TfShared sh;
  int item, grp;
  if (!gemm_unit(a.n_items, a.groups, &item, &grp)) return;
  const int4 itd = reinterpret_cast<const int4*>(a.items)[item];
  const int e = itd.x, nrows = itd.z;
  const int K = a.bits[e];
  const int64_t off = a.code_off[e];
  const int ns = min(8, a.out / 16 - grp * 8);
  for (int m = threadIdx.x; m < GEMM_MT; m += TF_THREADS) {
    const int slot = m < nrows ? a.pairs[itd.y + m] : 0;
    sh.slot[m] = slot;
    sh.gate[m] = (m < nrows && a.gates) ? a.gates[slot] : 1.0f;
  }
  __syncthreads();
  const uint32_t* unit = a.codes + off / 4;
  // the unit must be 16-byte aligned and lie inside the code buffer
  const bool inside = !(off & 15) && off >= 0 &&
                      off <= a.codes_bytes - (int64_t)a.out * a.in / 8 * (K >= 2 && K <= 4 ? K : 0);
  if (K == 2 && inside) {
    tf_item<2, CB>(a, sh, unit, e, grp, nrows, ns);
  } else if (K == 3 && inside) {
    tf_item<3, CB>(a, sh, unit, e, grp, nrows, ns);
  } else if (K == 4 && inside) {
    tf_item<4, CB>(a, sh, unit, e, grp, nrows, ns);
  } else {
    for (int v = threadIdx.x; v < nrows * ns * 16; v += TF_THREADS) {
      const int m = v / (ns * 16), o = grp * 128 + v % (ns * 16);
      a.y[(size_t)sh.slot[m] * a.out + o] = __builtin_nanf("");
    }
    if (threadIdx.x == 0) set_status(a.status, STATUS_BAD_UNIT);
  }
}

// ---- decode hook ------------------------------------------------------------------------------
// One wave per (strip, run of 4 tile columns): lane (g, n) decodes column n of tile g with
// the GEMM's decoder and writes the 16 E4M3 codes in input order as int16.
template <int K, int CB>
__global__ __launch_bounds__(256) void tf8_decode_kernel(const uint32_t* __restrict__ codes,
                                                         int out, int in, int16_t* __restrict__ q) {
  constexpr int TW = 8 * K;
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int n_ti = in / 16;
  const int runs = n_ti / 4;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= (out / 16) * runs) return;  // whole wave exits together
  const int strip = wave / runs, ti0 = (wave % runs) * 4;
  const LaneOffsets<K> lo(g, n);
  ColWords<K> cw;
  load_col<K>(codes + (size_t)(strip * n_ti + ti0) * TW, lo, cw);
  uint32_t D[4];
  fp8_col<K, CB>(cw, lo.sel3, D);
  int16_t* row = q + (size_t)(strip * 16 + n) * in + (ti0 + g) * 16;
#pragma unroll
  for (int d = 0; d < 4; ++d) {  // D[d] = [c(2d + 8), c(2d), c(2d + 9), c(2d + 1)]
    row[2 * d] = (int16_t)((D[d] >> 8) & 0xFF);
    row[2 * d + 1] = (int16_t)(D[d] >> 24);
    row[2 * d + 8] = (int16_t)(D[d] & 0xFF);
    row[2 * d + 9] = (int16_t)((D[d] >> 16) & 0xFF);
  }
}

}  // namespace

hipError_t launch_tf8_prep(const uint16_t* x, int64_t rows, int n, bool rotate,
                           const int8_t* signs, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nblocks = rows * (n / 128);
  if (nblocks == 0) return hipSuccess;
  const int64_t grid = (nblocks * 16 + 255) / 256;
  hipLaunchKernelGGL(tf8_prep_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, nblocks, n,
                     rotate ? 1 : 0, signs, codes, scales);
  return hipGetLastError();
}

hipError_t launch_tf8_gemm(const TrellisFp8GemmArgs& a, hipStream_t s) {
  const int blocks = gemm_grid(a.max_items, a.groups);
  if (blocks == 0) return hipSuccess;
  if (a.codebook == CB_MUL1)
    return launch_timed(tf8_gemm_kernel<CB_MUL1>, dim3(blocks), dim3(TF_THREADS), s, a);
  if (a.codebook == CB_PMCGX)
    return launch_timed(tf8_gemm_kernel<CB_PMCGX>, dim3(blocks), dim3(TF_THREADS), s, a);
  return launch_timed(tf8_gemm_kernel<CB_T16>, dim3(blocks), dim3(TF_THREADS), s, a);
}

template <int CB>
static void tf8_decode_launch(const uint32_t* codes, int K, int out, int in, int16_t* q,
                              int blocks, hipStream_t s) {
  if (K == 2)
    hipLaunchKernelGGL((tf8_decode_kernel<2, CB>), dim3(blocks), dim3(256), 0, s, codes, out, in, q);
  else if (K == 3)
    hipLaunchKernelGGL((tf8_decode_kernel<3, CB>), dim3(blocks), dim3(256), 0, s, codes, out, in, q);
  else
    hipLaunchKernelGGL((tf8_decode_kernel<4, CB>), dim3(blocks), dim3(256), 0, s, codes, out, in, q);
}

hipError_t launch_tf8_decode(const uint32_t* codes, int K, int out, int in, int16_t* q,
                             int codebook, hipStream_t s) {
  const int waves = (out / 16) * (in / 64);
  const int blocks = (waves + 3) / 4;
  if (codebook == CB_MUL1)
    tf8_decode_launch<CB_MUL1>(codes, K, out, in, q, blocks, s);
  else if (codebook == CB_PMCGX)
    tf8_decode_launch<CB_PMCGX>(codes, K, out, in, q, blocks, s);
  else
    tf8_decode_launch<CB_T16>(codes, K, out, in, q, blocks, s);
  return hipGetLastError();
}

}  // namespace tq

// FP8 matrix-core variant of the MXFP4 prefill (FORMAT F18; DeepSeek-V4.1-Flash-1017
// TrellisMX K2 Mix page, "Credits": FP8 E4M3 tensor-core operands; exlr8 page, "Stores": the
// official MXFP4 store): gfx950's block-scaled matrix cores multiply the stored E2M1 codes
// with their E8M0 scales as they are, against activations converted once to MXFP8.
//
// 1. mxfp8_prep_kernel: each thread converts one block of 32 inputs of one row: the block's
//    largest magnitude gives the E8M0 byte b (max / 2^(b - 127) in [128, 256)), the values
//    times 2^(127 - b) (exact) are rounded to E4M3 by the hardware conversion (nearest,
//    ties to even; no value can reach 448). Codes [rows][n], scales [rows][n / 32].
// 2. mx8_gemm_kernel: a work item is up to 128 routed rows of one expert times one group of
//    128 output channels over the whole input range, in steps of 128 inputs, on four waves,
//    wave w owning channels 32 w .. 32 w + 31 for all rows (so no weight is loaded twice).
//    Per step and wave: 8 x 2 products
//    v_mfma_scale_f32_16x16x128_f8f6f4 (A: E4M3 activations with their block scales, B: E2M1
//    weights with theirs, fp32 accumulation).
//      - weights: lane (n, q) of a 16-channel block supplies the 32 codes of inputs
//        32 q .. 32 q + 31 of its channel (16 contiguous bytes, one 16-byte load straight
//        from the unit) and that block's scale byte, so nothing is decoded; the scale bytes
//        come 16 at a time (4 steps of the channel's row) every fourth step, since a load's
//        cost is set by its lanes, not by its bytes;
//      - activations: the item's gathered rows are loaded into a 4-stage LDS ring two steps
//        ahead by buffer loads that write LDS (16-byte chunk c of row r at position
//        c ^ (r % 8)), with each row's 4 block scales; lane (r, q) reads the chunks of
//        inputs 16 q .. 16 q + 15 and 64 + 16 q .. 64 + 16 q + 15 of its row (the operand
//        layout of the fp8 source of this instruction) and the row's scale of block q.
//    The epilogue multiplies by the gate and writes each output once.
#include "gemm_core.h"
#include "mx_unit.h"

namespace tq {

namespace {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void mxfp8_prep_kernel(const uint16_t* __restrict__ x,
                                                         int64_t nblocks, int n,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= nblocks) return;
  const int per_row = n / 32;
  const int64_t row = blk / per_row;
  const int j = (int)(blk % per_row);
  const uint4* src = reinterpret_cast<const uint4*>(x + row * n + 32 * j);
  float f[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 u = src[q];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f[8 * q + 2 * t] = bf16_lo_to_f32(w[t]);
      f[8 * q + 2 * t + 1] = bf16_hi_to_f32(w[t]);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    const float m = fabsf(f[t]);
    amax = fmaxf(amax, m <= 3.4e38f ? m : __builtin_inff());
  }
  int b = 127;
  if (!(amax <= 3.4e38f)) {
    b = 255;
  } else if (amax > 0.0f) {
    int ex;
    (void)frexpf(amax, &ex);  // amax in [2^(ex - 1), 2^ex)
    b = min(max(ex - 1 - 7 + 127, 0), 254);
  }
  const float mul = b == 255 ? 0.0f : ldexpf(1.0f, 127 - b);
  uint32_t out[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[4 * t] * mul, f[4 * t + 1] * mul, 0, false);
    out[t] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[4 * t + 2] * mul, f[4 * t + 3] * mul, (int)lo, true);
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + row * n + 32 * j);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  scales[row * per_row + j] = (uint8_t)b;
}

constexpr int M8_THREADS = 256;
constexpr int M8_STAGES = 4;
constexpr int M8_ROW = 128;  // bytes of one row per step (128 inputs)

struct M8Shared {
  alignas(16) uint8_t a[M8_STAGES][GEMM_MT * M8_ROW];
  alignas(16) uint32_t s[M8_STAGES][GEMM_MT];  // the row's 4 block scales of the step
  int slot[GEMM_MT];
  float gate[GEMM_MT];
};

// Vector-memory instructions a wave issues per step: A chunks (4), the scale rows (waves 0
// and 1: one each) and the weight codes (2); every fourth step (the first of a window of
// four steps) also the weight scales of the next window (2).
constexpr int M8_NB = 2;  // 16-channel blocks per wave
template <bool SCALES>
constexpr int m8_step_loads() {
  return 4 + (SCALES ? 1 : 0) + M8_NB;
}

template <int LAYOUT>
__device__ void m8_item(const Mx8GemmArgs& a, M8Shared& sh, const uint8_t* unit, int grp,
                        int nrows, int ns) {
  using U = MxUnit<MX_FP4>;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nsteps = a.in / 128;  // a multiple of 4
  const bool scale_loader = w < 2;

  // activation chunks: instruction j of wave w fills rows 32 w + 8 j .. + 7 of a stage; lane
  // l writes position l % 8 of row 32 w + 8 j + l / 8, which holds chunk (l % 8) ^ (row % 8)
  const GemmRsrc ra = gemm_rsrc(a.xa, a.xa_bytes);
  uint32_t avo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * w + 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    avo[j] = r < nrows ? (uint32_t)((sh.slot[r] / a.topk) * a.in) + 16u * c : 0x80000000u;
  }
  // scale rows: lane l of wave w < 2 loads the 4 block scales of row 64 w + l
  const GemmRsrc rs = gemm_rsrc(a.xs, a.xs_bytes);
  const int srow = 64 * (w & 1) + lane;
  const uint32_t svo = srow < nrows ? (uint32_t)((sh.slot[srow] / a.topk) * (a.in / 32)) : 0x80000000u;
  // stage st receives the chunks of step kk (past the last step: the last step's again, into
  // a stage no step reads any more, so every step issues the same loads)
  auto load_a = [&](int st, int kk) {
    uint8_t* base = sh.a[st] + 32 * w * M8_ROW;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LdsPtr)(base + 8 * j * M8_ROW), 16, avo[j],
                                               (uint32_t)(M8_ROW * kk), 0, 0);
    if (scale_loader)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LdsPtr)(&sh.s[st][64 * w]), 4, svo,
                                               (uint32_t)(4 * kk), 0, 0);
  };

  // weights: lane (n, q) of block nb: channel o = 128 grp + 32 w + 16 nb + n (channels past
  // the group read its last one; their outputs are not stored), codes of 32-block 4 kk + q
  const GemmRsrc rb = gemm_rsrc(unit, (uint32_t)U::unit_bytes(a.out, a.in));
  uint32_t bvo[M8_NB], bso[M8_NB];
#pragma unroll
  for (int nb = 0; nb < M8_NB; ++nb) {
    const int oc = 32 * w + 16 * nb + n;
    const int o = grp * 128 + (oc < 16 * ns ? oc : 16 * ns - 1);
    bvo[nb] = LAYOUT ? U::packed_at(a.out, a.in, o, q) : U::stored_at(a.in, o, q);
    bso[nb] = U::scale_at(a.out, a.in, o, 0);  // the channel's scale row (16-byte aligned)
  }
  // scalar step offsets of the codes (kb = 4 kk + q: store order 64 kk bytes; read order one
  // chunk per step of the group)
  const uint32_t bstep = LAYOUT ? (uint32_t)(U::packed_at(a.out, a.in, grp * 128, 4) -
                                             U::packed_at(a.out, a.in, grp * 128, 0))
                                : 64u;
  u32x4 bc[2][M8_NB];
  auto load_b = [&](int slot, int kk) {
#pragma unroll
    for (int nb = 0; nb < M8_NB; ++nb)
      bc[slot][nb] = __builtin_amdgcn_raw_buffer_load_b128(rb, bvo[nb], (uint32_t)kk * bstep, 0);
  };
  // weight scales by windows of 4 steps: 16 bytes of the channel's scale row (blocks
  // 16 wi .. 16 wi + 15), one load per block of channels instead of one per step; byte
  // 4 t + q is the scale of step 4 wi + t for this lane. Two windows alternate.
  const int nwin = nsteps / 4;
  u32x4 sw[2][M8_NB];
  auto load_s = [&](int slot, int wi) {
    const uint32_t off = 16u * (uint32_t)(wi < nwin ? wi : nwin - 1);
#pragma unroll
    for (int nb = 0; nb < M8_NB; ++nb)
      sw[slot][nb] = __builtin_amdgcn_raw_buffer_load_b128(rb, bso[nb], off, 0);
  };

  f32x4 acc[8][M8_NB];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < M8_NB; ++nb) acc[mb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  int mblocks = (nrows + 15) / 16;
  mblocks = mblocks > 8 ? 8 : mblocks;

  // prologue: the first scale window, steps 0 and 1
  load_s(0, 0);
  load_a(0, 0);
  load_b(0, 0);
  load_a(1, 1);
  load_b(1, 1);

  // step kk, position t = kk % 4 in scale window slot ws; d = code slot
  auto step = [&](int kk, int d, int t, int ws) {
    // this wave's loads of step kk have landed (those of kk + 1 may be in flight; the second
    // step of a window also lets the next window's scales, issued by the first, be in flight)
    if (t == 1) {
      if (scale_loader)
        wait_vmcnt<m8_step_loads<true>() + M8_NB>();
      else
        wait_vmcnt<m8_step_loads<false>() + M8_NB>();
    } else {
      if (scale_loader)
        wait_vmcnt<m8_step_loads<true>()>();
      else
        wait_vmcnt<m8_step_loads<false>()>();
    }
    bare_barrier();
    if (t == 0) load_s(ws ^ 1, kk / 4 + 1);
    const int nxt = kk + 2 < nsteps ? kk + 2 : nsteps - 1;
    load_a((kk + 2) % M8_STAGES, nxt);
    const uint8_t* st = sh.a[kk % M8_STAGES];
    const uint32_t* ss = sh.s[kk % M8_STAGES];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      if (mb < mblocks) {
        const int r = 16 * mb + n;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(st + r * M8_ROW + 16 * (q ^ (r & 7)));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(st + r * M8_ROW + 16 * ((4 + q) ^ (r & 7)));
        const int sa = (int)((ss[r] >> (8 * q)) & 0xFFu);
        const i32x8 av = (i32x8){(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                 (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
        for (int nb = 0; nb < M8_NB; ++nb) {
          const u32x4 b = bc[d][nb];
          const i32x8 bv = (i32x8){(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
          const int sb = (int)((sw[ws][nb][t] >> (8 * q)) & 0xFFu);
          acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              av, bv, acc[mb][nb], 0, 4, 0, sa, 0, sb);
        }
      }
    }
    load_b(d, nxt);  // the slot just used, for step kk + 2
  };
  for (int kk = 0; kk < nsteps; kk += 8) {
    step(kk, 0, 0, 0);
    step(kk + 1, 1, 1, 0);
    step(kk + 2, 0, 2, 0);
    step(kk + 3, 1, 3, 0);
    if (kk + 4 < nsteps) {
      step(kk + 4, 0, 0, 1);
      step(kk + 5, 1, 1, 1);
      step(kk + 6, 0, 2, 1);
      step(kk + 7, 1, 3, 1);
    }
  }
  // no load may still be writing this workgroup's LDS when it ends
  wait_vmcnt<0>();

#pragma unroll
  for (int nb = 0; nb < M8_NB; ++nb) {
    const int oc = 32 * w + 16 * nb + n;
    if (oc < 16 * ns) {
      const int o = grp * 128 + oc;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * mb + 4 * q + i;
          if (row < nrows) a.y[(size_t)sh.slot[row] * a.out + o] = acc[mb][nb][i] * sh.gate[row];
        }
      }
    }
  }
}

__global__ __launch_bounds__(M8_THREADS, 2) void mx8_gemm_kernel(Mx8GemmArgs a) {
  __shared__ M8Shared sh;
  int item, grp;
  if (!gemm_unit(a.n_items, a.groups, &item, &grp)) return;
  const int4 itd = reinterpret_cast<const int4*>(a.items)[item];
  const int e = itd.x, nrows = itd.z;
  for (int m = threadIdx.x; m < GEMM_MT; m += M8_THREADS) {
    const int slot = m < nrows ? a.pairs[itd.y + m] : 0;
    sh.slot[m] = slot;
    sh.gate[m] = (m < nrows && a.gates) ? a.gates[slot] : 1.0f;
  }
  __syncthreads();
  const int ns = min(8, a.out / 16 - grp * 8);
  const uint8_t* unit = a.units + (size_t)e * MxUnit<MX_FP4>::unit_bytes(a.out, a.in);
  if (a.layout)
    m8_item<1>(a, sh, unit, grp, nrows, ns);
  else
    m8_item<0>(a, sh, unit, grp, nrows, ns);
}

}  // namespace

hipError_t launch_mxfp8_prep(const uint16_t* x, int64_t rows, int n, uint8_t* codes,
                             uint8_t* scales, hipStream_t s) {
  const int64_t nblocks = rows * (n / 32);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_prep_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s,
                     x, nblocks, n, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx8_gemm(const Mx8GemmArgs& a, hipStream_t s) {
  const int blocks = gemm_grid(a.max_items, a.groups);
  if (blocks == 0) return hipSuccess;
  return launch_timed(mx8_gemm_kernel, dim3(blocks), dim3(M8_THREADS), s, a);
}

}  // namespace tq

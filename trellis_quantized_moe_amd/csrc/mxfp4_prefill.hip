// Prefill grouped GEMM over the E8M0-scaled stores on the bf16 matrix cores (gfx950;
// DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores": MXFP4, the official expert store, E2M1
// codes with one E8M0 scale per 32 inputs of a channel; fp8b32, the shared expert's store,
// E4M3 codes with one E8M0 scale per 32 x 32 block).
//
// A work item is up to 128 routed rows of one expert times one group of up to 128 output
// channels over the whole input range, in steps of 64 inputs, on four waves: wave w owns
// channels 32 w .. 32 w + 31 (strips 2 w, 2 w + 1) for all rows, so no weight is loaded or
// converted twice and no weight passes through LDS.
//   - weights: lane (n, q) of a 16-channel strip takes inputs 16 q .. 16 q + 15 of the step
//     for channel n: 8 (MXFP4) or 16 (fp8b32) contiguous code bytes, one load in the store
//     order and in the GEMV's read order alike, and the scale of their 32-input block.
//     Eight hardware conversions (v_cvt_scalef32_pk_bf16_fp4 / _fp8, the scale applied
//     exactly) give the bf16 operands of the step's two 16x16x32 products: inputs
//     16 q .. 16 q + 7, then 16 q + 8 .. 16 q + 15. The activations take the same inputs in
//     the same order, so every product sums the same terms as the natural order.
//   - weight scales come 16 bytes of the scale row (the channel's, or its 32-channel
//     block's: 8 steps) per load, every eighth step, one window ahead;
//   - activations: the bf16 rows of the item are gathered into a 3-stage LDS ring, two steps
//     ahead, by loads that write LDS; each wave loads 32 of the 128 rows. Lane (r, q) needs
//     16-byte chunks 2 q and 2 q + 1 of row r, stored at positions q ^ (r % 8) and
//     (4 + q) ^ (r % 8) of the row (chunk 2 p at p, 2 p + 1 at 4 + p, then the xor): the 8
//     lanes the LDS serves together then hit 8 different chunk columns.
// Three items fit on a compute unit (49 KB of LDS each). The epilogue multiplies by the gate
// and writes each output once.
#include "gemm_core.h"
#include "mx_unit.h"

namespace tq {

namespace {

constexpr int MB_THREADS = 256;
constexpr int MB_STAGES = 3;
constexpr int MB_STEP = 64;            // inputs per step
constexpr int MB_ROW = MB_STEP * 2;    // bytes of one row per step
constexpr int MB_NB = 2;               // 16-channel strips per wave

struct MbShared {
  alignas(16) uint8_t a[MB_STAGES][GEMM_MT * MB_ROW];
  int slot[GEMM_MT];
  float gate[GEMM_MT];
};

// Vector-memory instructions a wave issues per step: 4 activation chunk loads and one code
// load per strip; the first step of each window of 8 also the next window's scales (one per
// strip).
constexpr int mb_step_loads() { return 4 + MB_NB; }

// A lane's code bytes of one step and strip: 8 (MXFP4) or 16 (fp8b32).
template <int FMT>
struct MbCodes;
template <>
struct MbCodes<MX_FP4> {
  u32x2 v;
  __device__ void load(GemmRsrc r, uint32_t vo, uint32_t so) {
    v = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0);
  }
  // bf16 operands of inputs 16 q .. 16 q + 7 (b0) and 16 q + 8 .. 16 q + 15 (b1)
  __device__ void convert(float sc, uint32_t b0[4], uint32_t b1[4]) const {
    fp4x8_to_bf16(v.x, sc, b0);
    fp4x8_to_bf16(v.y, sc, b1);
  }
};
template <>
struct MbCodes<MX_FP8B32> {
  u32x4 v;
  __device__ void load(GemmRsrc r, uint32_t vo, uint32_t so) {
    v = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0);
  }
  __device__ void convert(float sc, uint32_t b0[4], uint32_t b1[4]) const {
    fp8x4_to_bf16(v.x, sc, b0);
    fp8x4_to_bf16(v.y, sc, b0 + 2);
    fp8x4_to_bf16(v.z, sc, b1);
    fp8x4_to_bf16(v.w, sc, b1 + 2);
  }
};

// MBK: the row blocks of 16 the products run over (the item's rows rounded up to an even
// count of blocks; the rows past the item are zeros in the stages). A constant, so that the
// products of a step form one straight block in which the operand reads run ahead of the
// matrix-core work instead of each waiting on its own read.
template <int FMT, int LAYOUT, int MBK>
__device__ void mb_item(const Mxfp4GemmArgs& a, MbShared& sh, const uint8_t* unit, int grp,
                        int nrows, int ns) {
  using U = MxUnit<FMT>;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nsteps = a.in / MB_STEP;  // a multiple of 8 (in is a multiple of 512)

  // activation chunks: instruction j of wave w fills rows 32 w + 8 j .. + 7 of a stage; lane
  // l writes position l % 8 of row 32 w + 8 j + l / 8, which holds chunk 2 (x % 4) + x / 4,
  // x = (l % 8) ^ (row % 8). Rows past the item load from beyond the buffer's end
  // (x_bytes < 2^31) and read zeros.
  const GemmRsrc ra = gemm_rsrc(a.x, a.x_bytes);
  uint32_t avo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * w + 8 * j + (lane >> 3);
    const int x = (lane & 7) ^ (r & 7);
    const int c = 2 * (x & 3) + (x >> 2);
    avo[j] = r < nrows ? 2u * (uint32_t)((sh.slot[r] / a.topk) * a.in) + 16u * c : 0x80000000u;
  }
  // stage st receives the chunks of step kk (past the last step: the last step's again, into
  // a stage no step reads any more, so every step issues the same loads)
  auto load_a = [&](int st, int kk) {
    uint8_t* base = sh.a[st] + 32 * w * MB_ROW;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LdsPtr)(base + 8 * j * MB_ROW), 16, avo[j],
                                               (uint32_t)(MB_ROW * kk), 0, 0);
  };

  // weights: lane (n, q) of strip nb: channel o = 128 grp + 32 w + 16 nb + n (channels past
  // the group read its last one; their outputs are not stored). Step kk's code bytes: blocks
  // 2 kk and 2 kk + 1 (kCB bytes each) are adjacent in both layouts, and inputs
  // 16 q .. 16 q + 15 are bytes q kCB / 2 .. (q + 1) kCB / 2 - 1 of the pair.
  const GemmRsrc rb = gemm_rsrc(unit, (uint32_t)U::unit_bytes(a.out, a.in));
  uint32_t bvo[MB_NB], bso[MB_NB];
#pragma unroll
  for (int nb = 0; nb < MB_NB; ++nb) {
    const int oc = 32 * w + 16 * nb + n;
    const int o = grp * 128 + (oc < 16 * ns ? oc : 16 * ns - 1);
    bvo[nb] = (LAYOUT ? U::packed_at(a.out, a.in, o, 0) : U::stored_at(a.in, o, 0)) +
              (U::kCB / 2) * (uint32_t)q;
    bso[nb] = U::scale_at(a.out, a.in, o, 0);  // the scale row (16-byte aligned)
  }
  // scalar offset of step kk's codes: store order 2 kCB kk; read order, per 128-input step
  // of the group (ns strips of 64 kCB bytes), 2 kCB bytes for its second half
  const uint32_t pstep = (uint32_t)ns * 64u * U::kCB;
  auto code_off = [&](int kk) {
    return LAYOUT ? (uint32_t)(kk >> 1) * pstep + 2u * U::kCB * (uint32_t)(kk & 1)
                  : 2u * U::kCB * (uint32_t)kk;
  };
  MbCodes<FMT> bc[2][MB_NB];
  auto load_b = [&](int slot, int kk) {
#pragma unroll
    for (int nb = 0; nb < MB_NB; ++nb) bc[slot][nb].load(rb, bvo[nb], code_off(kk));
  };
  // scale windows: 16 bytes of the scale row (blocks 16 wi .. 16 wi + 15, steps
  // 8 wi .. 8 wi + 7); step 8 wi + t uses byte 2 t + q / 2. Two windows alternate.
  const int nwin = nsteps / 8;
  u32x4 sw[2][MB_NB];
  auto load_s = [&](int slot, int wi) {
    const uint32_t off = 16u * (uint32_t)(wi < nwin ? wi : nwin - 1);
#pragma unroll
    for (int nb = 0; nb < MB_NB; ++nb)
      sw[slot][nb] = __builtin_amdgcn_raw_buffer_load_b128(rb, bso[nb], off, 0);
  };

  f32x4 acc[MBK][MB_NB];
#pragma unroll
  for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
    for (int nb = 0; nb < MB_NB; ++nb) acc[mb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // lane (r, q) reads chunks 2 q and 2 q + 1 of row r = 16 mb + n (row % 8 = n % 8)
  const uint32_t rd0 = MB_ROW * n + 16u * (q ^ (n & 7));
  const uint32_t rd1 = MB_ROW * n + 16u * ((4 + q) ^ (n & 7));

  // prologue: the first scale window, steps 0 and 1
  load_s(0, 0);
  load_a(0, 0);
  load_b(0, 0);
  load_a(1, 1);
  load_b(1, 1);

  // step kk, position t = kk % 8 in scale window slot ws; d = code slot
  auto step = [&](int kk, int d, int t, int ws) {
    // this wave's loads of step kk have landed (those of kk + 1 may be in flight; at the
    // second step of a window also the next window's scales, issued by the first)
    if (t == 1)
      wait_vmcnt<mb_step_loads() + MB_NB>();
    else
      wait_vmcnt<mb_step_loads()>();
    bare_barrier();
    if (t == 0) load_s(ws ^ 1, kk / 8 + 1);
    const int nxt = kk + 2 < nsteps ? kk + 2 : nsteps - 1;
    load_a((kk + 2) % MB_STAGES, nxt);
    // the weights of the step as bf16 operands
    uint32_t b0[MB_NB][4], b1[MB_NB][4];
#pragma unroll
    for (int nb = 0; nb < MB_NB; ++nb) {
      const int bi = 2 * t + (q >> 1);  // scale byte of this lane's block in the window
      const float sc = e8m0_to_f32((sw[ws][nb][bi >> 2] >> (8 * (bi & 3))) & 0xFFu);
      bc[d][nb].convert(sc, b0[nb], b1[nb]);
    }
    load_b(d, nxt);  // the slot just converted, for step kk + 2
    const uint8_t* st = sh.a[kk % MB_STAGES];
    // the first half's products of every row block, then the second half's: the two
    // products of one accumulator are 16 products apart
#pragma unroll
    for (int mb = 0; mb < MBK; ++mb) {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(st + 16 * MB_ROW * mb + rd0);
#pragma unroll
      for (int nb = 0; nb < MB_NB; ++nb)
        acc[mb][nb] = mfma_bf16(a0, (u32x4){b0[nb][0], b0[nb][1], b0[nb][2], b0[nb][3]},
                                acc[mb][nb]);
    }
#pragma unroll
    for (int mb = 0; mb < MBK; ++mb) {
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(st + 16 * MB_ROW * mb + rd1);
#pragma unroll
      for (int nb = 0; nb < MB_NB; ++nb)
        acc[mb][nb] = mfma_bf16(a1, (u32x4){b1[nb][0], b1[nb][1], b1[nb][2], b1[nb][3]},
                                acc[mb][nb]);
    }
  };
  for (int kk = 0; kk < nsteps; kk += 16) {
#pragma unroll
    for (int t = 0; t < 8; ++t) step(kk + t, t & 1, t, 0);
    if (kk + 8 < nsteps) {
#pragma unroll
      for (int t = 0; t < 8; ++t) step(kk + 8 + t, t & 1, t, 1);
    }
  }
  // no load may still be writing this workgroup's LDS when it ends
  wait_vmcnt<0>();

#pragma unroll
  for (int nb = 0; nb < MB_NB; ++nb) {
    const int oc = 32 * w + 16 * nb + n;
    if (oc < 16 * ns) {
      const int o = grp * 128 + oc;
#pragma unroll
      for (int mb = 0; mb < MBK; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * mb + 4 * q + i;
          if (row < nrows) a.y[(size_t)sh.slot[row] * a.out + o] = acc[mb][nb][i] * sh.gate[row];
        }
      }
    }
  }
}

template <int FMT, int LAYOUT>
__device__ void mb_rows(const Mxfp4GemmArgs& a, MbShared& sh, const uint8_t* unit, int grp,
                        int nrows, int ns) {
  switch ((nrows + 31) >> 5) {
    case 1: mb_item<FMT, LAYOUT, 2>(a, sh, unit, grp, nrows, ns); break;
    case 2: mb_item<FMT, LAYOUT, 4>(a, sh, unit, grp, nrows, ns); break;
    case 3: mb_item<FMT, LAYOUT, 6>(a, sh, unit, grp, nrows, ns); break;
    default: mb_item<FMT, LAYOUT, 8>(a, sh, unit, grp, nrows, ns); break;
  }
}

template <int FMT>
__global__ __launch_bounds__(MB_THREADS, 3) void mxfp4_prefill_kernel(Mxfp4GemmArgs a) {
  __shared__ MbShared sh;
  int item, grp;
  if (!gemm_unit(a.n_items, a.groups, &item, &grp)) return;
  const int4 itd = reinterpret_cast<const int4*>(a.items)[item];
  const int e = itd.x, nrows = itd.z;
  for (int m = threadIdx.x; m < GEMM_MT; m += MB_THREADS) {
    const int slot = m < nrows ? a.pairs[itd.y + m] : 0;
    sh.slot[m] = slot;
    sh.gate[m] = (m < nrows && a.gates) ? a.gates[slot] : 1.0f;
  }
  __syncthreads();
  const int ns = min(8, a.out / 16 - grp * 8);
  const uint8_t* unit = a.units + (size_t)e * MxUnit<FMT>::unit_bytes(a.out, a.in);
  if (a.layout)
    mb_rows<FMT, 1>(a, sh, unit, grp, nrows, ns);
  else
    mb_rows<FMT, 0>(a, sh, unit, grp, nrows, ns);
}

}  // namespace

hipError_t launch_mxfp4_gemm(const Mxfp4GemmArgs& a, hipStream_t s) {
  const int blocks = gemm_grid(a.max_items, a.groups);
  if (blocks == 0) return hipSuccess;
  if (a.fmt == MX_FP8B32)
    return launch_timed(mxfp4_prefill_kernel<MX_FP8B32>, dim3(blocks), dim3(MB_THREADS), s, a);
  return launch_timed(mxfp4_prefill_kernel<MX_FP4>, dim3(blocks), dim3(MB_THREADS), s, a);
}

}  // namespace tq

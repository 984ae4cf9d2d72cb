// Prefill work-item core shared by the trellis and MXFP4 grouped GEMMs (gfx950).
//
// One workgroup (4 waves, 2 x 2 over a 128 x 128 output tile) multiplies up to 128 routed
// rows of one expert by one group of up to 128 output channels over the whole K range, in
// steps of 32 inputs:
//   - a B producer (format-specific) decodes the step's 32 x 128 weights into bf16, each
//     thread one run of 16 inputs of one output channel, stored in natural input order;
//   - each thread gathers 16 activations of one routed row into the A tile;
//   - each wave runs its 4 x 4 block of 16x16x32 bf16 matrix-core operations.
// Two LDS buffers alternate, so the next step is produced while this one multiplies. Each
// output is written once by the workgroup owning its row.
#pragma once

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

constexpr int GEMM_THREADS = 256;
constexpr int GEMM_KS = 32;          // inputs per step
constexpr int GEMM_LDS_STRIDE = 40;  // bf16 per LDS row (32 + 8 padding against bank conflicts)

struct GemmShared {
  uint16_t a[2][GEMM_MT * GEMM_LDS_STRIDE];
  uint16_t b[2][128 * GEMM_LDS_STRIDE];
  int slot[GEMM_MT];
};

struct GemmItem {
  const uint16_t* x;
  const float* gates;
  const uint16_t* scales;  // fp16 per output channel of this expert, or null
  float* y;
  int in, out, topk, grp, nrows, ns;
};

// Load slot indices of the item's rows into LDS (all threads; ends with a barrier).
__device__ inline void gemm_load_slots(GemmShared& sh, const int32_t* pairs, int row0,
                                       int nrows) {
  for (int m = threadIdx.x; m < GEMM_MT; m += GEMM_THREADS)
    sh.slot[m] = m < nrows ? pairs[row0 + m] : 0;
  __syncthreads();
}

// Producer interface: void operator()(int kk, int* o, int* h, uint32_t nat[8]) gives the
// thread's B run for step kk: output channel o (0..127, within the group), inputs
// 32 kk + 16 h .. + 15, as 8 dwords of bf16 pairs in natural order (zeros if unused).
template <class Producer>
__device__ void gemm_item(const GemmItem& it, GemmShared& sh, Producer& produce_b) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  const int wm = w >> 1, wn = w & 1;
  const int nsteps = it.in / GEMM_KS;
  const int a_m = tid >> 1, a_h = tid & 1;
  const bool a_valid = a_m < it.nrows;
  const uint16_t* a_src =
      it.x + (size_t)(a_valid ? sh.slot[a_m] / it.topk : 0) * it.in + 16 * a_h;

  auto produce = [&](int kk, int buf) {
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (a_valid) {
      const uint4* src = reinterpret_cast<const uint4*>(a_src + kk * GEMM_KS);
      v0 = src[0];
      v1 = src[1];
    }
    uint4* da = reinterpret_cast<uint4*>(&sh.a[buf][a_m * GEMM_LDS_STRIDE + 16 * a_h]);
    da[0] = v0;
    da[1] = v1;
    int o, h;
    uint32_t nat[8];
    produce_b(kk, &o, &h, nat);
    uint4* db = reinterpret_cast<uint4*>(&sh.b[buf][o * GEMM_LDS_STRIDE + 16 * h]);
    db[0] = make_uint4(nat[0], nat[1], nat[2], nat[3]);
    db[1] = make_uint4(nat[4], nat[5], nat[6], nat[7]);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  int mblocks = (it.nrows - 64 * wm + 15) / 16;
  mblocks = mblocks < 0 ? 0 : (mblocks > 4 ? 4 : mblocks);
  int nblocks = it.ns - 4 * wn;
  nblocks = nblocks < 0 ? 0 : (nblocks > 4 ? 4 : nblocks);

  produce(0, 0);
  __syncthreads();
  for (int kk = 0; kk < nsteps; ++kk) {
    const int buf = kk & 1;
    if (kk + 1 < nsteps) produce(kk + 1, buf ^ 1);
    u32x4 bop[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      bop[nb] = *reinterpret_cast<const u32x4*>(
          &sh.b[buf][(64 * wn + 16 * nb + n) * GEMM_LDS_STRIDE + 8 * g]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb < mblocks) {
        const u32x4 aop = *reinterpret_cast<const u32x4*>(
            &sh.a[buf][(64 * wm + 16 * mb + n) * GEMM_LDS_STRIDE + 8 * g]);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          if (nb < nblocks) acc[mb][nb] = mfma_bf16(aop, bop[nb], acc[mb][nb]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      if (mb < mblocks && nb < nblocks) {
        const int o = it.grp * 128 + 64 * wn + 16 * nb + n;
        const float sc = it.scales ? f16_bits_to_f32(it.scales[o]) : 1.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 64 * wm + 16 * mb + 4 * g + i;
          if (row < it.nrows) {
            const int slot = sh.slot[row];
            float v = acc[mb][nb][i] * sc;
            if (it.gates) v = v * it.gates[slot];
            it.y[(size_t)slot * it.out + o] = v;
          }
        }
      }
    }
  }
}

// NaN in every output of the item (bad unit descriptor).
__device__ inline void gemm_item_nan(const GemmItem& it, GemmShared& sh) {
  for (int v = threadIdx.x; v < it.nrows * it.ns * 16; v += GEMM_THREADS) {
    const int m = v / (it.ns * 16), o = it.grp * 128 + v % (it.ns * 16);
    it.y[(size_t)sh.slot[m] * it.out + o] = __builtin_nanf("");
  }
}

}  // namespace tq

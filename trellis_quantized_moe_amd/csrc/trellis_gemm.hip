// Prefill grouped GEMM over trellis-coded experts (gfx950).
//
// A work item is up to 128 routed rows of one expert times one group of up to 128 output
// channels, over the whole input range, in steps of 64 inputs (four 16-input tile columns).
// One workgroup of two waves runs an item; wave w owns output channels 64 w .. 64 w + 63
// (tile strips 4 w .. 4 w + 3) for all 128 rows, so no weight is decoded twice and no
// weight passes through LDS:
//   - weights: lane (g, n) of a wave (g = lane / 16, n = lane % 16) decodes, for each of
//     its four strips, the whole tile column g of the step for channel n: 16 weights as
//     eight f16 byte-sum pairs (trellis_decode.h). Pairs 0..3 are its operand of the
//     step's first 16x16x32 matrix-core product, pairs 4..7 of the second; the activation
//     operand is laid out to match, so the k order inside a product is a permutation of
//     the inputs and the sum is the same.
//   - activations: the prepared f16 rows (the same pair layout) are gathered straight
//     from global memory into LDS by buffer loads that write LDS (no registers), into a
//     ring of three 16 KB stages, two steps ahead. A stage holds 128 rows x 128 bytes in
//     16-byte chunks, chunk c of row r stored at position c ^ ((r / 2) % 8) of the row,
//     so the operand reads of one 16-lane group hit 16 different chunk columns.
//   - codes are loaded two steps ahead into registers.
// Each step: wait for this wave's loads of the step, one barrier (the partner wave's half
// of the stage has landed and both waves are done with the stage about to be refilled),
// start the loads of step + 2, decode, then 8 x 4 x 2 products. The epilogue scales by
// 2^24, removes 255 * sum(x) per token (the byte-sum offset), applies the channel scale and
// the gate, and writes each output once.
#include "gemm_core.h"
#include "trellis_decode.h"

#include <type_traits>

namespace tq {

namespace {

constexpr int TG_THREADS = 128;
constexpr int TG_STEP = 64;                       // inputs per step
constexpr int TG_ROW_BYTES = TG_STEP * 2;         // one row of a stage: 128 bytes
constexpr int TG_STAGE = GEMM_MT * TG_ROW_BYTES;  // 16 KB
constexpr int TG_STAGES = 3;

struct TgShared {
  alignas(16) uint8_t a[TG_STAGES][TG_STAGE];
  int slot[GEMM_MT];
  float rs[GEMM_MT];    // 255 * sum of the row's token activations
  float gate[GEMM_MT];  // the slot's gate, or 1
};

typedef __attribute__((address_space(3))) void* LdsPtr;

// s_waitcnt with only the vector-memory count limited (gfx9 encoding: vmcnt in bits 3:0
// and 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier with no memory fence. The loads that write LDS count on the vector
// memory counter, so an LDS fence would wait for all of them, including the ones meant to
// stay in flight; the waits are explicit instead (wait_vmcnt before the barrier). The empty
// asm statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int K>
struct ColWords {
  uint32_t w[K == 2 ? 1 : 2];
};

// Vector-memory instructions per step and wave: 8 activation loads and the code loads.
template <int K>
constexpr int step_loads() {
  return 8 + 4 * (K == 3 ? 2 : 1);
}

template <int K>
__device__ __forceinline__ void tg_item(const TrellisGemmArgs& a, TgShared& sh,
                                        const uint32_t* unit, int e, int grp, int nrows,
                                        int ns) {
  constexpr int TW = 8 * K;  // words per tile
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nsteps = a.in / TG_STEP;  // a multiple of 4
  const int n_ti = a.in / 16;

  // activation loads: instruction j of wave w fills rows 64 w + 8 j .. + 7 of a stage; lane l
  // writes LDS chunk l of the instruction's 1 KB, i.e. row 64 w + 8 j + l / 8, position l % 8,
  // which holds chunk (l % 8) ^ ((row / 2) % 8) of the row's 128 bytes. Rows past the item
  // load from beyond the buffer's end (x_bytes < 2^31) and read zeros.
  const GemmRsrc ra = gemm_rsrc(a.xp, a.x_bytes);
  uint32_t dvo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 64 * w + 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    dvo[j] = r < nrows ? 2u * (uint32_t)((sh.slot[r] / a.topk) * a.in) + 16u * c : 0x80000000u;
  }
  auto load_a = [&](int kk) {
    uint8_t* st = sh.a[kk % TG_STAGES] + 64 * w * TG_ROW_BYTES;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LdsPtr)(st + 8 * j * TG_ROW_BYTES), 16,
                                               dvo[j], (uint32_t)(TG_ROW_BYTES * kk), 0, 0);
  };

  // code loads: strip 8 grp + 4 w + nb (strips past the group read its last strip; their
  // outputs are never stored), tile column 4 kk + g, channel n of the strip
  const GemmRsrc rc = gemm_rsrc(unit, (uint32_t)((size_t)a.out * a.in * K / 8));
  uint32_t cvo[2] = {0, 0};
  uint32_t sel3 = 0;
  if constexpr (K == 2) {
    cvo[0] = 4u * (g * TW + n);
  } else if constexpr (K == 4) {
    cvo[0] = 4u * (g * TW + 2 * n);
  } else {
    int w0, w1;
    k3_column_words(n, &w0, &w1, &sel3);
    cvo[0] = 4u * (g * TW + w0);
    cvo[1] = 4u * (g * TW + w1);
  }
  uint32_t strip_off[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int s = 4 * w + nb;
    strip_off[nb] = 4u * (uint32_t)((8 * grp + (s < ns ? s : ns - 1)) * n_ti * TW);
  }
  ColWords<K> code[2][4];
  auto load_codes = [&](int slot, int kk) {
    const uint32_t so = 4u * (uint32_t)(4 * kk * TW);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const uint32_t o = strip_off[nb] + so;
      if constexpr (K == 2) {
        code[slot][nb].w[0] = __builtin_amdgcn_raw_buffer_load_b32(rc, cvo[0], o, 0);
      } else if constexpr (K == 4) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, cvo[0], o, 0);
        code[slot][nb].w[0] = v.x;
        code[slot][nb].w[1] = v.y;
      } else {
        code[slot][nb].w[0] = __builtin_amdgcn_raw_buffer_load_b32(rc, cvo[0], o, 0);
        code[slot][nb].w[1] = __builtin_amdgcn_raw_buffer_load_b32(rc, cvo[1], o, 0);
      }
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int mblocks = (nrows + 15) >> 4;
  // operand reads of lane (g, n): row 16 mb + n, chunks 2 g and 2 g + 1 of the step
  const uint32_t rd0 = 128u * n + 16u * ((2 * g) ^ (n >> 1));
  const uint32_t rd1 = 128u * n + 16u * ((2 * g + 1) ^ (n >> 1));

  // B0 / B1: operand registers of the step's first / second product for each strip (pairs
  // 0..3 / 4..7 of the lane's tile column). For K = 2, 3 the halves are decoded apart, so
  // that each half is decoded while the matrix cores run the other half's products.
  uint32_t B0[4][4], B1[4][4];
  auto dec_half = [&](int slot, int h, uint32_t Bh[4][4]) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const ColWords<K>& c = code[slot][nb];
      uint32_t M[4];
      if constexpr (K == 2)
        half_mpairs_k2(c.w[0], row_next(c.w[0]), h, M);
      else if constexpr (K == 3)
        half_mpairs_k3(c.w[0], c.w[1], row_next(c.w[0]), sel3, h, M);
#pragma unroll
      for (int r = 0; r < 4; ++r) Bh[nb][r] = byte_sum_pair(M[r]);
    }
  };
  auto dec_full = [&](int slot) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const ColWords<K>& c = code[slot][nb];
      uint32_t M[8], V[8];
      if constexpr (K == 2)
        col_mpairs_k2(c.w[0], row_next(c.w[0]), M);
      else if constexpr (K == 4)
        col_mpairs_k4(c.w[0], c.w[1], row_next(c.w[0]), M);
      else
        col_mpairs_k3(c.w[0], c.w[1], row_next(c.w[0]), sel3, M);
      byte_sums<K>(M, V);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        B0[nb][r] = V[r];
        B1[nb][r] = V[4 + r];
      }
    }
  };
  auto products = [&](const uint8_t* st, uint32_t rd, const uint32_t Bh[4][4], auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      if (FULL || mb < mblocks) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(st + 2048 * mb + rd);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = mfma_f16(av, (u32x4){Bh[nb][0], Bh[nb][1], Bh[nb][2], Bh[nb][3]},
                                 acc[mb][nb]);
      }
    }
  };

  // prologue: steps 0 and 1 (every step issues its loads in the order activations, codes)
  load_a(0);
  load_codes(0, 0);
  load_a(1);
  load_codes(1, 1);
  if constexpr (K == 4)
    dec_full(0);
  else
    dec_half(0, 0, B0);

  auto run = [&](auto full_tag) {
    for (int kk = 0; kk < nsteps; kk += 2) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int step = kk + d;
        // this wave's loads of `step` have landed (those of step + 1 may be in flight)
        wait_vmcnt<step_loads<K>()>();
        bare_barrier();
        // refill the stage read two steps ago (every load is issued, clamped to the last
        // step, so the wait counts above stay exact)
        const int nxt = step + 2 < nsteps ? step + 2 : nsteps - 1;
        load_a(nxt);
        const uint8_t* st = sh.a[step % TG_STAGES];
        if constexpr (K == 4) {
          products(st, rd0, B0, full_tag);
          products(st, rd1, B1, full_tag);
          load_codes(d, nxt);
          dec_full(d ^ 1);  // the next step (past the last: unused)
        } else {
          // each half's products overlap the decoding of the other half; the scheduling
          // barrier keeps the next step's first half from being decoded while this step's
          // first-half products still read B0
          dec_half(d, 1, B1);
          products(st, rd0, B0, full_tag);
          load_codes(d, nxt);
          __builtin_amdgcn_sched_barrier(0);
          dec_half(d ^ 1, 0, B0);  // the next step's first half (past the last: unused)
          products(st, rd1, B1, full_tag);
        }
      }
    }
  };
  if (mblocks == 8)
    run(std::integral_constant<bool, true>());
  else
    run(std::integral_constant<bool, false>());
  // no load may still be writing this workgroup's LDS when it ends
  wait_vmcnt<0>();

#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    if (4 * w + nb < ns) {
      const int o = grp * 128 + 64 * w + 16 * nb + n;
      const float sc = f16_bits_to_f32(a.scales[(size_t)e * a.out + o]);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * mb + 4 * g + i;
          if (row < nrows) {
            float v = acc[mb][nb][i] * BYTE_SUM_SCALE - sh.rs[row];
            v = v * sc;
            v = v * sh.gate[row];
            a.y[(size_t)sh.slot[row] * a.out + o] = v;
          }
        }
      }
    }
  }
}

// One kernel for every width: the decoder is chosen per item from the expert's width byte
// (the register budget is that of the widest decoder).
__global__ __launch_bounds__(TG_THREADS, 2) void trellis_gemm_kernel(TrellisGemmArgs a) {
  __shared__ TgShared sh;
  int item, grp;
  if (!gemm_unit(a.n_items, a.groups, &item, &grp)) return;
  const int4 itd = reinterpret_cast<const int4*>(a.items)[item];
  const int e = itd.x;
  const int nrows = itd.z;
  const int K = a.bits[e];
  const int64_t off = a.code_off[e];
  const int ns = min(8, a.out / 16 - grp * 8);
  for (int m = threadIdx.x; m < GEMM_MT; m += TG_THREADS) {
    int slot = 0;
    float rs = 0.0f, gt = 1.0f;
    if (m < nrows) {
      slot = a.pairs[itd.y + m];
      rs = BYTE_SUM_OFFSET * a.rowsum[slot / a.topk];
      if (a.gates) gt = a.gates[slot];
    }
    sh.slot[m] = slot;
    sh.rs[m] = rs;
    sh.gate[m] = gt;
  }
  __syncthreads();
  const uint32_t* unit = a.codes + off / 4;
  if (K == 2 && !(off & 15)) {
    tg_item<2>(a, sh, unit, e, grp, nrows, ns);
  } else if (K == 3 && !(off & 15)) {
    tg_item<3>(a, sh, unit, e, grp, nrows, ns);
  } else if (K == 4 && !(off & 15)) {
    tg_item<4>(a, sh, unit, e, grp, nrows, ns);
  } else {
    for (int v = threadIdx.x; v < nrows * ns * 16; v += TG_THREADS) {
      const int m = v / (ns * 16), o = grp * 128 + v % (ns * 16);
      a.y[(size_t)sh.slot[m] * a.out + o] = __builtin_nanf("");
    }
    if (threadIdx.x == 0) set_status(a.status, STATUS_BAD_UNIT);
  }
}

}  // namespace

hipError_t launch_trellis_gemm(const TrellisGemmArgs& a, hipStream_t s) {
  const int blocks = gemm_grid(a.max_items, a.groups);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(trellis_gemm_kernel, dim3(blocks), dim3(TG_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq

// Prefill grouped GEMM over trellis-coded experts (gfx950).
//
// A work item is up to 128 routed rows of one expert times one group of up to 128 output
// channels, over the whole input range, in steps of 64 inputs (four 16-input tile columns).
// One workgroup of four waves runs an item; wave w owns output channels 32 w .. 32 w + 31
// (tile strips 2 w, 2 w + 1) for all 128 rows, so no weight is decoded twice and no weight
// passes through LDS:
//   - weights: lane (g, n) of a wave (g = lane / 16, n = lane % 16) decodes, for each of
//     its two strips, the whole tile column g of the step for channel n: 16 weights as
//     eight f16 byte-sum pairs (trellis_decode.h). Pairs 0..3 are its operand of the
//     step's first 16x16x32 matrix-core product, pairs 4..7 of the second; the activation
//     operand is laid out to match, so the k order inside a product is a permutation of
//     the inputs and the sum is the same.
//   - activations: the prepared f16 rows (the same pair layout) are gathered straight
//     from global memory into LDS by buffer loads that write LDS (no registers), into a
//     ring of three 16 KB stages, two steps ahead; each wave loads 32 of the 128 rows. A
//     stage holds 128 rows x 128 bytes in 16-byte chunks; lane group g of the operand reads
//     needs chunks 2 g and 2 g + 1 of a row, stored at positions g ^ (r % 8) and
//     (4 + g) ^ (r % 8) of row r (chunk 2 p at p, 2 p + 1 at 4 + p, then the xor), so the 8
//     lanes the LDS serves together hit 8 different chunk columns.
//   - codes are loaded two steps ahead into registers (one load per strip and step).
// Three items fit on a compute unit (50 KB of LDS each, 142 registers per lane), so every
// item of a prefill chunk is resident at once and each SIMD runs three waves, whose decode
// and matrix-core work overlap. The loads a step needs are few: the cost of a load is set by
// its lanes, not its bytes.
// Each step: wait for this wave's loads of the step, one barrier (the other waves' parts
// of the stage have landed and every wave is done with the stage about to be refilled),
// start the loads of step + 2, decode, then 8 x 2 x 2 products. The epilogue scales by
// 2^24, removes 255 * sum(x) per token (the byte-sum offset), applies the channel scale,
// the gate and the token's 2^-s (the prep's power-of-two scale), and writes each output
// once.
#include "gemm_core.h"
#include "trellis_decode.h"

#include <type_traits>

namespace tq {

namespace {

constexpr int TG_WAVES = 4;                    // waves per item
constexpr int TG_THREADS = 64 * TG_WAVES;
constexpr int TG_NS = 8 / TG_WAVES;            // 16-channel strips per wave
constexpr int TG_AROWS = GEMM_MT / TG_WAVES;   // activation rows each wave loads per step
constexpr int TG_STEP = 64;                       // inputs per step
constexpr int TG_ROW_BYTES = TG_STEP * 2;         // one row of a stage: 128 bytes
constexpr int TG_STAGE = GEMM_MT * TG_ROW_BYTES;  // 16 KB
constexpr int TG_STAGES = 3;

struct TgShared {
  alignas(16) uint8_t a[TG_STAGES][TG_STAGE];
  int slot[GEMM_MT];
  float rs[GEMM_MT];    // 255 * sum of the row's token activations (scaled by 2^s)
  float gate[GEMM_MT];  // the slot's gate (or 1) times the token's 2^-s
};

template <int K>
struct ColWords {
  uint32_t w[K == 2 ? 1 : 2];
};

// Vector-memory instructions per step and wave: the activation loads (rows / 8 of them)
// and one code load per strip.
template <int K>
constexpr int step_loads() {
  return TG_AROWS / 8 + TG_NS;
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

  // activation loads: instruction j of wave w fills rows TG_AROWS w + 8 j .. + 7 of a stage;
  // lane l writes LDS chunk l of the instruction's 1 KB, i.e. row TG_AROWS w + 8 j + l / 8,
  // position l % 8, which holds chunk 2 (x % 4) + x / 4 of the row's 128 bytes, x =
  // (l % 8) ^ (row % 8). Rows past the item load from beyond the buffer's end
  // (x_bytes < 2^31) and read zeros.
  const GemmRsrc ra = gemm_rsrc(a.xp, a.x_bytes);
  uint32_t dvo[TG_AROWS / 8];
#pragma unroll
  for (int j = 0; j < TG_AROWS / 8; ++j) {
    const int r = TG_AROWS * w + 8 * j + (lane >> 3);
    const int x = (lane & 7) ^ (r & 7);
    const int c = 2 * (x & 3) + (x >> 2);
    dvo[j] = r < nrows ? 2u * (uint32_t)((sh.slot[r] / a.topk) * a.in) + 16u * c : 0x80000000u;
  }
  auto load_a = [&](int kk) {
    uint8_t* st = sh.a[kk % TG_STAGES] + TG_AROWS * w * TG_ROW_BYTES;
#pragma unroll
    for (int j = 0; j < TG_AROWS / 8; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LdsPtr)(st + 8 * j * TG_ROW_BYTES), 16,
                                               dvo[j], (uint32_t)(TG_ROW_BYTES * kk), 0, 0);
  };

  // code loads: strip 8 grp + TG_NS w + nb (strips past the group read its last strip; their
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
  // run (strip 8 grp + s, step kk) at strip_off[nb] + step_off(kk) bytes (run_word)
  const int S = n_ti / 4, nst = a.out / 16;
  const uint32_t base = 4u * run_word(a.layout, 8 * grp, 0, S, nst, TW);
  auto step_off = [&](int kk) { return 4u * run_word(a.layout, 8 * grp, kk, S, nst, TW) - base; };
  uint32_t strip_off[TG_NS];
#pragma unroll
  for (int nb = 0; nb < TG_NS; ++nb) {
    const int s = TG_NS * w + nb;
    strip_off[nb] = 4u * run_word(a.layout, 8 * grp + (s < ns ? s : ns - 1), 0, S, nst, TW);
  }
  ColWords<K> code[2][TG_NS];
  auto load_codes = [&](int slot, int kk) {
    const uint32_t so = step_off(kk);
#pragma unroll
    for (int nb = 0; nb < TG_NS; ++nb) {
      const uint32_t o = strip_off[nb] + so;
      if constexpr (K == 2) {
        code[slot][nb].w[0] = __builtin_amdgcn_raw_buffer_load_b32(rc, cvo[0], o, 0);
      } else if constexpr (K == 4) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, cvo[0], o, 0);
        code[slot][nb].w[0] = v.x;
        code[slot][nb].w[1] = v.y;
      } else {  // words p and p + 1 of k3_column_words, adjacent: one 8-byte load
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, cvo[0], o, 0);
        code[slot][nb].w[0] = v.x;
        code[slot][nb].w[1] = v.y;
      }
    }
  };

  f32x4 acc[8][TG_NS];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < TG_NS; ++nb) acc[mb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // operand reads of lane (g, n): row 16 mb + n, chunks 2 g and 2 g + 1 of the step
  const uint32_t rd0 = 128u * n + 16u * (g ^ (n & 7));
  const uint32_t rd1 = 128u * n + 16u * ((4 + g) ^ (n & 7));

  // B0 / B1: operand registers of the step's first / second product for each strip (pairs
  // 0..3 / 4..7 of the lane's tile column). For K = 2, 3 the halves are decoded apart, so
  // that each half is decoded while the matrix cores run the other half's products.
  uint32_t B0[TG_NS][4], B1[TG_NS][4];
  auto dec_half = [&](int slot, int h, uint32_t Bh[TG_NS][4]) {
    if constexpr (K != 4) {
#pragma unroll
      for (int nb = 0; nb < TG_NS; ++nb) {
        const ColWords<K>& c = code[slot][nb];
        prefill_half<K>(c.w[0], c.w[K == 2 ? 0 : 1], row_next(c.w[0]), sel3, h, Bh[nb]);
      }
    }
  };
  auto dec_full = [&](int slot) {
#pragma unroll
    for (int nb = 0; nb < TG_NS; ++nb) {
      const ColWords<K>& c = code[slot][nb];
      prefill_full<K>(c.w[0], c.w[K == 2 ? 0 : 1], row_next(c.w[0]), sel3, B0[nb], B1[nb]);
    }
  };
  // the products of a step over the first MBK row blocks (a constant: one straight block in
  // which the operand reads run ahead of the matrix-core work; rows past the item are zeros)
  auto products = [&](const uint8_t* st, uint32_t rd, const uint32_t Bh[TG_NS][4], auto mbk) {
    constexpr int MBK = decltype(mbk)::value;
#pragma unroll
    for (int mb = 0; mb < MBK; ++mb) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(st + 2048 * mb + rd);
#pragma unroll
      for (int nb = 0; nb < TG_NS; ++nb)
        acc[mb][nb] = mfma_f16(av, (u32x4){Bh[nb][0], Bh[nb][1], Bh[nb][2], Bh[nb][3]},
                               acc[mb][nb]);
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

  auto run = [&](auto mbk) {
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
          products(st, rd0, B0, mbk);
          products(st, rd1, B1, mbk);
          load_codes(d, nxt);
          dec_full(d ^ 1);  // the next step (past the last: unused)
        } else {
          // each half's products overlap the decoding of the other half; the scheduling
          // barrier keeps the next step's first half from being decoded while this step's
          // first-half products still read B0
          dec_half(d, 1, B1);
          products(st, rd0, B0, mbk);
          load_codes(d, nxt);
          __builtin_amdgcn_sched_barrier(0);
          dec_half(d ^ 1, 0, B0);  // the next step's first half (past the last: unused)
          products(st, rd1, B1, mbk);
        }
      }
    }
  };
  // the item's rows rounded up to an even count of row blocks
  switch ((nrows + 31) >> 5) {
    case 1: run(std::integral_constant<int, 2>()); break;
    case 2: run(std::integral_constant<int, 4>()); break;
    case 3: run(std::integral_constant<int, 6>()); break;
    default: run(std::integral_constant<int, 8>()); break;
  }
  // no load may still be writing this workgroup's LDS when it ends
  wait_vmcnt<0>();

#pragma unroll
  for (int nb = 0; nb < TG_NS; ++nb) {
    if (TG_NS * w + nb < ns) {
      const int o = grp * 128 + 16 * (TG_NS * w + nb) + n;
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
__global__ __launch_bounds__(TG_THREADS, 3) void trellis_gemm_kernel(TrellisGemmArgs a) {
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
      const float2 rw = a.rowsum[slot / a.topk];
      rs = BYTE_SUM_OFFSET * rw.x;
      gt = rw.y;  // a power of two: the product below is exact
      if (a.gates) gt = a.gates[slot] * gt;
    }
    sh.slot[m] = slot;
    sh.rs[m] = rs;
    sh.gate[m] = gt;
  }
  __syncthreads();
  const uint32_t* unit = a.codes + off / 4;
  // the unit must be 16-byte aligned and lie inside the code buffer
  const bool inside = !(off & 15) && off >= 0 &&
                      off <= a.codes_bytes - (int64_t)a.out * a.in / 8 * (K >= 2 && K <= 4 ? K : 0);
  if (K == 2 && inside) {
    tg_item<2>(a, sh, unit, e, grp, nrows, ns);
  } else if (K == 3 && inside) {
    tg_item<3>(a, sh, unit, e, grp, nrows, ns);
  } else if (K == 4 && inside) {
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
  return launch_timed(trellis_gemm_kernel, dim3(blocks), dim3(TG_THREADS), s, a);
}

}  // namespace tq

// Decode-batch plan and activation prep, one launch (see gemv_plan.h for the scheme).
//
// Block 0 plans. It counts the slots of every expert with shared-memory atomics, which
// also gives each slot its position in its expert's list. Positions within one expert
// therefore follow arrival order, but every output is computed by arithmetic that does not
// depend on its row position, so the results are the same bits whatever the order. A
// block-wide scan then gives list starts, the active experts in ascending id order and,
// per cost class, how many active experts precede each one. The split (pieces per group
// for each cost class) is the smallest feasible per-wave cost bound, found by testing all
// candidates at once. Last come the slot lists, the per-slot records and every wave's
// piece (each active expert's thread writes its own waves').
//
// Blocks 1..T convert token t = block - 1 of x~ (bf16, rotated first when asked) to the
// int8 operands of the decode GEMV (see prep_block). The prefill GEMM's f16 operands come
// from the same conversion code, launched on its own (launch_activation_prep).
#include "gemv_plan.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr int PLAN_R = 4;                            // slots per thread kept in registers
constexpr int PLAN_PER = PLAN_MAX_E / PLAN_THREADS;  // experts per thread in the scan
constexpr int PLAN_WAVES = PLAN_THREADS / 64;

// Inclusive scan of v over the 64 lanes of a wave: row shifts 1, 2, 4, 8 and the row
// broadcasts 15 and 31 (DPP, no LDS round trip).
__device__ __forceinline__ int wave_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Exclusive block scan of NV ints over PLAN_THREADS threads, in place; tot = totals.
template <int NV>
__device__ void block_scan(int (&x)[NV], int (&tot)[NV]) {
  __shared__ int part[NV][PLAN_WAVES];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int in[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) in[v] = wave_scan(x[v]);
  if (lane == 63) {
#pragma unroll
    for (int v = 0; v < NV; ++v) part[v][w] = in[v];
  }
  lds_barrier();
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    int b = 0, t = 0;
#pragma unroll
    for (int u = 0; u < PLAN_WAVES; ++u) {
      const int p = part[v][u];
      if (u < w) b += p;
      t += p;
    }
    tot[v] = t;
    x[v] = b + in[v] - x[v];
  }
}

// n / d for 0 <= n < 2^22 and d > 0, given rd = 1 / d in fp32: the product is within one of
// the quotient there (its relative error is a few ulp, the quotient below 2^22), and one
// remainder test corrects it. A handful of instructions in place of the integer divide.
__device__ __forceinline__ int small_div(int n, int d, float rd) {
  const int q = (int)((float)n * rd);
  const int r = n - q * d;
  return q + (r >= d) - (r < 0);
}

// Pieces per group for a step cost k under the per-wave cost bound T (T >= k): the steps
// S split into pieces of at most per = floor(T / k) steps, ceil(S / per) =
// floor((S + per - 1) / per), by small_div with the hardware reciprocal (its error is an
// ulp or two, and S + per - 1 < 2^22 here: S <= 2^15).
__device__ __forceinline__ int pieces_for(int S, int T, int k) {
  const int per = T / k;
  return small_div(S + per - 1, per, __builtin_amdgcn_rcpf((float)per));
}

// The smallest v over the wave's 64 lanes (all active): DPP within each row of 16 lanes,
// then the four rows' results read out.
__device__ __forceinline__ int wave_min(int v) {
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));   // quad_perm [1, 0, 3, 2]
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));   // quad_perm [2, 3, 0, 1]
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true));  // row_half_mirror
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true));  // row_mirror
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// The plan is one block of PLAN_THREADS threads; each phase gives a thread about one slot
// or one expert (ceil(E / PLAN_THREADS) of them), so that no thread runs a long chain of
// dependent steps.
template <bool TRELLIS>
__device__ void plan_block(const PlanArgs& a) {
  __shared__ int s_start[PLAN_MAX_E];   // slot counts, then list starts
  __shared__ int s_aidx[PLAN_MAX_E];    // active index, or SLOT_EMPTY / SLOT_BAD_UNIT
  __shared__ uint8_t s_ka[PLAN_MAX_E];  // step cost by active index
  __shared__ int4 s_big[PLAN_MAX_BIG];  // experts whose pieces the whole block writes
  __shared__ int s_nbig;
  __shared__ int s_T;
  __shared__ uint32_t s_status;
  const int tid = threadIdx.x;
  const int N = a.N, E = a.E, S = a.S, groups = a.groups;
  const bool in_regs = N <= PLAN_THREADS * PLAN_R;
  const int rsh = 31 - __builtin_clz(a.R);  // R is a power of two: chunks by a shift
  const int per = (E + PLAN_THREADS - 1) / PLAN_THREADS;  // experts per thread, <= PLAN_PER

  // all route and descriptor loads are issued before any is used (indices clamped; slots
  // past N and experts past E are skipped where used)
  int id[PLAN_R], rk[PLAN_R];
  if (in_regs) {
#pragma unroll
    for (int j = 0; j < PLAN_R; ++j) id[j] = a.ids[min(tid + PLAN_THREADS * j, N - 1)];
  }
  const int e0 = tid * per;  // this thread's experts e0 .. e0 + per - 1
  int kk[PLAN_PER];
  int64_t off[PLAN_PER];
  if constexpr (TRELLIS) {
#pragma unroll
    for (int j = 0; j < PLAN_PER; ++j) {
      const int e = min(e0 + j, E - 1);
      kk[j] = a.bits[e];
      off[j] = a.code_off[e];
    }
    // a unit is good when its width is 2, 3 or 4 and it lies, 16-byte aligned, inside codes
    const int64_t ub = a.unit_bytes;  // a unit's bytes per bit of width: out * in / 8
#pragma unroll
    for (int j = 0; j < PLAN_PER; ++j) {
      const bool good = kk[j] >= 2 && kk[j] <= 4 && (off[j] & 15) == 0 && off[j] >= 0 &&
                        off[j] <= a.codes_bytes - ub * kk[j];
      kk[j] = good ? kk[j] : 0;
    }
  } else {
#pragma unroll
    for (int j = 0; j < PLAN_PER; ++j) {
      kk[j] = 1;
      off[j] = (int64_t)(e0 + j) * a.unit_bytes;
    }
  }
  auto mine = [&](int j) { return j < per && e0 + j < E; };
#pragma unroll
  for (int j = 0; j < PLAN_PER; ++j)
    if (mine(j)) s_start[e0 + j] = 0;
  if (tid == 0) {
    s_status = 0;
    s_nbig = 0;
    s_T = 0x7FFFFFFF;
  }
  lds_barrier();

  // counts; a slot's position in its expert's list is the count before its own increment
  uint32_t bad = 0;
  if (in_regs) {
#pragma unroll
    for (int j = 0; j < PLAN_R; ++j) {
      rk[j] = 0;
      if (PLAN_THREADS * j < N) {  // uniform
        if (tid + PLAN_THREADS * j < N && id[j] >= 0 && id[j] < E)
          rk[j] = atomicAdd(&s_start[id[j]], 1);
      }
    }
  } else {
    for (int i = tid; i < N; i += PLAN_THREADS) {
      const int v = a.ids[i];
      if (v >= 0 && v < E) a.rank[i] = atomicAdd(&s_start[v], 1);
    }
  }
  lds_barrier();

  // scan over experts: list starts, the active experts before each (its active index) and,
  // per step cost 1..4, the chunks of R slots of the active experts before each (chunks of
  // cost 1 and 2 share one int, 3 and 4 another: 16 bits each, as the host keeps
  // E + N / R <= GEMV_MAX_G)
  int cnt[PLAN_PER];
  int sv[4] = {0, 0, 0, 0};  // slots; chunks of cost 1 | 2 << 16; of cost 3 | 4 << 16; active
#pragma unroll
  for (int j = 0; j < PLAN_PER; ++j) {
    cnt[j] = mine(j) ? s_start[e0 + j] : 0;
    sv[0] += cnt[j];
    if (cnt[j] > 0 && kk[j] > 0) {
      const int nch = (cnt[j] + a.R - 1) >> rsh;
      sv[kk[j] >= 3 ? 2 : 1] += (kk[j] & 1) ? nch : (nch << 16);
      sv[3] += 1;
    }
  }
  int tot4[4];
  block_scan<4>(sv, tot4);
  const int tot[5] = {0, tot4[1] & 0xFFFF, tot4[1] >> 16, tot4[2] & 0xFFFF, tot4[2] >> 16};
  const int n_act = tot4[3];
  const int n_chunks = tot[1] + tot[2] + tot[3] + tot[4];
  const int kmax = tot[4] ? 4 : tot[3] ? 3 : tot[2] ? 2 : 1;

  // the split: the smallest cost bound T in [4 kmax, S kmax] whose waves fit the target;
  // T = S kmax (one piece per group and chunk) always does
  const int64_t target = max((int64_t)a.G, (int64_t)groups * n_chunks);
  for (int T0 = 4 * kmax; T0 <= S * kmax; T0 += PLAN_THREADS) {  // uniform
    const int T = T0 + tid;
    int best = 0x7FFFFFFF;
    if (T <= S * kmax) {
      int64_t waves = 0;
#pragma unroll
      for (int k = 1; k <= 4; ++k)
        if (tot[k]) waves += (int64_t)tot[k] * pieces_for(S, T, k);
      if (waves * groups <= target) best = T;
    }
    best = wave_min(best);
    if ((tid & 63) == 0 && best != 0x7FFFFFFF) atomicMin(&s_T, best);
  }
  lds_barrier();
  const int Tb = s_T < S * kmax ? s_T : S * kmax;
  int Wk[5];
  Wk[0] = 0;
#pragma unroll
  for (int k = 1; k <= 4; ++k) Wk[k] = k <= Tb ? pieces_for(S, Tb, k) : 1;
  const int waves = groups * (tot[1] * Wk[1] + tot[2] * Wk[2] + tot[3] * Wk[3] + tot[4] * Wk[4]);

  // active experts: records, and their waves' pieces, group-major, then chunk by chunk of
  // the slot list, piece p of a group and chunk taking steps floor(p S / W) .. floor((p + 1)
  // S / W) - 1 (advanced without division)
  const int pre[5] = {0, sv[1] & 0xFFFF, sv[1] >> 16, sv[2] & 0xFFFF, sv[2] >> 16};
  int sc = sv[0], sa = sv[3];
  int wb = groups * (pre[1] * Wk[1] + pre[2] * Wk[2] + pre[3] * Wk[3] + pre[4] * Wk[4]);
#pragma unroll
  for (int j = 0; j < PLAN_PER; ++j) {
    if (mine(j)) {
      const int e = e0 + j;
      s_start[e] = sc;
      if (cnt[j] > 0 && kk[j] > 0) {
        const int W = Wk[kk[j]];
        s_aidx[e] = sa;
        s_ka[sa] = (uint8_t)kk[j];
        PlanRec r;
        r.e = e;
        r.start = sc;
        r.cnt = cnt[j];
        r.k = kk[j];
        r.off = off[j];
        r.wave0 = wb;
        r.np = W;
        a.rec[sa] = r;
        const int base = S / W, rem = S - base * W;
        const int nch = (cnt[j] + a.R - 1) >> rsh;
        if (groups * nch * W <= PLAN_OWN_PIECES) {
          for (int grp = 0, q = wb; grp < groups; ++grp) {
            for (int c = 0; c < nch; ++c) {
              int s0 = 0, acc = 0;
              for (int p = 0; p < W; ++p, ++q) {
                acc += rem;
                const int s1 = s0 + base + (acc >= W ? 1 : 0);
                acc -= acc >= W ? W : 0;
                a.desc[q] = make_int4(sa, grp | (c << 16), p, s0 | (s1 << 16));
                s0 = s1;
              }
            }
          }
        } else {  // many pieces (a hot expert, or many groups): the whole block writes them
          s_big[atomicAdd(&s_nbig, 1)] = make_int4(sa, wb, W, nch);
        }
        sa += 1;
        wb += groups * W * nch;
      } else {
        s_aidx[e] = cnt[j] > 0 ? SLOT_BAD_UNIT : SLOT_EMPTY;
      }
      sc += cnt[j];
    }
  }
  if (tid == 0) {
    a.info[0] = n_act;
    a.info[1] = waves;
    a.info[2] = Tb;
    a.info[3] = n_chunks;
  }
  lds_barrier();

  // the pieces of the experts with many: wave v of the block takes experts v, v + 16, ...,
  // its lanes every 64th piece: wave wb + l is group l / (nch W), chunk (l / W) % nch,
  // piece l % W, whose steps are floor(p S / W) .. floor((p + 1) S / W) - 1 (the same as
  // the advancing form above)
  const int nbig = s_nbig;
  for (int b = tid >> 6; b < nbig; b += PLAN_WAVES) {  // uniform per wave
    const int4 bg = s_big[b];
    const int W = bg.z, cw = bg.w * W, nd = groups * cw;
    const float rcw = 1.0f / (float)cw, rw = 1.0f / (float)W;
    const bool fast = W * S < (1 << 22);  // l < nd <= GEMV_MAX_G always is
    for (int l = tid & 63; l < nd; l += 64) {
      const int grp = small_div(l, cw, rcw), r = l - grp * cw;
      const int c = small_div(r, W, rw), p = r - c * W;
      const int s0 = fast ? small_div(p * S, W, rw) : p * S / W;
      const int s1 = fast ? small_div((p + 1) * S, W, rw) : (p + 1) * S / W;
      a.desc[bg.y + l] = make_int4(bg.x, grp | (c << 16), p, s0 | (s1 << 16));
    }
  }

  // slot lists and per-slot records
  auto place = [&](int i, int v, int r) {
    int4 inf = make_int4(SLOT_EMPTY, 0, 0, 0);
    if (v == -1) {
    } else if (v < -1 || v >= E) {
      inf.x = SLOT_BAD_ID;
      bad |= STATUS_BAD_EXPERT;
    } else {
      const int ai = s_aidx[v];
      if (ai < 0) {
        inf.x = SLOT_BAD_UNIT;
        bad |= STATUS_BAD_UNIT;
      } else {
        a.list[s_start[v] + r] = i;
        const int k = s_ka[ai];
        inf = make_int4(v, Wk[k], k, 0);
      }
    }
    a.slot_info[i] = inf;
  };
  if (in_regs) {
#pragma unroll
    for (int j = 0; j < PLAN_R; ++j) {
      const int i = tid + PLAN_THREADS * j;
      if (i < N) place(i, id[j], rk[j]);
    }
  } else {
    for (int i = tid; i < N; i += PLAN_THREADS) {
      const int v = a.ids[i];
      place(i, v, (v >= 0 && v < E) ? a.rank[i] : 0);
    }
  }

  // launched waves past the split get no piece
  for (int w = waves + tid; w < a.Gl; w += PLAN_THREADS) a.desc[w] = make_int4(-1, 0, 0, 0);

  if (bad) atomicOr(&s_status, bad);
  lds_barrier();
  if (tid == 0 && s_status) set_status(a.status, s_status);
}

// Optional input rotation, the 128-wide Hadamard of FORMAT F8 on the 16 values of tile
// column c held by this lane: signs, then fp32 butterflies (a, b) -> (a + b, a - b) with
// strides 1, 2, 4, 8 inside the lane and 16, 32, 64 across lanes c ^ 1, 2, 4 (the 8 lanes
// of one 128-block), then x 0x3DB504F3 and bf16 round-to-nearest-even. Every stage is the
// same fp32 operation on the same values as in hadamard128, so the bits are the same: a
// sign is applied by flipping the sign bit, and the upper lane of a cross-lane pair forms
// a - b as (-b) + a.

// Sign-bit masks of the 16 signs of column c (0 or 0x80000000), or zeros without signs.
__device__ __forceinline__ void sign_masks(const int8_t* signs, int c, uint32_t m[16]) {
  if (!signs) {
#pragma unroll
    for (int j = 0; j < 16; ++j) m[j] = 0;
    return;
  }
  const uint4 sg = *reinterpret_cast<const uint4*>(signs + 16 * c);
  const uint32_t s4[4] = {sg.x, sg.y, sg.z, sg.w};
#pragma unroll
  for (int j = 0; j < 16; ++j) m[j] = (s4[j >> 2] << (24 - 8 * (j & 3))) & 0x80000000u;
}

// The value of lane l ^ D (D = 1, 2, 4; all lanes of the 8-lane group active), by DPP:
// quad permutations for 1 and 2, a quad reversal then a half-row mirror for 4.
template <int D>
__device__ __forceinline__ float lane_xor(float v) {
  int x = __float_as_int(v);
  if constexpr (D == 1) {
    x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (D == 2) {
    x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);  // quad_perm [2, 3, 0, 1]
  } else {
    static_assert(D == 4, "lane_xor: D is 1, 2 or 4");
    x = __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, true);   // quad_perm [3, 2, 1, 0]
    x = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);  // row_half_mirror
  }
  return __int_as_float(x);
}

template <int D>
__device__ __forceinline__ void cross_stage(float f[16], int c) {
  const uint32_t up = (c & D) ? 0x80000000u : 0u;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float other = lane_xor<D>(f[j]);
    f[j] = __uint_as_float(__float_as_uint(f[j]) ^ up) + other;
  }
}

// Signs and butterflies, then the scale; the caller rounds to bf16.
__device__ __forceinline__ void rotate_column_f32(float f[16], const uint32_t m[16], int c) {
#pragma unroll
  for (int j = 0; j < 16; ++j) f[j] = __uint_as_float(__float_as_uint(f[j]) ^ m[j]);
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if ((j & h) == 0) {
        const float x0 = f[j], x1 = f[j + h];
        f[j] = x0 + x1;
        f[j + h] = x0 - x1;
      }
    }
  }
  cross_stage<1>(f, c);
  cross_stage<2>(f, c);
  cross_stage<4>(f, c);
  const float scale = __uint_as_float(0x3DB504F3u);
#pragma unroll
  for (int j = 0; j < 16; ++j) f[j] = f[j] * scale;
}

__device__ __forceinline__ void rotate_column(float f[16], const uint32_t m[16], int c) {
  rotate_column_f32(f, m, c);
  round_bf16_pairs<16>(f);
}

// x~ of tile column c of token t as 16 floats (bf16 values), rotated when asked.
__device__ __forceinline__ void load_column(const PlanArgs& a, int t, int c, float f[16]) {
  const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)t * a.in);
  const uint4 u = src[2 * c], v = src[2 * c + 1];
  const uint32_t wv[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    f[2 * k] = bf16_lo_to_f32(wv[k]);
    f[2 * k + 1] = bf16_hi_to_f32(wv[k]);
  }
  if (a.rotate) {
    uint32_t m[16];
    sign_masks(a.signs, c, m);
    rotate_column(f, m, c);
  }
}

// Block-wide reductions over the waves that hold columns (nw of them).
__device__ __forceinline__ float block_max(float v, float* red, int nw) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  lds_barrier();
  float m = red[0];
  for (int w = 1; w < nw; ++w) m = fmaxf(m, red[w]);
  return m;
}

// Decode-GEMV operands of token t, one token per block: thread c converts tile column c
// (columns c + PLAN_THREADS, ... when in > 16 * PLAN_THREADS), rotating it first when asked.
// Waves without a column leave at once (a 128-block's 8 columns are always in one wave and
// all present or all absent). The token's scale 2^e is the largest power of two with
// max |x~| * 2^e <= 32639; every element becomes the integer x = rint(x~ * 2^e) (ties to
// even; exact for elements within 2^7 of the maximum), split as x = 256 hi + lo with hi, lo
// in [-128, 127]. Operand register r of a tile column holds bytes [v[r + 8], v[r + 8], v[r],
// v[r]] of one half (v = hi, then v = lo: two 32-byte rows per column), matching the
// weights' signed bytes (trellis_decode.h). The token's sum of the integers x and 2^-e are
// kept for the epilogue; a token with a non-finite element gets the scale NaN.
__device__ void prep_block(const PlanArgs& a, int t) {
  __shared__ float s_red[PLAN_WAVES];
  __shared__ int s_ired[PLAN_WAVES];
  const int tid = threadIdx.x;
  const int n_ti = a.in / 16;
  const int active = n_ti < PLAN_THREADS ? n_ti : PLAN_THREADS;
  const int nw = (active + 63) / 64;
  if ((tid & ~63) >= active) return;  // whole wave
  // pass 1: the largest magnitude (non-finite elements flagged as +inf); with at most
  // one column per thread the rotated column stays in registers for pass 2
  const bool one = n_ti <= PLAN_THREADS;
  float f0[16];
  float amax = 0.0f;
  auto fold_max = [&](const float f[16]) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float m = fabsf(f[j]);
      amax = fmaxf(amax, m <= 3.4e38f ? m : __builtin_inff());
    }
  };
  if (one) {
    if (tid < n_ti) {
      load_column(a, t, tid, f0);
      fold_max(f0);
    }
  } else {
    for (int c = tid; c < n_ti; c += PLAN_THREADS) {
      float f[16];
      load_column(a, t, c, f);
      fold_max(f);
    }
  }
  amax = block_max(amax, s_red, nw);
  int e = 0;
  bool finite = amax <= 3.4e38f;
  if (finite && amax > 0.0f) {
    int ex;
    (void)frexpf(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1)
    e = 15 - ex;
    if (ldexpf(amax, e) > 32639.0f) e -= 1;
  }
  // pass 2: integers, halves, operand layout
  int isum = 0;
  auto quantize = [&](const float f[16], int c) {
    int hi[16], lo[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float v = finite ? rintf(ldexpf(f[j], e)) : 0.0f;
      v = fminf(fmaxf(v, -32639.0f), 32639.0f);
      const int xi = (int)v;
      isum += xi;
      hi[j] = (xi + 128) >> 8;
      lo[j] = xi - (hi[j] << 8);
    }
    uint32_t H[8], L[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t h8 = (uint32_t)hi[r + 8] & 0xFFu, h0 = (uint32_t)hi[r] & 0xFFu;
      const uint32_t l8 = (uint32_t)lo[r + 8] & 0xFFu, l0 = (uint32_t)lo[r] & 0xFFu;
      H[r] = h8 | (h8 << 8) | (h0 << 16) | (h0 << 24);
      L[r] = l8 | (l8 << 8) | (l0 << 16) | (l0 << 24);
    }
    uint4* dh = reinterpret_cast<uint4*>(a.xq + ((size_t)(2 * t) * n_ti + c) * 8);
    uint4* dl = reinterpret_cast<uint4*>(a.xq + ((size_t)(2 * t + 1) * n_ti + c) * 8);
    dh[0] = make_uint4(H[0], H[1], H[2], H[3]);
    dh[1] = make_uint4(H[4], H[5], H[6], H[7]);
    dl[0] = make_uint4(L[0], L[1], L[2], L[3]);
    dl[1] = make_uint4(L[4], L[5], L[6], L[7]);
  };
  if (one) {
    if (tid < n_ti) quantize(f0, tid);
  } else {
    for (int c = tid; c < n_ti; c += PLAN_THREADS) {
      float f[16];
      load_column(a, t, c, f);
      quantize(f, c);
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) isum += __shfl_xor(isum, d, 64);
  if ((tid & 63) == 0) s_ired[tid >> 6] = isum;
  lds_barrier();
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < nw; ++w) s += s_ired[w];
    a.xsum[t] = s;
    a.xscale[t] = finite ? ldexpf(1.0f, -e) : __builtin_nanf("");
  }
}

template <bool TRELLIS>
__global__ __launch_bounds__(PLAN_THREADS) void gemv_plan_kernel(PlanArgs a) {
  if (blockIdx.x == 0)
    plan_block<TRELLIS>(a);
  else
    prep_block(a, blockIdx.x - 1);
}

// The routed FFN: block 0 plans the gate/up projection, block 1 the down projection (every
// slot a row of its own), the others prepare the tokens' gate/up operands.
__global__ __launch_bounds__(PLAN_THREADS) void ffn_plan_kernel(PlanArgs gu, PlanArgs dn) {
  if (blockIdx.x == 0)
    plan_block<true>(gu);
  else if (blockIdx.x == 1)
    plan_block<true>(dn);
  else
    prep_block(gu, blockIdx.x - 2);
}

// Prefill-GEMM operands, one token per block: thread c converts tile column c (columns
// c + blockDim, ... when in > 16 * blockDim), rotating it first when asked (bf16 rounding
// as hadamard128 does it), into f16 pairs [lo: x[r + 8], hi: x[r]]. Each token is first
// scaled by a power of two 2^s, the one that puts its largest magnitude in [2^14, 2^15):
// every element within 2^31 of that largest one is then exact in f16 (bf16 has 8
// significant bits, f16 11 above 2^-14), and no token can overflow the f16 range. The
// token's sum of its f16 values (in a fixed order: a column's 8 pairs in order, a thread's
// columns in order, the waves' butterfly, the waves in order) and 2^-s are kept
// for the epilogue; a token with a non-finite element gets 2^-s = NaN.
// At most 64 registers (8 waves per SIMD): the kernel waits on memory, so occupancy counts.
__global__ __launch_bounds__(PLAN_THREADS) __attribute__((amdgpu_waves_per_eu(8, 8)))
void activation_prep_kernel(PlanArgs a) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  __shared__ float s_red[PLAN_WAVES];
  __shared__ float s_sum[PLAN_WAVES];
  const int tid = threadIdx.x, stride = blockDim.x, nw = stride / 64;
  const int n_ti = a.in / 16;
  const int t = blockIdx.x;
  const bool one = n_ti <= stride;  // one column per thread: kept in registers
  const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)t * a.in);
  auto column = [&](int c, float f[16]) {
    const uint4 u = src[2 * c], v = src[2 * c + 1];
    const uint32_t wv[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      f[2 * q] = bf16_lo_to_f32(wv[q]);
      f[2 * q + 1] = bf16_hi_to_f32(wv[q]);
    }
    if (a.rotate) {
      uint32_t m[16];
      sign_masks(a.signs, c, m);
      rotate_column(f, m, c);
    }
  };
  float amax = 0.0f;
  auto fold_max = [&](const float f[16]) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float m = fabsf(f[j]);
      amax = fmaxf(amax, m <= 3.4e38f ? m : __builtin_inff());
    }
  };
  float f0[16];
  if (one) {
    if (tid < n_ti) {
      column(tid, f0);
      fold_max(f0);
    }
  } else {
    for (int c = tid; c < n_ti; c += stride) {
      float f[16];
      column(c, f);
      fold_max(f);
    }
  }
  amax = block_max(amax, s_red, nw);
  const bool finite = amax <= 3.4e38f;
  int e = 0;
  if (finite && amax > 0.0f) {
    int ex;
    (void)frexpf(amax, &ex);  // amax in [2^(ex - 1), 2^ex)
    e = min(15 - ex, 100);
  }
  float sum = 0.0f;
  auto convert = [&](const float f[16], int c) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    uint32_t P[8];
    float cs = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {  // one packed conversion and one dot product per pair
      const h2 p = __builtin_convertvector((f2){ldexpf(f[r + 8], e), ldexpf(f[r], e)}, h2);
      P[r] = __builtin_bit_cast(uint32_t, p);
      cs = __builtin_amdgcn_fdot2(p, (h2){(_Float16)1.0f, (_Float16)1.0f}, cs, false);
    }
    sum += cs;
    uint4* dst = reinterpret_cast<uint4*>(a.xp + (size_t)t * n_ti * 8);
    dst[2 * c] = make_uint4(P[0], P[1], P[2], P[3]);
    dst[2 * c + 1] = make_uint4(P[4], P[5], P[6], P[7]);
  };
  if (one) {
    if (tid < n_ti) convert(f0, tid);
  } else {
    for (int c = tid; c < n_ti; c += stride) {
      float f[16];
      column(c, f);
      convert(f, c);
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 64);
  if ((tid & 63) == 0) s_sum[tid >> 6] = sum;
  lds_barrier();
  if (tid == 0) {
    float v = 0.0f;
    for (int w = 0; w < nw; ++w) v += s_sum[w];
    a.rowsum[t] = make_float2(v, finite ? ldexpf(1.0f, -e) : __builtin_nanf(""));
  }
}

}  // namespace

hipError_t launch_gemv_plan(const PlanArgs& a, hipStream_t s) {
  const unsigned blocks = 1 + (a.x ? (unsigned)a.T : 0u);
  if (a.bits)
    hipLaunchKernelGGL(gemv_plan_kernel<true>, dim3(blocks), dim3(PLAN_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(gemv_plan_kernel<false>, dim3(blocks), dim3(PLAN_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ffn_plan(const PlanArgs& gate_up, const PlanArgs& down, hipStream_t s) {
  const unsigned blocks = 2 + (gate_up.x ? (unsigned)gate_up.T : 0u);
  hipLaunchKernelGGL(ffn_plan_kernel, dim3(blocks), dim3(PLAN_THREADS), 0, s, gate_up, down);
  return hipGetLastError();
}

hipError_t launch_activation_prep(const uint16_t* x, int64_t T, int in, uint32_t* xp,
                                  float2* rowsum, bool rotate, const int8_t* signs,
                                  hipStream_t s) {
  if (T == 0) return hipSuccess;
  PlanArgs a{};
  a.x = x;
  a.rotate = rotate;
  a.signs = signs;
  a.T = (int)T;
  a.in = in;
  a.xp = xp;
  a.rowsum = rowsum;
  // one thread per tile column (up to PLAN_THREADS): no wave without a column is launched
  const int n_ti = in / 16;
  const int threads = n_ti >= PLAN_THREADS ? PLAN_THREADS : (n_ti + 63) / 64 * 64;
  const unsigned blocks = (unsigned)T;
  hipLaunchKernelGGL(activation_prep_kernel, dim3(blocks), dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq

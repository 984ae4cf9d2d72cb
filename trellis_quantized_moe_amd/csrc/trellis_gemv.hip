// Decode-batch grouped GEMV over trellis-coded experts (gfx950).
//
// One workgroup of 4 waves per (expert, group of up to 8 output strips = 128 channels,
// K-slice); each wave owns a quarter of the slice and runs as an independent pipeline
// until one final barrier:
//   1. route scan: the wave reads the routes and keeps, in index order, the first 16
//      slots routed to its expert (ballot + bit count; no barrier);
//   2. stream: per step of 4 tile columns, every lane decodes one tile column (16
//      weights) of each of the 8 strips and feeds the matrix cores; the activations of
//      the 16 token rows come straight from the prepared f16 buffer (gemv_prep, once per
//      call) into A-operand registers. Code words and activations of the next step are
//      requested while the current step is decoded;
//   3. the four waves' accumulators are added through LDS in wave order and either
//      finished (one slice) or stored as the slice's partial sums.
// Per tile column a lane issues one load; the 16 lanes of a row read consecutive words and
// the 4 rows of a wave read 4 consecutive tiles, so each load instruction is one
// contiguous run. Tile addresses are wave-uniform (scalar registers).
//
// The matrix cores see each weight as two f16 subnormal operands, lo8(m) * 2^-24 and
// hi8(m) * 2^-24 (see trellis_decode.h), both against the same activation; the epilogue
// scales by 2^24 and removes 255 * sum(x) per token.
#include "gemv_common.h"
#include "tq_internal.h"
#include "trellis_decode.h"

namespace tq {

namespace {

struct Shared {
  float red[4 * 8 * 4 * 64];  // [wave][strip][i][lane]
  int slots[4][16];           // per wave: the chunk's slots (identical in every wave)
  SlotChunk ch;               // the chunk as seen by the epilogue
};

// ---- wave-level route scan ---------------------------------------------------------------
// Up to 16 slots with ids[slot] == e from position pos on, ascending, into sl[0..cnt).
// Returns cnt; *next = where the following chunk resumes (N when the routes are done).
// 1024 ids are requested at once, so a decode batch takes one round trip.
__device__ __forceinline__ int wave_collect(const int32_t* __restrict__ ids, int N, int e, int pos,
                                   int* sl, int* next) {
  const int lane = threadIdx.x & 63;
  int have = 0;
  *next = N;
  for (int base = pos; base < N; base += 1024) {
    int id[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = base + 64 * j + lane;
      id[j] = i < N ? ids[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint64_t m = __ballot(id[j] == e);
      const int r = have + (int)__builtin_amdgcn_mbcnt_hi(
                               (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      if (id[j] == e && r < 16) sl[r] = base + 64 * j + lane;
      const int total = have + (int)__popcll(m);
      if (total >= 16 && have < 16) {
        // the (16 - have)-th match of this ballot ends the chunk: resume after it
        uint64_t mm = m;
        for (int t = 1; t < 16 - have; ++t) mm &= mm - 1;
        *next = base + 64 * j + (int)__builtin_ctzll(mm) + 1;
      }
      have = total;
    }
    if (have >= 16) break;
  }
  __builtin_amdgcn_wave_barrier();
  return have < 16 ? have : 16;
}

// ---- code words --------------------------------------------------------------------------
// Words of one tile column a lane holds (see trellis_decode.h): K = 2 one word, K = 4 two,
// K = 3 three.
template <int K>
struct ColWords {
  uint32_t w[K == 2 ? 1 : (K == 4 ? 2 : 3)];
};

// Per-lane word offsets inside the wave's run of 4 consecutive tiles.
template <int K>
struct LaneOffsets {
  int o[3];
  uint32_t sh3;
  __device__ LaneOffsets(int g, int n) {
    constexpr int TW = 8 * K;
    o[0] = o[1] = o[2] = 0;
    sh3 = 0;
    if constexpr (K == 2) {
      o[0] = g * TW + n;
    } else if constexpr (K == 4) {
      o[0] = g * TW + 2 * n;
    } else {
      int a, b, c;
      k3_column_words(n, &a, &b, &c, &sh3);
      o[0] = g * TW + a;
      o[1] = g * TW + b;
      o[2] = g * TW + c;
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
    cw.w[2] = run[lo.o[2]];
  }
}

template <int K>
__device__ __forceinline__ void decode_col(const ColWords<K>& cw, uint32_t sh3, uint32_t M[8]) {
  if constexpr (K == 2)
    col_mpairs_k2(cw.w[0], row_next(cw.w[0]), M);
  else if constexpr (K == 4)
    col_mpairs_k4(cw.w[0], cw.w[1], row_next(cw.w[0]), M);
  else
    col_mpairs_k3(cw.w[0], cw.w[1], cw.w[2], sh3, M);
}

// ---- one chunk: stream this wave's quarter of the slice --------------------------------
// The wave's `steps` steps of 4 tile columns. One register set holds the current step's
// code words and activations; as soon as a strip's words are decoded, the same registers
// are reloaded with that strip's words of the next step, and the next step's activations
// are requested as soon as the current ones are in the A operands. Each load thus has about
// one step of work to arrive, at the register cost of a single step. (The last step
// reloads its own addresses, which hit in cache, so every load is unconditional.)
template <int K>
__device__ __forceinline__ void stream(const TrellisGemvArgs& a, const uint32_t* __restrict__ unit,
                                       int tok, int grp, int ns, int kcol0, f32x4 acc[8]) {
  constexpr int TW = 8 * K;
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int steps = a.steps;
  const int n_ti = a.in / 16;
  const int wcol0 = kcol0 + w * 4 * steps;  // first tile column of this wave
  const LaneOffsets<K> lo(g, n);
  const uint32_t* run = unit + ((size_t)grp * 8 * n_ti + wcol0) * TW;
  int sidx[8];
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) sidx[s8] = (s8 < ns ? s8 : ns - 1) * n_ti * TW;
  // A operand row n = this lane's token; tile column wcol0 + g of the step
  const uint4* xrow = reinterpret_cast<const uint4*>(a.xp + ((size_t)tok * n_ti + wcol0 + g) * 8);

  ColWords<K> cw[8];
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) load_col<K>(run + sidx[s8], lo, cw[s8]);
  uint4 xa = xrow[0], xb = xrow[1];
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) acc[s8] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int st = 0; st < steps; ++st) {
    const bool more = st + 1 < steps;
    const uint32_t* nrun = more ? run + 4 * TW : run;
    const uint4* nxrow = more ? xrow + 8 : xrow;  // 4 tile columns of 32 bytes further
    const u32x4 A0 = {xa.x, xa.y, xa.z, xa.w};   // pairs 0..3
    const u32x4 A1 = {xb.x, xb.y, xb.z, xb.w};   // pairs 4..7
    xa = nxrow[0];
    xb = nxrow[1];
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      uint32_t M[8], L[8], H[8];
      decode_col<K>(cw[s8], lo.sh3, M);
      load_col<K>(nrun + sidx[s8], lo, cw[s8]);
      bytes_as_f16<K>(M, L, H);
      acc[s8] = mfma_f16(A0, (u32x4){L[0], L[1], L[2], L[3]}, acc[s8]);
      acc[s8] = mfma_f16(A0, (u32x4){H[0], H[1], H[2], H[3]}, acc[s8]);
      acc[s8] = mfma_f16(A1, (u32x4){L[4], L[5], L[6], L[7]}, acc[s8]);
      acc[s8] = mfma_f16(A1, (u32x4){H[4], H[5], H[6], H[7]}, acc[s8]);
    }
    run = nrun;
    xrow = nxrow;
  }
}

// All chunks of expert e for this (group, slice).
template <int K>
__device__ __forceinline__ void run_expert(const TrellisGemvArgs& a, const GemvCommon& c, Shared& sh, int e,
                           int grp, int s, int ns, const uint32_t* __restrict__ unit) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kcol0 = s * 16 * a.steps;
  int pos = 0;
  while (true) {
    int next;
    const int cnt = wave_collect(a.ids, c.N, e, pos, sh.slots[w], &next);
    if (cnt == 0) break;  // identical in all waves: the whole workgroup leaves together
    pos = next;
    f32x4 acc[8];
    // rows past the chunk multiply token 0's activations; those rows are never stored
    const int n = lane & 15;
    const int tok = n < cnt ? sh.slots[w][n] / a.topk : 0;
    stream<K>(a, unit, tok, grp, ns, kcol0, acc);
    if (tid == 0) {
      sh.ch.cnt = cnt;
      sh.ch.next = next;
    }
    if (tid < 16) sh.ch.slots[tid] = sh.slots[0][tid];
    gemv_reduce_store(c, sh.red, acc, sh.ch, e, grp, s, ns);
    if (pos >= c.N) break;
  }
}

__global__ __launch_bounds__(GEMV_THREADS, 4) void trellis_gemv_kernel(TrellisGemvArgs a) {
  __shared__ Shared sh;
  GemvCommon c;
  c.ids = a.ids;
  c.gates = a.gates;
  c.scales = a.scales;
  c.rowsum = a.rowsum;
  c.acc_scale = GEMV_BYTE_SCALE;
  c.offset = GEMV_BYTE_OFFSET;
  c.y = a.y;
  c.partial = a.partial;
  c.N = (int)a.N;
  c.E = a.E;
  c.out = a.out;
  c.topk = a.topk;
  c.S = a.S;
  c.groups = a.groups;
  const int work = a.E * a.groups * a.S;
  const int bid = blockIdx.x;
  if (bid == work) {  // only launched with S == 1; with S > 1 the reduce launch does this
    special_slots(a.ids, c.N, a.E, a.out, a.y, a.status);
    return;
  }
  const int e = bid % a.E;
  const int rest = bid / a.E;
  const int grp = rest % a.groups;
  const int s = rest / a.groups;
  const int ns = min(8, a.out / 16 - grp * 8);
  const int K = a.bits[e];
  const int64_t off = a.code_off[e];
  if ((K < 2 || K > 4) || (off & 15)) {
    gemv_bad_unit(c, sh.ch, a.status, e, grp, s, ns);
    return;
  }
  const uint32_t* unit = a.codes + off / 4;
  if (K == 2)
    run_expert<2>(a, c, sh, e, grp, s, ns, unit);
  else if (K == 3)
    run_expert<3>(a, c, sh, e, grp, s, ns, unit);
  else
    run_expert<4>(a, c, sh, e, grp, s, ns, unit);
}

// ---- activation prep -----------------------------------------------------------------------
// One wave per token: each lane converts tile columns lane, lane + 64, ... (16 bf16 -> f16,
// round to nearest even) into the pair layout and sums the f16 values in a fixed order;
// the lane sums are combined by a fixed butterfly.
__global__ __launch_bounds__(64) void gemv_prep_kernel(const uint16_t* __restrict__ x, int in,
                                                      uint32_t* __restrict__ xp,
                                                      float* __restrict__ rowsum) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const int t = blockIdx.x, lane = threadIdx.x;
  const int n_ti = in / 16;
  float sum = 0.0f;
  for (int c = lane; c < n_ti; c += 64) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * in + (size_t)c * 16);
    const uint4 u = src[0], v = src[1];
    const uint32_t wv[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
    float f[16];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      f[2 * k] = bf16_lo_to_f32(wv[k]);
      f[2 * k + 1] = bf16_hi_to_f32(wv[k]);
    }
    uint32_t P[8];
    float hf[16];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const h2 p = (h2){(_Float16)f[r + 8], (_Float16)f[r]};
      P[r] = __builtin_bit_cast(uint32_t, p);
      hf[r] = (float)p.y;
      hf[r + 8] = (float)p.x;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += hf[i];
    uint4* dst = reinterpret_cast<uint4*>(xp + ((size_t)t * n_ti + c) * 8);
    dst[0] = make_uint4(P[0], P[1], P[2], P[3]);
    dst[1] = make_uint4(P[4], P[5], P[6], P[7]);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 64);
  if (lane == 0) rowsum[t] = sum;
}

// ---- decode hook ------------------------------------------------------------------------
// One wave per (strip, 4 tile columns); lane (g, n) decodes column n of tile column
// 4 * blk + g with the GEMV (path 0) or prefill (path 1) operand conversion, and writes
// q[out][in] as int16.
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
  decode_col<K>(cw, lo.sh3, M);
  int16_t* row = q + (size_t)(strip * 16 + n) * in + (ti0 + g) * 16;
  if (path == 0) {
    // the operands the matrix cores receive: L[r], H[r] hold inputs r (high half) and
    // r + 8 (low half) as f16 subnormals
    uint32_t L[8], H[8];
    bytes_as_f16<K>(M, L, H);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float qh = (f16_bits_to_f32(L[r] >> 16) + f16_bits_to_f32(H[r] >> 16)) * GEMV_BYTE_SCALE -
                       GEMV_BYTE_OFFSET;
      const float ql = (f16_bits_to_f32(L[r]) + f16_bits_to_f32(H[r])) * GEMV_BYTE_SCALE -
                       GEMV_BYTE_OFFSET;
      row[r] = (int16_t)qh;
      row[r + 8] = (int16_t)ql;
    }
  } else {
    uint32_t nat[8];
    mpairs_to_bf16_natural<K>(M, nat);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      row[2 * t] = (int16_t)bf16_lo_to_f32(nat[t]);
      row[2 * t + 1] = (int16_t)bf16_hi_to_f32(nat[t]);
    }
  }
}

}  // namespace

hipError_t launch_trellis_gemv(const TrellisGemvArgs& a, hipStream_t s) {
  const int blocks = a.E * a.groups * a.S + (a.S == 1 ? 1 : 0);
  hipLaunchKernelGGL(trellis_gemv_kernel, dim3(blocks), dim3(GEMV_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemv_prep(const uint16_t* x, int64_t T, int in, uint32_t* xp, float* rowsum,
                            hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(gemv_prep_kernel, dim3((unsigned)T), dim3(64), 0, s, x, in, xp, rowsum);
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

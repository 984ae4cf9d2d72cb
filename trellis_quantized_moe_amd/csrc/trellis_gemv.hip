// Decode-batch grouped GEMV over trellis-coded experts (gfx950).
//
// One workgroup (4 waves) per (expert, group of up to 8 output strips = 128 channels,
// K-slice). The workgroup scans the routes for its expert's slots (16 at a time), stages
// those tokens' activations for its K-slice in LDS as f16, packed in the pair order the
// decoder produces, and each wave streams its share of the slice: per step, every lane
// decodes one tile column (16 weights) of each strip and feeds the matrix cores. Per tile
// column a lane issues one load; the 16 lanes of a row read consecutive words and the 4
// rows of a wave read 4 consecutive tiles, so a wave's load is one contiguous run.
//
// The matrix cores see each weight as two f16 operands, 1024 + lo8(m) and 1024 + hi8(m)
// (see trellis_decode.h), both against the same activation; the constant part
// 2303 * sum(x) is removed from each row after accumulation.
#include "gemv_common.h"
#include "tq_internal.h"
#include "trellis_decode.h"

namespace tq {

namespace {

constexpr int MAX_STEPS = 5;
constexpr int SMEM_A_WORDS = 16 * MAX_STEPS * 16 * 8;   // [col][row][pair]
constexpr int SMEM_RED_WORDS = 4 * 8 * 4 * 64;          // [wave][strip][i][lane]
constexpr int SMEM_WORDS = SMEM_A_WORDS > SMEM_RED_WORDS ? SMEM_A_WORDS : SMEM_RED_WORDS;

struct Shared {
  uint32_t buf[SMEM_WORDS];
  float colsum[16 * MAX_STEPS * 16];
  float rowsum[16];
  SlotChunk ch;
};

// Stage A for one chunk: task (col c, row m) converts the 16 activations of tile column
// kcol0 + c of token m to f16 and packs them as the decoder's pairs: word r holds
// [lo: x[IL(r)], hi: x[IH(r)]]. Also the f16 values' sum per (col, row).
template <int K>
__device__ void stage_a(const TrellisGemvArgs& a, Shared& sh, int kcol0, int ncol) {
  for (int task = threadIdx.x; task < ncol * 16; task += GEMV_THREADS) {
    const int c = task >> 4, m = task & 15;
    uint32_t P[8];
    float sum = 0.0f;
    if (m < sh.ch.cnt) {
      const int tok = sh.ch.slots[m] / a.topk;
      const uint4* src = reinterpret_cast<const uint4*>(
          a.x + (size_t)tok * a.in + (size_t)(kcol0 + c) * 16);
      const uint4 v0 = src[0], v1 = src[1];
      const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      uint32_t h[16];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        h[2 * t] = f32_to_f16_bits(bf16_lo_to_f32(w[t]));
        h[2 * t + 1] = f32_to_f16_bits(bf16_hi_to_f32(w[t]));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += f16_bits_to_f32(h[i]);
#pragma unroll
      for (int r = 0; r < 8; ++r) P[r] = (h[pair_ih<K>(r)] << 16) | h[pair_il<K>(r)];
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) P[r] = 0u;
    }
    uint4* dst = reinterpret_cast<uint4*>(sh.buf + (size_t)(c * 16 + m) * 8);
    dst[0] = make_uint4(P[0], P[1], P[2], P[3]);
    dst[1] = make_uint4(P[4], P[5], P[6], P[7]);
    sh.colsum[c * 16 + m] = sum;
  }
}

// Words of one tile column and its m-pairs (see trellis_decode.h).
template <int K>
__device__ __forceinline__ void load_decode(const uint32_t* __restrict__ tile, int n,
                                            int o0, int o1, int o2, uint32_t sh3,
                                            uint32_t M[8]) {
  if constexpr (K == 2) {
    const uint32_t w = tile[n];
    col_mpairs_k2(w, row_next(w), M);
  } else if constexpr (K == 4) {
    const uint2 ww = *reinterpret_cast<const uint2*>(tile + 2 * n);
    col_mpairs_k4(ww.x, ww.y, row_next(ww.x), M);
  } else {
    col_mpairs_k3(tile[o0], tile[o1], tile[o2], sh3, M);
  }
}

template <int K>
__device__ void main_loop(const TrellisGemvArgs& a, Shared& sh,
                          const uint32_t* __restrict__ unit, int grp, int ns, int kcol0,
                          f32x4 acc[8]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  const int n_ti = a.in / 16;
  int o0 = 0, o1 = 0, o2 = 0;
  uint32_t sh3 = 0;
  if constexpr (K == 3) k3_column_words(n, &o0, &o1, &o2, &sh3);
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) acc[s8] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int st = 0; st < a.steps; ++st) {
    const int col = w * 4 * a.steps + 4 * st + g;
    const uint4* pa = reinterpret_cast<const uint4*>(sh.buf + (size_t)(col * 16 + n) * 8);
    const uint4 p0 = pa[0], p1 = pa[1];
    const u32x4 A0 = {p0.x, p0.x, p0.y, p0.y};
    const u32x4 A1 = {p0.z, p0.z, p0.w, p0.w};
    const u32x4 A2 = {p1.x, p1.x, p1.y, p1.y};
    const u32x4 A3 = {p1.z, p1.z, p1.w, p1.w};
    const int ti = kcol0 + col;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      if (s8 < ns) {
        const uint32_t* tile = unit + (size_t)((grp * 8 + s8) * n_ti + ti) * (8 * K);
        uint32_t M[8];
        load_decode<K>(tile, n, o0, o1, o2, sh3, M);
        u32x4 B;
        B = (u32x4){mpair_low_bytes_f16(M[0]), mpair_high_bytes_f16(M[0]),
                    mpair_low_bytes_f16(M[1]), mpair_high_bytes_f16(M[1])};
        acc[s8] = mfma_f16(A0, B, acc[s8]);
        B = (u32x4){mpair_low_bytes_f16(M[2]), mpair_high_bytes_f16(M[2]),
                    mpair_low_bytes_f16(M[3]), mpair_high_bytes_f16(M[3])};
        acc[s8] = mfma_f16(A1, B, acc[s8]);
        B = (u32x4){mpair_low_bytes_f16(M[4]), mpair_high_bytes_f16(M[4]),
                    mpair_low_bytes_f16(M[5]), mpair_high_bytes_f16(M[5])};
        acc[s8] = mfma_f16(A2, B, acc[s8]);
        B = (u32x4){mpair_low_bytes_f16(M[6]), mpair_high_bytes_f16(M[6]),
                    mpair_low_bytes_f16(M[7]), mpair_high_bytes_f16(M[7])};
        acc[s8] = mfma_f16(A3, B, acc[s8]);
      }
    }
  }
}

// All chunks of expert e for this (group, slice). Returns the number of slots found.
template <int K>
__device__ int run_expert(const TrellisGemvArgs& a, const GemvCommon& c, Shared& sh, int e,
                          int grp, int s, int ns, const uint32_t* __restrict__ unit) {
  const int tid = threadIdx.x;
  const int ncol = 16 * a.steps;
  const int kcol0 = s * ncol;
  int pos = 0, found = 0;
  while (true) {
    collect_slots(a.ids, c.N, e, pos, sh.ch);
    const int cnt = sh.ch.cnt;
    if (cnt == 0) break;
    found += cnt;
    pos = sh.ch.next;
    stage_a<K>(a, sh, kcol0, ncol);
    __syncthreads();
    if (tid < 16) {
      float r = 0.0f;
      for (int col = 0; col < ncol; ++col) r += sh.colsum[col * 16 + tid];
      sh.rowsum[tid] = r;
    }
    f32x4 acc[8];
    main_loop<K>(a, sh, unit, grp, ns, kcol0, acc);
    __syncthreads();
    gemv_reduce_store(c, reinterpret_cast<float*>(sh.buf), acc, sh.ch, sh.rowsum,
                      GEMV_BYTE_OFFSET, e, grp, s, ns);
    if (pos >= c.N) break;
  }
  return found;
}

__global__ __launch_bounds__(GEMV_THREADS) void trellis_gemv_kernel(TrellisGemvArgs a) {
  __shared__ Shared sh;
  GemvCommon c;
  c.ids = a.ids;
  c.gates = a.gates;
  c.scales = a.scales;
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

// ---- decode hook ------------------------------------------------------------------------
// One wave per (strip, 4 tile columns); lane (g, n) decodes column n of tile column
// 4 * blk + g with the GEMV (path 0) or prefill (path 1) operand conversion, and writes
// q[out][in] as int16.
template <int K>
__global__ __launch_bounds__(256) void trellis_decode_kernel(const uint32_t* __restrict__ codes,
                                                             int out, int in,
                                                             int16_t* __restrict__ q, int path) {
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int n_ti = in / 16;
  const int groups_per_strip = n_ti / 4;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= (out / 16) * groups_per_strip) return;  // whole wave exits together
  const int strip = wave / groups_per_strip;
  const int ti = (wave % groups_per_strip) * 4 + g;
  const uint32_t* tile = codes + (size_t)(strip * n_ti + ti) * (8 * K);
  int o0 = 0, o1 = 0, o2 = 0;
  uint32_t sh3 = 0;
  if constexpr (K == 3) k3_column_words(n, &o0, &o1, &o2, &sh3);
  uint32_t M[8];
  load_decode<K>(tile, n, o0, o1, o2, sh3, M);
  int16_t* row = q + (size_t)(strip * 16 + n) * in + ti * 16;
  if (path == 0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t lo = mpair_low_bytes_f16(M[r]), hi = mpair_high_bytes_f16(M[r]);
      const float qh = f16_bits_to_f32(lo >> 16) + f16_bits_to_f32(hi >> 16) - GEMV_BYTE_OFFSET;
      const float ql = f16_bits_to_f32(lo) + f16_bits_to_f32(hi) - GEMV_BYTE_OFFSET;
      row[pair_ih<K>(r)] = (int16_t)qh;
      row[pair_il<K>(r)] = (int16_t)ql;
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

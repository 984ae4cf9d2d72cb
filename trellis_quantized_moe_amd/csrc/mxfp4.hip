// MXFP4 routed-expert kernels (gfx950): decode hook, decode-batch GEMV, prefill GEMM.
//
// A unit is codes [out][in/2] (element 2j in the low nibble of byte j) followed by E8M0
// scales [out][in/32] (DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores"). gfx950 converts
// FP4 E2M1 pairs straight to bf16 with an fp32 scale (v_cvt_scalef32_pk_bf16_fp4), so a
// dword of 8 codes becomes 4 bf16 pairs in 4 instructions; E2M1 * 2^e is exact in bf16
// for every finite E8M0 scale, so decoding is bit-exact.
#include "gemm_core.h"
#include "gemv_common.h"
#include "tq_internal.h"

namespace tq {

namespace {

// E8M0 byte -> fp32 scale 2^(b-127): the byte is the fp32 exponent field; b = 0 is the
// subnormal 2^-127, b = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  uint32_t bits = b << 23;
  bits = (b == 0u) ? 0x00400000u : bits;
  bits = (b == 255u) ? 0x7FC00000u : bits;
  return __uint_as_float(bits);
}

// 8 codes (inputs 8j .. 8j+7, low nibble first) -> 4 dwords of bf16 pairs, natural order.
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t codes, float scale, uint32_t out[4]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
}

// ---- decode hook -----------------------------------------------------------------------
__global__ __launch_bounds__(256) void mxfp4_decode_kernel(const uint8_t* __restrict__ unit,
                                                           int out, int in,
                                                           uint16_t* __restrict__ wout) {
  const int per_row = in / 8;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= out * per_row) return;
  const int o = idx / per_row, j = idx % per_row;
  const uint32_t codes = *reinterpret_cast<const uint32_t*>(unit + (size_t)o * (in / 2) + 4 * j);
  const uint32_t sb = unit[(size_t)out * (in / 2) + (size_t)o * (in / 32) + (8 * j) / 32];
  uint32_t r[4];
  fp4x8_to_bf16(codes, e8m0_to_f32(sb), r);
  uint4* dst = reinterpret_cast<uint4*>(wout + (size_t)o * in + 8 * j);
  *dst = make_uint4(r[0], r[1], r[2], r[3]);
}

// ---- decode-batch GEMV -------------------------------------------------------------------
// One workgroup (4 waves) per (expert, group of 8 strips, K-slice). The slice's activations
// of the chunk's tokens sit in LDS as bf16 rows. Per step a wave covers 128 inputs: lane
// (g, n) loads 32 codes (16 bytes) of output n, inputs 32g .. 32g+31 of the step, plus the
// dword of scales of the step's 4 blocks, and feeds 4 matrix-core operations; operation c
// takes inputs 32g + 8c .. +7 of every lane group, and the A operand is read to match.
constexpr int MX_MAX_STEPS = 4;                            // 128-input steps per wave
constexpr int MX_SLICE_MAX = 4 * 128 * MX_MAX_STEPS;       // inputs per workgroup
constexpr int MX_ROW = MX_SLICE_MAX + 8;                   // bf16 per LDS row (+16 B pad)
constexpr int MX_SMEM_A_WORDS = 16 * MX_ROW / 2;
constexpr int MX_SMEM_RED_WORDS = 4 * 8 * 4 * 64;
constexpr int MX_SMEM_WORDS =
    MX_SMEM_A_WORDS > MX_SMEM_RED_WORDS ? MX_SMEM_A_WORDS : MX_SMEM_RED_WORDS;

struct MxShared {
  uint32_t buf[MX_SMEM_WORDS];
  SlotChunk ch;
};

__device__ int mx_run_expert(const Mxfp4GemvArgs& a, const GemvCommon& c, MxShared& sh, int e,
                             int grp, int s, int ns) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  const int slice = 512 * a.steps;
  const int kbase = s * slice;
  const int row_stride = slice + 8;  // bf16
  const size_t unit_bytes = (size_t)a.out * a.in / 2 + (size_t)a.out * a.in / 32;
  const uint8_t* unit = a.units + (size_t)e * unit_bytes;
  const uint8_t* scales = unit + (size_t)a.out * a.in / 2;
  uint16_t* A = reinterpret_cast<uint16_t*>(sh.buf);
  int pos = 0, found = 0;
  while (true) {
    collect_slots(a.ids, c.N, e, pos, sh.ch);
    const int cnt = sh.ch.cnt;
    if (cnt == 0) break;
    found += cnt;
    pos = sh.ch.next;
    // stage A: 16 rows x slice bf16, 16 bytes per task
    const int chunks = slice / 8;
    for (int task = tid; task < 16 * chunks; task += GEMV_THREADS) {
      const int m = task / chunks, q = task % chunks;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < cnt) {
        const int tok = sh.ch.slots[m] / a.topk;
        v = *reinterpret_cast<const uint4*>(a.x + (size_t)tok * a.in + kbase + 8 * q);
      }
      *reinterpret_cast<uint4*>(A + (size_t)m * row_stride + 8 * q) = v;
    }
    __syncthreads();
    f32x4 acc[8];
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) acc[s8] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int st = 0; st < a.steps; ++st) {
      const int k0 = w * 128 * a.steps + 128 * st;  // within the slice
      u32x4 Aop[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        Aop[cc] = *reinterpret_cast<const u32x4*>(A + (size_t)n * row_stride + k0 + 32 * g + 8 * cc);
      const int kg = kbase + k0;  // global input of the step
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) {
        if (s8 < ns) {
          const int o = grp * 128 + 16 * s8 + n;
          const uint4 cw = *reinterpret_cast<const uint4*>(unit + (size_t)o * (a.in / 2) +
                                                           (kg + 32 * g) / 2);
          const uint32_t sw = *reinterpret_cast<const uint32_t*>(scales + (size_t)o * (a.in / 32) +
                                                                 kg / 32);
          const float sc = e8m0_to_f32((sw >> (8 * g)) & 0xFFu);
          const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            uint32_t b[4];
            fp4x8_to_bf16(cws[cc], sc, b);
            acc[s8] = mfma_bf16(Aop[cc], (u32x4){b[0], b[1], b[2], b[3]}, acc[s8]);
          }
        }
      }
    }
    __syncthreads();
    gemv_reduce_store(c, reinterpret_cast<float*>(sh.buf), acc, sh.ch, e, grp, s, ns);
    if (pos >= c.N) break;
  }
  return found;
}

__global__ __launch_bounds__(GEMV_THREADS) void mxfp4_gemv_kernel(Mxfp4GemvArgs a) {
  __shared__ MxShared sh;
  GemvCommon c;
  c.ids = a.ids;
  c.gates = a.gates;
  c.scales = nullptr;
  c.rowsum = nullptr;
  c.acc_scale = 1.0f;
  c.offset = 0.0f;
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
  if (bid == work) {
    special_slots(a.ids, c.N, a.E, a.out, a.y, a.status);
    return;
  }
  const int e = bid % a.E;
  const int rest = bid / a.E;
  const int grp = rest % a.groups;
  const int s = rest / a.groups;
  const int ns = min(8, a.out / 16 - grp * 8);
  mx_run_expert(a, c, sh, e, grp, s, ns);
}

// ---- prefill GEMM --------------------------------------------------------------------------
// B producer: thread (o = tid / 2, h = tid % 2) decodes 16 codes of output o, inputs
// 32 kk + 16 h .. +15, with the scale of block kk.
// Thread t decodes, each step, inputs 16 h .. + 15 (h = t % 2) of the step for output
// channel o = t / 2: 8 code bytes and the channel's scale byte of the step's 32-block.
struct Mxfp4Producer {
  static constexpr bool kF16 = false;
  struct Raw {
    uint32_t c0, c1, sb;
  };
  GemmRsrc rc;
  uint32_t vo_c, vo_s;
  int o, h;

  __device__ Mxfp4Producer(const uint8_t* unit, int out, int in, int grp, int ns) {
    o = threadIdx.x >> 1;
    h = threadIdx.x & 1;
    rc = gemm_rsrc(unit, (uint32_t)((size_t)out * in / 2 + (size_t)out * in / 32));
    // channels past the group read its last channel (their rows of the B tile are unused)
    const int og = grp * 128 + (o < 16 * ns ? o : 16 * ns - 1);
    vo_c = (uint32_t)((size_t)og * (in / 2) + 8 * h);
    vo_s = (uint32_t)((size_t)out * in / 2 + (size_t)og * (in / 32));
  }

  __device__ __forceinline__ void load(int kk, Raw& r) const {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, vo_c, 16u * kk, 0);
    r.c0 = v.x;
    r.c1 = v.y;
    r.sb = __builtin_amdgcn_raw_buffer_load_b8(rc, vo_s, (uint32_t)kk, 0);
  }

  __device__ __forceinline__ void decode(const Raw& r, uint32_t nat[8]) const {
    const float sc = e8m0_to_f32(r.sb);
    fp4x8_to_bf16(r.c0, sc, nat);
    fp4x8_to_bf16(r.c1, sc, nat + 4);
  }
};

__global__ __launch_bounds__(GEMM_THREADS, 2) void mxfp4_gemm_kernel(Mxfp4GemmArgs a) {
  __shared__ GemmShared sh;
  const int item = blockIdx.x / a.groups;
  const int grp = blockIdx.x % a.groups;
  if (item >= *a.n_items) return;
  const int4 itd = reinterpret_cast<const int4*>(a.items)[item];
  const int e = itd.x;
  gemm_load_slots(sh, a.pairs, itd.y, itd.z);
  GemmItem it;
  it.x = a.x;
  it.x_bytes = a.x_bytes;
  it.rowsum = nullptr;
  it.gates = a.gates;
  it.scales = nullptr;
  it.y = a.y;
  it.in = a.in;
  it.out = a.out;
  it.topk = a.topk;
  it.grp = grp;
  it.nrows = itd.z;
  it.ns = min(8, a.out / 16 - grp * 8);
  const size_t unit_bytes = (size_t)a.out * a.in / 2 + (size_t)a.out * a.in / 32;
  Mxfp4Producer p(a.units + (size_t)e * unit_bytes, a.out, a.in, grp, it.ns);
  gemm_item(it, sh, p);
}

}  // namespace

hipError_t launch_mxfp4_decode(const uint8_t* unit, int out, int in, uint16_t* w,
                               hipStream_t s) {
  const int total = out * (in / 8);
  hipLaunchKernelGGL(mxfp4_decode_kernel, dim3((total + 255) / 256), dim3(256), 0, s, unit, out,
                     in, w);
  return hipGetLastError();
}

hipError_t launch_mxfp4_gemv(const Mxfp4GemvArgs& a, hipStream_t s) {
  const int blocks = a.E * a.groups * a.S + (a.S == 1 ? 1 : 0);
  hipLaunchKernelGGL(mxfp4_gemv_kernel, dim3(blocks), dim3(GEMV_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mxfp4_gemm(const Mxfp4GemmArgs& a, hipStream_t s) {
  const int blocks = a.max_items * a.groups;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp4_gemm_kernel, dim3(blocks), dim3(GEMM_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq

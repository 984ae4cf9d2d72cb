// Kernels of the two E8M0-scaled expert stores (gfx950): decode hooks, decode-batch GEMV,
// prefill GEMM (DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores").
//
// MXFP4 (routed experts): codes [out][in/2] (element 2j in the low nibble of byte j)
// followed by E8M0 scales [out][in/32]. gfx950 converts FP4 E2M1 pairs straight to bf16
// with an fp32 scale (v_cvt_scalef32_pk_bf16_fp4), so a dword of 8 codes becomes 4 bf16
// pairs in 4 instructions; E2M1 * 2^e is exact in bf16 for every finite E8M0 scale.
//
// fp8b32 (the shared expert): codes [out][in], one FP8 E4M3 byte per weight, followed by
// E8M0 scales [out/32][in/32], one per 32 x 32 block. v_cvt_scalef32_pk_bf16_fp8 turns two
// E4M3 bytes into a bf16 pair with the fp32 scale, so 32 codes also take 16 instructions;
// E4M3 * 2^e is exact in bf16 while the product stays a normal bf16 value.
//
// Both share one GEMV and one GEMM, with the unit format as a template parameter.
#include "gemm_core.h"
#include "gemv_wave.h"
#include "mx_unit.h"
#include "tq_internal.h"

namespace tq {

namespace {

// Repack kernel: thread i copies one (row, 32-input block) chunk of kCB code bytes of unit
// blockIdx.y from store order to the GEMV's read order; the scales are copied as they are.
template <int FMT>
__global__ __launch_bounds__(256) void mx_repack_kernel(const uint8_t* __restrict__ src,
                                                        uint8_t* __restrict__ dst, int out,
                                                        int in) {
  using U = MxUnit<FMT>;
  const size_t ub = U::unit_bytes(out, in);
  const uint8_t* su = src + (size_t)blockIdx.y * ub;
  uint8_t* du = dst + (size_t)blockIdx.y * ub;
  const int nkb = in / 32;
  const int64_t chunks = (int64_t)out * nkb;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < chunks) {
    const int o = (int)(i / nkb), kb = (int)(i % nkb);
    const uint4* a = reinterpret_cast<const uint4*>(su + U::stored_at(in, o, kb));
    uint4* b = reinterpret_cast<uint4*>(du + U::packed_at(out, in, o, kb));
    b[0] = a[0];
    if constexpr (U::kFp8) b[1] = a[1];
  }
  // the scales: 16-byte pieces after the codes
  const size_t cb = U::code_bytes(out, in), sbytes = ub - cb;
  for (size_t j = (size_t)i * 16; j < sbytes; j += (size_t)gridDim.x * 256 * 16) {
    if (j + 16 <= sbytes) {
      *reinterpret_cast<uint4*>(du + cb + j) = *reinterpret_cast<const uint4*>(su + cb + j);
    } else {
      for (size_t q = j; q < sbytes; ++q) du[cb + q] = su[cb + q];
    }
  }
}

// ---- decode hooks ----------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp8b32_decode_kernel(const uint8_t* __restrict__ unit,
                                                            int out, int in,
                                                            uint16_t* __restrict__ wout) {
  const int per_row = in / 8;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= out * per_row) return;
  const int o = idx / per_row, j = idx % per_row;
  const uint2 codes = *reinterpret_cast<const uint2*>(unit + (size_t)o * in + 8 * j);
  const uint32_t sb = unit[MxUnit<MX_FP8B32>::scale_at(out, in, o, (8 * j) / 32)];
  const float sc = e8m0_to_f32(sb);
  uint32_t r[4];
  fp8x4_to_bf16(codes.x, sc, r);
  fp8x4_to_bf16(codes.y, sc, r + 2);
  *reinterpret_cast<uint4*>(wout + (size_t)o * in + 8 * j) = make_uint4(r[0], r[1], r[2], r[3]);
}

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
// One wave is one worker of the plan (gemv_plan.h, every step costing 1): wave w streams its
// piece, 128-input steps s0 .. s1 - 1 of one group of 8 strips (128 output channels) of one
// expert, on its own. Per step and strip, lane (g, n) loads the 32 codes of output n,
// inputs 32 g .. 32 g + 31 of the step (16 bytes of MXFP4, 32 of fp8b32), takes that
// block's scale, and feeds 4 bf16 16 x 16 x 32 matrix-core operations: operation c takes
// inputs 32 g + 8 c .. + 7 of every lane group, against the same inputs of up to 16 routed
// token rows of one chunk of the expert's slot list (bf16 x as given; rows past the
// expert's count are zero). Codes are requested one step ahead, strip by strip after each
// strip's last use; activations one step ahead too, into a second register set, at the
// start of a step, so a step's first products never wait for its last code loads. The scales
// come in blocks of 4 steps: 16-byte loads bring the group's scale bytes of the next block
// into registers (MXFP4: 128 rows, two loads per lane; fp8b32: the 4 row blocks, lanes
// 0..3), which go to a double-buffered LDS stage at the block boundary; each lane then
// reads its byte per strip and step from LDS, so a step issues no scale load of its own.
// At the end the wave stores its accumulators as the piece's partial sums.
constexpr int MX_THREADS = 64;
constexpr int MX_WAVES_PER_SIMD = 3;  // MXFP4; fp8b32 (twice the code registers) 2
constexpr int MX_GEMV_TARGET_PER_CU = 12;

template <int FMT>
struct MxStep {
  u32x4 code[8][MxUnit<FMT>::kFp8 ? 2 : 1];
};

struct MxShared {
  // MXFP4: [row][step of the block][block of the step]; fp8b32: [row block][step][block]
  alignas(16) uint8_t sc[2][128 * 16];
};

// LDS offset of strip s8's scale byte relative to strip 0's
template <int FMT>
__device__ __forceinline__ int strip_scale_offset(int s8) {
  return MxUnit<FMT>::kFp8 ? 16 * (s8 >> 1) : 256 * s8;
}

__device__ __forceinline__ void load_x4(u32x4 (&x)[4], Rsrc rx, uint32_t xvo, uint32_t xst) {
#pragma unroll
  for (int c = 0; c < 4; ++c) x[c] = __builtin_amdgcn_raw_buffer_load_b128(rx, xvo, xst + 16u * c, 0);
}

// One step: 8 strips of the codes in `cur` against the activations x. With RELOAD, each
// strip's codes are replaced by those of the next step (scalar offset cst) after their
// last use.
template <int FMT, bool RELOAD>
__device__ __forceinline__ void mx_step(MxStep<FMT>& cur, const uint8_t* sc, Rsrc ru, uint32_t cvo,
                                        const uint32_t cso[8], uint32_t cst,
                                        const u32x4 (&x)[4], f32x4 acc[8]) {
  // sc: this lane's scale byte of strip 0 for this step; the 8 strips' bytes are read
  // together, so one LDS wait covers them
  uint32_t sbyte[8];
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) sbyte[s8] = sc[strip_scale_offset<FMT>(s8)];
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) {
    const float scale = e8m0_to_f32(sbyte[s8]);
    uint32_t b[4][4];
    if constexpr (MxUnit<FMT>::kFp8) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // inputs 8c .. 8c + 7 of the lane's 32: dwords 2c and 2c + 1 of its codes
        fp8x4_to_bf16(cur.code[s8][c >> 1][(2 * c) & 3], scale, b[c]);
        fp8x4_to_bf16(cur.code[s8][c >> 1][(2 * c + 1) & 3], scale, b[c] + 2);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) fp4x8_to_bf16(cur.code[s8][0][c], scale, b[c]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (RELOAD) {
      cur.code[s8][0] = __builtin_amdgcn_raw_buffer_load_b128(ru, cvo, cso[s8] + cst, 0);
      if constexpr (MxUnit<FMT>::kFp8)
        cur.code[s8][1] = __builtin_amdgcn_raw_buffer_load_b128(ru, cvo + 16u, cso[s8] + cst, 0);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc[s8] = mfma_bf16(x[c], (u32x4){b[c][0], b[c][1], b[c][2], b[c][3]}, acc[s8]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int FMT>
__device__ __forceinline__ void mx_stream(const Mxfp4GemvArgs& a, MxShared& sh, Rsrc ru, int tok,
                                          int grp, int ns, int s0, int s1, f32x4 acc[8]) {
  using U = MxUnit<FMT>;
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  // codes of output n, block g of a step: a per-lane offset, a scalar offset per strip and
  // one per step, in either layout
  uint32_t cvo, cstep, cso[8];
  if (a.layout == 0) {  // store order: rows of in/32 blocks
    const uint32_t row = U::row_bytes(a.in);
    cvo = n * row + U::kCB * g;
    cstep = 4 * U::kCB;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8)
      cso[s8] = (uint32_t)(grp * 128 + 16 * (s8 < ns ? s8 : ns - 1)) * row;
  } else {  // the GEMV's read order: a strip-step is 64 kCB contiguous bytes
    const uint32_t chunk = 64 * U::kCB;
    cvo = n * 4 * U::kCB + U::kCB * g;
    cstep = (uint32_t)ns * chunk;
    const uint32_t base = U::packed_at(a.out, a.in, grp * 128, 0);
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) cso[s8] = base + (uint32_t)(s8 < ns ? s8 : ns - 1) * chunk;
  }
  // scale rows of a 4-step block, 16 bytes each (4 steps x 4 blocks): MXFP4 lane L brings
  // rows L and L + 64 of the group; fp8b32 lanes 0..3 bring the group's 4 row blocks
  uint32_t svo0, svo1;
  if constexpr (U::kFp8) {
    svo0 = U::scale_at(a.out, a.in, 32 * (grp * 4 + (lane & 3)), 0);
    svo1 = svo0;
  } else {
    svo0 = U::scale_at(a.out, a.in, grp * 128 + lane, 0);
    svo1 = U::scale_at(a.out, a.in, grp * 128 + lane + 64, 0);
  }
  const Rsrc rx = make_rsrc(a.x, a.x_bytes);
  const uint32_t xvo = tok >= 0 ? (uint32_t)tok * (uint32_t)a.in * 2u + 64u * g : 0x80000000u;
  const int steps = s1 - s0;
  auto cst = [&](int st) { return cstep * (uint32_t)(s0 + st); };
  auto xst = [&](int st) { return 256u * (uint32_t)(s0 + st); };
  // scale bytes of the 4-step block starting at step st (4 bytes per row and step)
  auto bso = [&](int st) { return 4u * (uint32_t)(s0 + st); };
  // codes one step ahead, reloaded strip by strip; activations in two register sets, the
  // next step's requested at the start of a step (ahead of its codes), so a step's first
  // products wait only for what they use
  MxStep<FMT> ring;
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) {
    ring.code[s8][0] = __builtin_amdgcn_raw_buffer_load_b128(ru, cvo, cso[s8] + cst(0), 0);
    if constexpr (U::kFp8)
      ring.code[s8][1] = __builtin_amdgcn_raw_buffer_load_b128(ru, cvo + 16u, cso[s8] + cst(0), 0);
  }
  u32x4 sa = __builtin_amdgcn_raw_buffer_load_b128(ru, svo0, bso(0), 0);
  u32x4 sb = U::kFp8 ? sa : __builtin_amdgcn_raw_buffer_load_b128(ru, svo1, bso(0), 0);
  u32x4 xr[2][4];
  load_x4(xr[0], rx, xvo, xst(0));
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) acc[s8] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // this lane's scale byte of strip 0: step k of the block at + 4 k, block g of the step
  const int sbase = U::kFp8 ? g : 16 * n + g;
  // the wave's issue priority drops by quarters of its piece, so that the waves sharing a
  // SIMD stream together to the end (the SIMD otherwise issues for its oldest wave first)
  const int q1 = steps >> 2, q2 = steps >> 1, q3 = (3 * steps) >> 2;
  __builtin_amdgcn_s_setprio(3);
  for (int blk = 0; blk < steps; blk += 4) {
    if (blk >= q1 && blk < q1 + 4) __builtin_amdgcn_s_setprio(2);
    if (blk >= q2 && blk < q2 + 4) __builtin_amdgcn_s_setprio(1);
    if (blk >= q3 && blk < q3 + 4) __builtin_amdgcn_s_setprio(0);
    const int buf = (blk >> 2) & 1;
    if constexpr (U::kFp8) {
      if (lane < 4) *reinterpret_cast<u32x4*>(&sh.sc[buf][16 * lane]) = sa;
    } else {
      *reinterpret_cast<u32x4*>(&sh.sc[buf][16 * lane]) = sa;
      *reinterpret_cast<u32x4*>(&sh.sc[buf][16 * (lane + 64)]) = sb;
    }
    if (blk + 4 < steps) {  // the next block's scales, in flight during this block
      sa = __builtin_amdgcn_raw_buffer_load_b128(ru, svo0, bso(blk + 4), 0);
      if constexpr (!U::kFp8) sb = __builtin_amdgcn_raw_buffer_load_b128(ru, svo1, bso(blk + 4), 0);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int st = blk + k;  // its activations are in xr[k & 1] (blk is a multiple of 4)
      if (st < steps) {        // uniform
        if (st + 1 < steps) {
          load_x4(xr[(k + 1) & 1], rx, xvo, xst(st + 1));
          mx_step<FMT, true>(ring, &sh.sc[buf][sbase + 4 * k], ru, cvo, cso, cst(st + 1),
                             xr[k & 1], acc);
        } else {
          mx_step<FMT, false>(ring, &sh.sc[buf][sbase + 4 * k], ru, cvo, cso, 0, xr[k & 1], acc);
        }
      }
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(MX_THREADS, MxUnit<FMT>::kFp8 ? 2 : MX_WAVES_PER_SIMD) void mxfp4_gemv_kernel(Mxfp4GemvArgs a) {
  __shared__ MxShared sh;
  Piece pc;
  if (!load_piece(a.desc, blockIdx.x, pc)) return;
  const PlanRec r = load_rec(a.rec, pc.ai);
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int ns = min(8, a.out / 16 - pc.grp * 8);
  const Rsrc ru = make_rsrc(a.units + r.off, (uint32_t)MxUnit<FMT>::unit_bytes(a.out, a.in));
  float* dst = a.partial + (size_t)pc.idx * a.N * a.out + pc.grp * 128 + n;
  {
    const int c0 = 16 * pc.chunk;  // this wave's chunk of the slot list
    const int rows = min(16, r.cnt - c0);
    const int slot = n < rows ? a.list[r.start + c0 + n] : -1;
    f32x4 acc[8];
    mx_stream<FMT>(a, sh, ru, slot >= 0 ? slot / a.topk : -1, pc.grp, ns, pc.s0, pc.s1, acc);
    // accumulator element i of lane (g, n) is token row 4 g + i, output channel n of its strip
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      const int sm = __shfl(slot, m);
      if (m < rows) {
        float* rowp = dst + (size_t)sm * a.out;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8)
          if (s8 < ns) rowp[s8 * 16] = acc[s8][i];
      }
    }
  }
}

}  // namespace

hipError_t launch_mxfp4_decode(const uint8_t* unit, int out, int in, uint16_t* w,
                               hipStream_t s) {
  const int total = out * (in / 8);
  hipLaunchKernelGGL(mxfp4_decode_kernel, dim3((total + 255) / 256), dim3(256), 0, s, unit, out,
                     in, w);
  return hipGetLastError();
}

hipError_t launch_fp8b32_decode(const uint8_t* unit, int out, int in, uint16_t* w,
                                hipStream_t s) {
  const int total = out * (in / 8);
  hipLaunchKernelGGL(fp8b32_decode_kernel, dim3((total + 255) / 256), dim3(256), 0, s, unit, out,
                     in, w);
  return hipGetLastError();
}

hipError_t launch_mx_repack(int fmt, const uint8_t* src, uint8_t* dst, int E, int out, int in,
                            hipStream_t s) {
  const int64_t chunks = (int64_t)out * (in / 32);
  const dim3 grid((unsigned)((chunks + 255) / 256), (unsigned)E);
  if (fmt == MX_FP8B32)
    hipLaunchKernelGGL(mx_repack_kernel<MX_FP8B32>, grid, dim3(256), 0, s, src, dst, out, in);
  else
    hipLaunchKernelGGL(mx_repack_kernel<MX_FP4>, grid, dim3(256), 0, s, src, dst, out, in);
  return hipGetLastError();
}

int mxfp4_gemv_grid(int fmt) {
  static int cache[2][64];
  int dev = 0;
  if (fmt != MX_FP4 && fmt != MX_FP8B32) return 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[fmt][dev]) return cache[fmt][dev];
  int per_cu = 0, cus = 0;
  const hipError_t e =
      fmt == MX_FP8B32
          ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mxfp4_gemv_kernel<MX_FP8B32>, MX_THREADS, 0)
          : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mxfp4_gemv_kernel<MX_FP4>, MX_THREADS, 0);
  if (e != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  // the MXFP4 GEMV waits on memory more than it issues: as many waves as its registers
  // allow (3 per SIMD; fp8b32 2), up to 3 per SIMD
  int g = std::min(per_cu, MX_GEMV_TARGET_PER_CU) * cus;
  if (g > GEMV_MAX_G) g = GEMV_MAX_G;
  if (g < 1) g = 1;
  if (dev >= 0 && dev < 64) cache[fmt][dev] = g;
  return g;
}

hipError_t launch_mxfp4_gemv(const Mxfp4GemvArgs& a, hipStream_t s) {
  if (a.fmt == MX_FP8B32)
    return launch_timed(mxfp4_gemv_kernel<MX_FP8B32>, dim3(a.G), dim3(MX_THREADS), s, a);
  return launch_timed(mxfp4_gemv_kernel<MX_FP4>, dim3(a.G), dim3(MX_THREADS), s, a);
}

}  // namespace tq

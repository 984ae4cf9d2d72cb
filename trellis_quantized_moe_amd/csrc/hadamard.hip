// 128-wide Hadamard rotation of bf16 rows (FORMAT F8; DeepSeek-V4.1-Flash-1017 · dsx T16
// page, "How T16 works", opening paragraph; exlr8 page, "Stores": per-layer signs).
//
// HBM-bound: each element is read and written once. A 128-block is held by 16 lanes, 8
// consecutive elements each (one 16-byte load and store per lane), so a wave rotates 4
// blocks. Butterfly strides 1, 2, 4 run inside a lane; strides 8 .. 64 pair lane l with
// lane l ^ 1, 2, 4, 8 of the same block. Every stage is the fp32 pair map
// (a, b) -> (a + b, a - b) with a the lower index; the result is scaled by fp32
// 0x3DB504F3 and rounded to bf16 nearest-even. No multiply-add is fused (the file is
// compiled with -ffp-contract=off), so the bits do not depend on scheduling.
#include "hadamard_lane.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

__global__ __launch_bounds__(256) void hadamard128_kernel(const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ y,
                                                          int64_t nblocks, int64_t n,
                                                          const int8_t* __restrict__ signs) {
  const int64_t gtid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gtid >> 4;        // 128-block index (row-major over [rows][n/128])
  const int sub = threadIdx.x & 15;     // lane within the block: elements 8 sub .. 8 sub + 7
  const bool active = blk < nblocks;
  const int64_t bpr = n / 128;
  const int64_t row = active ? blk / bpr : 0;
  const int64_t col0 = active ? (blk % bpr) * 128 + 8 * sub : 0;
  float v[8];
  if (active) {
    const uint4 w = *reinterpret_cast<const uint4*>(x + row * n + col0);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[2 * t] = bf16_lo_to_f32(ww[t]);
      v[2 * t + 1] = bf16_hi_to_f32(ww[t]);
    }
    if (signs) {
      const uint2 sg = *reinterpret_cast<const uint2*>(signs + col0);
      const uint32_t s2[2] = {sg.x, sg.y};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int8_t sj = (int8_t)((s2[j >> 2] >> (8 * (j & 3))) & 0xFF);
        if (sj < 0) v[j] = -v[j];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  }
  fwht128_lane8(v, sub);
  if (!active) return;
  const float scale = __uint_as_float(0x3DB504F3u);
  uint32_t o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t lo = f32_to_bf16_rne(v[2 * t] * scale);
    const uint32_t hi = f32_to_bf16_rne(v[2 * t + 1] * scale);
    o[t] = lo | (hi << 16);
  }
  *reinterpret_cast<uint4*>(y + row * n + col0) = make_uint4(o[0], o[1], o[2], o[3]);
}

// Output-side rotation of fp32 rows, in place (FORMAT F17; exlr8 page, "Stores": the
// Hadamard on both sides): per block of 128 outputs y = s * ((H / sqrt(128)) y). A block is
// held by 32 lanes, 4 consecutive values each (one 16-byte load and store per lane);
// strides 1, 2 run inside a lane, 4 .. 64 pair lane l with lane l ^ 1 .. 16 of the block.
__device__ __forceinline__ void fwht128_quad(float v[4], int sub) {
#pragma unroll
  for (int h = 1; h < 4; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if ((j & h) == 0) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int d = 1; d < 32; d <<= 1) {
    const bool upper = (sub & d) != 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float other = __shfl_xor(v[j], d, 64);
      v[j] = upper ? other - v[j] : v[j] + other;
    }
  }
}

__global__ __launch_bounds__(256) void rotate_out_kernel(float* __restrict__ y, int64_t nblocks,
                                                         const int8_t* __restrict__ signs,
                                                         int out) {
  const int64_t gtid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gtid >> 5;   // 128-block, row-major over [rows][out / 128]
  const int sub = threadIdx.x & 31;
  const bool active = blk < nblocks;
  const int64_t bpr = out / 128;
  const int64_t row = active ? blk / bpr : 0;
  const int col0 = active ? (int)(blk % bpr) * 128 + 4 * sub : 0;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  float4* p = reinterpret_cast<float4*>(y + row * out + col0);
  if (active) {
    const float4 a = *p;
    v[0] = a.x;
    v[1] = a.y;
    v[2] = a.z;
    v[3] = a.w;
  }
  fwht128_quad(v, sub);
  if (!active) return;
  const float scale = __uint_as_float(0x3DB504F3u);
  const uint32_t sg = *reinterpret_cast<const uint32_t*>(signs + col0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = v[j] * scale;
    if ((int8_t)((sg >> (8 * j)) & 0xFF) < 0) v[j] = -v[j];
  }
  *p = make_float4(v[0], v[1], v[2], v[3]);
}

}  // namespace

hipError_t launch_rotate_out(float* y, int64_t rows, int out, const int8_t* signs,
                             hipStream_t s) {
  const int64_t nblocks = rows * (out / 128);
  if (nblocks == 0) return hipSuccess;
  const int64_t grid = (nblocks * 32 + 255) / 256;
  hipLaunchKernelGGL(rotate_out_kernel, dim3((unsigned)grid), dim3(256), 0, s, y, nblocks, signs,
                     out);
  return hipGetLastError();
}

hipError_t launch_hadamard(const uint16_t* x, uint16_t* y, int64_t rows, int64_t n,
                           const int8_t* signs, hipStream_t s) {
  const int64_t nblocks = rows * (n / 128);
  if (nblocks == 0) return hipSuccess;
  const int64_t threads = nblocks * 16;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(hadamard128_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, y, nblocks,
                     n, signs);
  return hipGetLastError();
}

}  // namespace tq

// MXFP4 -> NVFP4 transcode (gfx950; FORMAT F13, DeepSeek-V4.1-Flash-1017 NVFP4 page,
// "Model": the 16-element blocks refine the 32-element blocks of the official store).
//
// Per unit (one expert's out x in MXFP4 weights): the E2M1 nibbles stay as they are; each
// 32-block with E8M0 byte b becomes two 16-blocks with the E4M3 scale 2^(b - bmax + 8),
// where bmax is the unit's largest scale byte, and the unit gets the fp32 second-level
// scale 2^(bmax - 127 - 8). The product of the two scales is 2^(b - 127), the MXFP4 scale,
// exactly whenever 2^(b - bmax + 8) is an E4M3 value, i.e. bmax - b <= 17; a block further
// below the maximum gets the scale 0 (its values flush to zero) and the unit is flagged
// lossy. A block whose E8M0 byte is 255 (NaN) gets the E4M3 NaN 0x7F in both halves and the
// unit is flagged; the other blocks are anchored at the largest non-NaN byte.
//
// The pass is a stream: every block of a unit reads the unit's scale bytes (L2-served after
// the first) to find bmax, then writes its share of the scale pairs and copies its share of
// the nibbles with 16-byte loads and stores.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr int NV_THREADS = 256;
constexpr int NV_SPLIT = 16;  // blocks per unit

// E4M3 byte of 2^k for k <= 8: normal for k >= -6, subnormal for -9 <= k < -6, 0 below.
__device__ __forceinline__ uint32_t e4m3_pow2(int k) {
  if (k >= -6) return (uint32_t)(k + 7) << 3;
  if (k >= -9) return 1u << (k + 9);
  return 0u;
}

// Bytes of v (4 per word) mapped to E4M3 scale pairs: 16 scale bytes -> 32 output bytes.
__device__ __forceinline__ uint32_t pair_bytes(uint32_t w, int half, int bmax) {
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int b = (int)((w >> (8 * (2 * half + j))) & 0xFFu);
    const uint32_t s = b == 255 ? 0x7Fu : e4m3_pow2(b - bmax + 8);
    r |= (s | (s << 8)) << (16 * j);
  }
  return r;
}

__global__ __launch_bounds__(NV_THREADS) void nvfp4_transcode_kernel(
    const uint8_t* __restrict__ units, int out, int in, uint8_t* __restrict__ codes_out,
    uint8_t* __restrict__ scales_out, float* __restrict__ scale2_out,
    uint8_t* __restrict__ status_out) {
  __shared__ int s_max[NV_THREADS / 64], s_min[NV_THREADS / 64], s_nan[NV_THREADS / 64];
  const int e = blockIdx.y, part = blockIdx.x, tid = threadIdx.x;
  const size_t ncode = (size_t)out * in / 2, nsc = (size_t)out * in / 32;
  const uint8_t* unit = units + (size_t)e * (ncode + nsc);
  const uint4* sc4 = reinterpret_cast<const uint4*>(unit + ncode);
  const int n4 = (int)(nsc / 16);

  // 1. largest and smallest non-NaN scale byte of the unit, and whether any is NaN
  int bmax = 0, bmin = 255, nan = 0;
  for (int i = tid; i < n4; i += NV_THREADS) {
    const uint4 v = sc4[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int b = (int)((w[q >> 2] >> (8 * (q & 3))) & 0xFFu);
      if (b == 255) {
        nan = 1;
      } else {
        bmax = max(bmax, b);
        bmin = min(bmin, b);
      }
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    bmax = max(bmax, __shfl_xor(bmax, d, 64));
    bmin = min(bmin, __shfl_xor(bmin, d, 64));
    nan |= __shfl_xor(nan, d, 64);
  }
  if ((tid & 63) == 0) {
    s_max[tid >> 6] = bmax;
    s_min[tid >> 6] = bmin;
    s_nan[tid >> 6] = nan;
  }
  __syncthreads();
  bmax = s_max[0];
  bmin = s_min[0];
  nan = s_nan[0];
#pragma unroll
  for (int w = 1; w < NV_THREADS / 64; ++w) {
    bmax = max(bmax, s_max[w]);
    bmin = min(bmin, s_min[w]);
    nan |= s_nan[w];
  }

  // 2. this block's share of the scale pairs: 16 scale bytes -> 32 bytes of E4M3 pairs
  uint4* ws4 = reinterpret_cast<uint4*>(scales_out + (size_t)e * 2 * nsc);
  const int per_s = (n4 + NV_SPLIT - 1) / NV_SPLIT;
  for (int i = part * per_s + tid; i < min(n4, (part + 1) * per_s); i += NV_THREADS) {
    const uint4 v = sc4[i];
    ws4[2 * i] = make_uint4(pair_bytes(v.x, 0, bmax), pair_bytes(v.x, 1, bmax),
                            pair_bytes(v.y, 0, bmax), pair_bytes(v.y, 1, bmax));
    ws4[2 * i + 1] = make_uint4(pair_bytes(v.z, 0, bmax), pair_bytes(v.z, 1, bmax),
                                pair_bytes(v.w, 0, bmax), pair_bytes(v.w, 1, bmax));
  }

  // 3. this block's share of the nibbles, unchanged
  const uint4* c4 = reinterpret_cast<const uint4*>(unit);
  uint4* o4 = reinterpret_cast<uint4*>(codes_out + (size_t)e * ncode);
  const int nc4 = (int)(ncode / 16), per_c = (nc4 + NV_SPLIT - 1) / NV_SPLIT;
  for (int i = part * per_c + tid; i < min(nc4, (part + 1) * per_c); i += NV_THREADS)
    o4[i] = c4[i];

  if (part == 0 && tid == 0) {
    // 2^(bmax - 135) as fp32: normal for bmax >= 9, subnormal below
    const uint32_t bits = bmax >= 9 ? (uint32_t)(bmax - 8) << 23 : 1u << (bmax + 14);
    scale2_out[e] = __uint_as_float(bits);
    status_out[e] = nan ? 2 : (bmax - bmin <= 17 ? 1 : 0);
  }
}

}  // namespace

hipError_t launch_nvfp4_transcode(const uint8_t* units, int E, int out, int in,
                                  uint8_t* codes, uint8_t* scales, float* scale2,
                                  uint8_t* status, hipStream_t s) {
  hipLaunchKernelGGL(nvfp4_transcode_kernel, dim3(NV_SPLIT, E), dim3(NV_THREADS), 0, s, units,
                     out, in, codes, scales, scale2, status);
  return hipGetLastError();
}

}  // namespace tq

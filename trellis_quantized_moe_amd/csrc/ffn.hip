// The routed expert FFN's middle step (FORMAT F15), one workgroup per routed slot: from the
// slot's fused gate/up outputs gu (2I channels: the gate's I, then the up's) it forms
// h = silu(g) * u, rotates h with the down projection's signs, and writes the down
// projection's activation operands for that slot's row; h and its rotation stay in fp32
// registers (never stored).
//
// Thread j takes channels 4 j .. 4 j + 3 of the intermediate (I / 4 threads, so a 128-block
// is 32 lanes of one wave):
//   1. g and u: decode batches reduce the gate/up GEMV's pieces of outputs 4 j and I + 4 j
//      exactly as the piece reduction does (piece_slot); prefill reads the GEMM's fp32 rows;
//   2. the gate/up layer's output-side rotation when it has one (F17), per 128-block of g
//      and of u;
//   3. h = silu(g) * u, silu(a) = a / (1 + e^-a), fp32;
//   4. v = (H / sqrt(128)) (s * h) per 128-block: fp32 butterflies (strides 1, 2 in the
//      lane, 4 .. 64 across lanes), times fp32 0x3DB504F3;
//   5. the row's largest |v| (a block reduction), then the mode's operands:
//      decode: 16-bit integers rint(v 2^e) (the largest 2^e with max |v| 2^e <= 32639) in
//      the GEMV's int8-half layout, with the row's sum of integers and 2^-e;
//      prefill: f16 values of v 2^e (2^e putting max |v| in [2^14, 2^15)) in the GEMM's
//      pair layout, with the row's sum of them and 2^-e.
// A slot whose g or u is not finite (a bad id or unit upstream) gets 2^-e = NaN, so its
// down-projection output is NaN; an empty slot's row is zero.
#include "gemv_reduce.h"

namespace tq {

namespace {

// Butterflies of a 128-block held as 4 consecutive values by each of 32 lanes (sub = lane
// index within the block): strides 1, 2 in the lane, 4 .. 64 across lanes l ^ 1 .. 16.
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

__device__ __forceinline__ void flip4(float v[4], const int8_t* signs, int c) {
  if (!signs) return;
  const uint32_t sg = *reinterpret_cast<const uint32_t*>(signs + c);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if ((int8_t)((sg >> (8 * j)) & 0xFF) < 0) v[j] = -v[j];
}

constexpr int MID_MAX_THREADS = 1024;  // I <= 4096
constexpr int MID_MAX_WAVES = MID_MAX_THREADS / 64;

template <bool DECODE>
__global__ __launch_bounds__(MID_MAX_THREADS) void ffn_mid_kernel(FfnMidArgs a) {
  __shared__ float s_red[MID_MAX_WAVES];
  __shared__ float s_sum[MID_MAX_WAVES];
  __shared__ int s_isum[MID_MAX_WAVES];
  __shared__ int32_t s_x[4 * MID_MAX_THREADS];  // decode: the row's 16-bit integers
  __shared__ float s_f[4 * MID_MAX_THREADS];    // prefill: the row's scaled f16 values
  const int n = blockIdx.x, j = threadIdx.x, I = a.I;
  const int nw = blockDim.x / 64, sub = j & 31;
  float g[4], u[4];
  if constexpr (DECODE) {
    const float4 gv = piece_slot<true>(a.gu, n, 4 * j);
    const float4 uv = piece_slot<true>(a.gu, n, I + 4 * j);
    g[0] = gv.x; g[1] = gv.y; g[2] = gv.z; g[3] = gv.w;
    u[0] = uv.x; u[1] = uv.y; u[2] = uv.z; u[3] = uv.w;
  } else {
    const float4 gv = *reinterpret_cast<const float4*>(a.gu_rows + (size_t)n * 2 * I + 4 * j);
    const float4 uv = *reinterpret_cast<const float4*>(a.gu_rows + (size_t)n * 2 * I + I + 4 * j);
    g[0] = gv.x; g[1] = gv.y; g[2] = gv.z; g[3] = gv.w;
    u[0] = uv.x; u[1] = uv.y; u[2] = uv.z; u[3] = uv.w;
  }
  const float rs = __uint_as_float(0x3DB504F3u);
  if (a.gu_out_signs) {  // F17 on the gate/up outputs, per 128-block of g and of u
    fwht128_quad(g, sub);
    fwht128_quad(u, sub);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      g[q] = g[q] * rs;
      u[q] = u[q] * rs;
    }
    flip4(g, a.gu_out_signs, 4 * j);
    flip4(u, a.gu_out_signs, I + 4 * j);
  }
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = g[q] / (1.0f + expf(-g[q])) * u[q];
  flip4(v, a.down_signs, 4 * j);
  fwht128_quad(v, sub);
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = v[q] * rs;
    const float m = fabsf(v[q]);
    amax = fmaxf(amax, m <= 3.4e38f ? m : __builtin_inff());
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  if ((j & 63) == 0) s_red[j >> 6] = amax;
  lds_barrier();
  amax = s_red[0];
  for (int w = 1; w < nw; ++w) amax = fmaxf(amax, s_red[w]);
  const bool finite = amax <= 3.4e38f;
  int ex = 0;
  if (finite && amax > 0.0f) (void)frexpf(amax, &ex);  // amax in [2^(ex - 1), 2^ex)
  const int n_ti = I / 16;
  if constexpr (DECODE) {
    int e = 0;
    if (finite && amax > 0.0f) {
      e = 15 - ex;
      if (ldexpf(amax, e) > 32639.0f) e -= 1;
    }
    int isum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float r = finite ? rintf(ldexpf(v[q], e)) : 0.0f;
      r = fminf(fmaxf(r, -32639.0f), 32639.0f);
      s_x[4 * j + q] = (int)r;
      isum += (int)r;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) isum += __shfl_xor(isum, d, 64);
    if ((j & 63) == 0) s_isum[j >> 6] = isum;
    lds_barrier();
    // dwords 4 j .. 4 j + 3 of the row's operands: half h, tile column c, registers r .. r + 3
    // (register r holds the bytes [v[r + 8], v[r + 8], v[r], v[r]] of the half)
    const int d0 = 4 * j, per_half = I / 2;
    const int h = d0 / per_half, dd = d0 % per_half, c = dd / 8, r0 = dd % 8;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = r0 + q;
      const int x0 = s_x[16 * c + r], x8 = s_x[16 * c + r + 8];
      const int hi0 = (x0 + 128) >> 8, hi8 = (x8 + 128) >> 8;
      const uint32_t b0 = (uint32_t)(h == 0 ? hi0 : x0 - (hi0 << 8)) & 0xFFu;
      const uint32_t b8 = (uint32_t)(h == 0 ? hi8 : x8 - (hi8 << 8)) & 0xFFu;
      w[q] = b8 | (b8 << 8) | (b0 << 16) | (b0 << 24);
    }
    uint4* dst = reinterpret_cast<uint4*>(a.xq + ((size_t)(2 * n + h) * n_ti + c) * 8 + r0);
    *dst = make_uint4(w[0], w[1], w[2], w[3]);
    if (j == 0) {
      int t = 0;
      for (int q = 0; q < nw; ++q) t += s_isum[q];
      a.xsum[n] = t;
      a.xscale[n] = finite ? ldexpf(1.0f, -e) : __builtin_nanf("");
    }
  } else {
    const int e = (finite && amax > 0.0f) ? min(15 - ex, 100) : 0;
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float f = (float)(_Float16)ldexpf(v[q], e);
      s_f[4 * j + q] = f;
      sum += f;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 64);
    if ((j & 63) == 0) s_sum[j >> 6] = sum;
    lds_barrier();
    // words 2 j, 2 j + 1 of the row: tile column c, word r = [lo: x[16 c + r + 8], hi: x[16 c + r]]
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    uint32_t w[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int wd = 2 * j + q, c = wd / 8, r = wd % 8;
      const h2 p = (h2){(_Float16)s_f[16 * c + r + 8], (_Float16)s_f[16 * c + r]};
      w[q] = __builtin_bit_cast(uint32_t, p);
    }
    *reinterpret_cast<uint2*>(a.xp + (size_t)n * n_ti * 8 + 2 * j) = make_uint2(w[0], w[1]);
    if (j == 0) {
      float t = 0.0f;
      for (int q = 0; q < nw; ++q) t += s_sum[q];
      a.rowsum[n] = make_float2(t, finite ? ldexpf(1.0f, -e) : __builtin_nanf(""));
    }
  }
}

}  // namespace

hipError_t launch_ffn_mid(const FfnMidArgs& a, bool decode, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  const int threads = a.I / 4;
  if (decode)
    hipLaunchKernelGGL(ffn_mid_kernel<true>, dim3((unsigned)a.N), dim3(threads), 0, s, a);
  else
    hipLaunchKernelGGL(ffn_mid_kernel<false>, dim3((unsigned)a.N), dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq

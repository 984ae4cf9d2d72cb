// SwiGLU step of the routed expert FFN (gfx950): for every routed slot and intermediate
// channel, h = bf16_rne(silu(g) * u) with silu(g) = g / (1 + e^-g), from the fp32 outputs g and u
// of the gate and up projections (FORMAT F15). Elementwise: four channels per thread, 16-byte
// loads, 8-byte stores.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

__global__ __launch_bounds__(256) void swiglu_kernel(const float4* __restrict__ g,
                                                     const float4* __restrict__ u,
                                                     uint2* __restrict__ h, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 a = g[i], b = u[i];
  const float ga[4] = {a.x, a.y, a.z, a.w}, ua[4] = {b.x, b.y, b.z, b.w};
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float s = ga[j] / (1.0f + expf(-ga[j]));
    r[j] = f32_to_bf16_rne(s * ua[j]);
  }
  h[i] = make_uint2(r[0] | (r[1] << 16), r[2] | (r[3] << 16));
}

}  // namespace

hipError_t launch_swiglu(const float* g, const float* u, uint16_t* h, int64_t n,
                         hipStream_t s) {
  const int64_t n4 = n / 4;  // n is a multiple of 16
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(g), reinterpret_cast<const float4*>(u),
                     reinterpret_cast<uint2*>(h), n4);
  return hipGetLastError();
}

}  // namespace tq

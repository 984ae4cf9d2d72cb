// Second launch of the decode-batch path when the K range is split into S slices: for each
// output, the S slice partials are added in slice order, scaled by acc_scale, corrected by
// offset * rowsum[token] (the trellis byte encoding), then the per-channel scale and the
// gate are applied. Empty slots (-1) give 0; ids outside [-1, E) give NaN and set the
// status bit. With combine, y[t][o] = sum over k = 0..topk-1 (in order) of the slot values.
#include "gemv_common.h"

namespace tq {

namespace {

__device__ __forceinline__ float slot_value(const GemvReduceArgs& a, int slot, int o) {
  const int id = a.ids[slot];
  if (id == -1) return 0.0f;
  if (id < -1 || id >= a.E) {
    set_status(a.status, STATUS_BAD_EXPERT);
    return __builtin_nanf("");
  }
  const size_t stride = (size_t)a.N * a.out;
  const float* p = a.partial + (size_t)slot * a.out + o;
  float sum = p[0];
  for (int s = 1; s < a.S; ++s) sum += p[(size_t)s * stride];
  float val = sum * a.acc_scale;
  if (a.rowsum) val = val - a.offset * a.rowsum[slot / a.topk];
  return gemv_epilogue(a.scales, a.gates, a.out, id, o, slot, val);
}

__global__ __launch_bounds__(256) void gemv_reduce_kernel(GemvReduceArgs a) {
  const int rows = a.combine ? a.N / a.topk : a.N;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rows * a.out) return;
  const int r = (int)(idx / a.out), o = (int)(idx % a.out);
  if (!a.combine) {
    a.y[idx] = slot_value(a, r, o);
    return;
  }
  float acc = 0.0f;
  for (int k = 0; k < a.topk; ++k) acc += slot_value(a, r * a.topk + k, o);
  a.y[idx] = acc;
}

}  // namespace

hipError_t launch_gemv_reduce(const GemvReduceArgs& a, hipStream_t s) {
  const int rows = a.combine ? a.N / a.topk : a.N;
  const int64_t total = (int64_t)rows * a.out;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq

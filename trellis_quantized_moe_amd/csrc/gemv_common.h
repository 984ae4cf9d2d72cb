// Reductions and epilogue shared by the decode-batch (GEMV) kernels.
//
// A GEMV workgroup owns (expert e, group of up to 8 strips = 128 output channels,
// K-slice s). Its four waves hold 16 x 16 accumulator tiles for the same outputs over
// different K ranges; they are added through LDS in wave order. With one slice the
// workgroup applies the epilogue and writes y. With S > 1 slices it stores its slice's
// sums to a partial buffer indexed by flat slot, and a second launch (gemv_reduce) adds
// the S slices in slice order. The launch boundary makes the partials visible; no
// device-wide fence (which would write back and invalidate a whole L2) is needed.
#pragma once

#include "route_scan.h"
#include "tq_device.h"

namespace tq {

constexpr int GEMV_THREADS = 256;

struct GemvCommon {
  const int32_t* ids;
  const float* gates;
  const uint16_t* scales;  // fp16 [E][out] or null (scale 1)
  const float* rowsum;     // [T]: per-token sum the epilogue removes, or null
  float* y;                // per-slot output [N][out] (S == 1)
  float* partial;          // [S][N][out] (S > 1)
  float acc_scale;         // accumulator scale (2^24 for subnormal byte operands, else 1)
  float offset;            // y = acc * acc_scale - offset * rowsum[token]
  int N, E, out, topk, S, groups;
};

__device__ __forceinline__ float gemv_epilogue(const uint16_t* scales, const float* gates, int out,
                                               int e, int o, int slot, float v) {
  float r = v;
  if (scales) r = r * f16_bits_to_f32(scales[(size_t)e * out + o]);
  if (gates) r = r * gates[slot];
  return r;
}

// red: LDS float [4 waves][8 strips][4][64 lanes]. Each wave writes acc, then the sums
// (wave order) go to the partial buffer (S > 1), or, scaled and corrected, through the
// epilogue to y (S == 1).
__device__ inline void gemv_reduce_store(const GemvCommon& c, float* red, const f32x4 acc[8],
                                         const SlotChunk& ch, int e, int grp, int s, int ns) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((w * 8 + s8) * 4 + i) * 64 + lane] = acc[s8][i];
  __syncthreads();
  const int cnt = ch.cnt;
  for (int v = tid; v < ns * 256; v += GEMV_THREADS) {
    const int s8 = v >> 8, i = (v >> 6) & 3, ln = v & 63;
    float sum = red[((0 * 8 + s8) * 4 + i) * 64 + ln];
    sum += red[((1 * 8 + s8) * 4 + i) * 64 + ln];
    sum += red[((2 * 8 + s8) * 4 + i) * 64 + ln];
    sum += red[((3 * 8 + s8) * 4 + i) * 64 + ln];
    const int m = 4 * (ln >> 4) + i;
    if (m < cnt) {
      const int o = grp * 128 + s8 * 16 + (ln & 15);
      const int slot = ch.slots[m];
      if (c.S == 1) {
        float val = sum * c.acc_scale;
        if (c.rowsum) val = val - c.offset * c.rowsum[slot / c.topk];
        c.y[(size_t)slot * c.out + o] = gemv_epilogue(c.scales, c.gates, c.out, e, o, slot, val);
      } else {
        c.partial[((size_t)s * c.N + slot) * c.out + o] = sum;
      }
    }
  }
  __syncthreads();
}

// NaN in this (group, slice)'s outputs of expert e's slots; status bit. With S > 1 the NaN
// goes to the slice's partials, so the reduced outputs are NaN too.
__device__ inline void gemv_bad_unit(const GemvCommon& c, SlotChunk& ch, uint32_t* status,
                                     int e, int grp, int s, int ns) {
  int pos = 0;
  while (true) {
    collect_slots(c.ids, c.N, e, pos, ch);
    if (ch.cnt == 0) break;
    pos = ch.next;
    for (int v = threadIdx.x; v < ch.cnt * ns * 16; v += GEMV_THREADS) {
      const int m = v / (ns * 16), o = grp * 128 + v % (ns * 16);
      float* dst = c.S == 1 ? c.y + (size_t)ch.slots[m] * c.out + o
                            : c.partial + ((size_t)s * c.N + ch.slots[m]) * c.out + o;
      *dst = __builtin_nanf("");
    }
    if (threadIdx.x == 0) set_status(status, STATUS_BAD_UNIT);
    __syncthreads();
    if (pos >= c.N) break;
  }
}

struct GemvReduceArgs {
  const int32_t* ids;
  const float* partial;    // [S][N][out]
  const uint16_t* scales;  // or null
  const float* gates;      // or null
  const float* rowsum;     // [T] or null
  float* y;                // [N][out], or [T][out] when combine
  uint32_t* status;
  float acc_scale, offset;
  int N, E, out, topk, S, combine;
};

hipError_t launch_gemv_reduce(const GemvReduceArgs& a, hipStream_t s);

}  // namespace tq

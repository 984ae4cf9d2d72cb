// Reductions and epilogue shared by the decode-batch (GEMV) kernels.
//
// A GEMV workgroup owns (expert e, group of up to 8 strips = 128 output channels,
// K-slice s). Its four waves hold 16 x 16 accumulator tiles for the same outputs over
// different K ranges; they are added through LDS in wave order. With S > 1 slices the
// workgroup stores its slice's sums to a partial buffer indexed by flat slot, and the
// last workgroup of (e, group) to arrive (device-scope counter) adds the S slices in slice
// order and applies the epilogue. The counter is reset by that workgroup, so the workspace
// is left zeroed for the next call.
#pragma once

#include "route_scan.h"
#include "tq_device.h"

namespace tq {

constexpr int GEMV_THREADS = 256;

struct GemvCommon {
  const int32_t* ids;
  const float* gates;
  const uint16_t* scales;  // fp16 [E][out] or null (scale 1)
  float* y;                // per-slot output [N][out]
  float* partial;          // [S][N][out]
  int32_t* counters;       // [E][groups]
  int N, E, out, topk, S, groups;
};

__device__ __forceinline__ float gemv_epilogue(const GemvCommon& c, int e, int o, int slot,
                                               float v) {
  float r = v;
  if (c.scales) r = r * f16_bits_to_f32(c.scales[(size_t)e * c.out + o]);
  if (c.gates) r = r * c.gates[slot];
  return r;
}

// red: LDS float [4 waves][8 strips][4][64 lanes]. Each wave writes acc, then the sums
// (wave order) minus offset * rowsum[m] go to y (S == 1) or to the partial buffer.
__device__ inline void gemv_reduce_store(const GemvCommon& c, float* red, const f32x4 acc[8],
                                         const SlotChunk& ch, const float* rowsum, float offset,
                                         int e, int grp, int s, int ns) {
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
      const float val = rowsum ? sum - offset * rowsum[m] : sum;
      const int o = grp * 128 + s8 * 16 + (ln & 15);
      const int slot = ch.slots[m];
      if (c.S == 1)
        c.y[(size_t)slot * c.out + o] = gemv_epilogue(c, e, o, slot, val);
      else
        c.partial[((size_t)s * c.N + slot) * c.out + o] = val;
    }
  }
  __syncthreads();
}

// Called by every workgroup of (e, grp) that found slots, after its last chunk. Returns
// after the last arriving workgroup has written the outputs.
__device__ inline void gemv_finish(const GemvCommon& c, SlotChunk& ch, int* last_flag, int e,
                                   int grp, int ns) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = atomicAdd(&c.counters[e * c.groups + grp], 1);
    *last_flag = (old == c.S - 1);
  }
  __syncthreads();
  if (!*last_flag) return;
  __threadfence();
  const int width = ns * 16;
  int pos = 0;
  while (true) {
    collect_slots(c.ids, c.N, e, pos, ch);
    const int cnt = ch.cnt;
    if (cnt == 0) break;
    pos = ch.next;
    for (int v = threadIdx.x; v < cnt * width; v += GEMV_THREADS) {
      const int m = v / width, o = grp * 128 + v % width;
      const int slot = ch.slots[m];
      float sum = 0.0f;
      for (int s = 0; s < c.S; ++s) sum += c.partial[((size_t)s * c.N + slot) * c.out + o];
      c.y[(size_t)slot * c.out + o] = gemv_epilogue(c, e, o, slot, sum);
    }
    __syncthreads();
    if (pos >= c.N) break;
  }
  if (threadIdx.x == 0) c.counters[e * c.groups + grp] = 0;
}

// NaN in every output of expert e's slots for this group; status bit 2.
__device__ inline void gemv_bad_unit(const GemvCommon& c, SlotChunk& ch, uint32_t* status,
                                     int e, int grp, int ns) {
  int pos = 0;
  while (true) {
    collect_slots(c.ids, c.N, e, pos, ch);
    if (ch.cnt == 0) break;
    pos = ch.next;
    for (int v = threadIdx.x; v < ch.cnt * ns * 16; v += GEMV_THREADS) {
      const int m = v / (ns * 16), o = grp * 128 + v % (ns * 16);
      c.y[(size_t)ch.slots[m] * c.out + o] = __builtin_nanf("");
    }
    if (threadIdx.x == 0) set_status(status, STATUS_BAD_UNIT);
    __syncthreads();
    if (pos >= c.N) break;
  }
}

}  // namespace tq

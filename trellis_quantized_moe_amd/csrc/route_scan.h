// Per-expert slot collection for the decode-batch kernels.
//
// A decode batch routes a few tokens to each expert, so each workgroup finds its own
// expert's (token, slot) pairs by scanning the routes itself instead of waiting for a
// separate bucketing pass: a block-wide stream compaction in ascending flat index, which
// is exactly the order a stable counting sort by expert would give (FORMAT F14).
#pragma once

#include "tq_device.h"

namespace tq {

struct SlotChunk {
  int slots[16];   // flat slot indices t * topk + k, ascending
  int cnt;         // valid entries
  int next;        // where the next scan resumes
  int wave_tot[4];
};

// Collect up to 16 slots with ids[slot] == e from position `pos` on. 256 threads; every
// thread must call it. On return (after a barrier) ch.cnt, ch.slots, ch.next are valid.
__device__ inline void collect_slots(const int32_t* __restrict__ ids, int N, int e, int pos,
                                     SlotChunk& ch) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) {
    ch.cnt = 0;
    ch.next = N;
  }
  __syncthreads();
  for (int base = pos; base < N; base += 1024) {
    const int i0 = base + 4 * tid;
    int m[4];
    int c = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = i0 + k;
      m[k] = (idx < N) && (ids[idx] == e);
      c += m[k];
    }
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    if (lane == 63) ch.wave_tot[wid] = incl;
    __syncthreads();
    int wpre = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int t = ch.wave_tot[w];
      wpre += (w < wid) ? t : 0;
      total += t;
    }
    const int have = ch.cnt;
    const int need = 16 - have;
    int r = wpre + incl - c;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (m[k]) {
        if (r < need) {
          ch.slots[have + r] = i0 + k;
          if (r == need - 1) ch.next = i0 + k + 1;
        }
        ++r;
      }
    }
    __syncthreads();
    if (total >= need) {
      if (tid == 0) ch.cnt = 16;
      __syncthreads();
      break;
    }
    if (tid == 0) ch.cnt = have + total;
    __syncthreads();
  }
}

// Slots with id -1 get zero outputs; ids outside [-1, E) get NaN and set the status bit.
// One workgroup of 256 threads scans all N slots (decode batches: N is small).
__device__ inline void special_slots(const int32_t* __restrict__ ids, int N, int E, int out,
                                     float* __restrict__ y, uint32_t* status) {
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    const int id = ids[i];
    if (id >= 0 && id < E) continue;
    const float v = (id == -1) ? 0.0f : __builtin_nanf("");
    if (id != -1) set_status(status, STATUS_BAD_EXPERT);
    float4* row = reinterpret_cast<float4*>(y + (size_t)i * out);
    for (int o = 0; o < out / 4; ++o) row[o] = make_float4(v, v, v, v);
  }
}

}  // namespace tq

// Decode-batch plan: which workgroup streams which part of which routed expert.
//
// The decode-batch path runs three launches:
//   1. plan + prep (gemv_plan.hip): one block buckets the routes by expert (slot lists,
//      the active experts in ascending id order, a cost prefix over them, per-slot records,
//      and the start of every workgroup's range); the other blocks prepare activations;
//   2. the grouped GEMV: exactly as many workgroups as the GPU holds at once (G), each
//      streaming a contiguous, equal share of the active experts' cost;
//   3. the piece reduction (gemv_reduce.hip): per slot, the partial sums of the pieces an
//      expert was split into, added in piece order, then the epilogue (and the combine).
//
// Work is counted in units: one unit is 128 output channels (a group of 8 strips) by 256
// inputs. An expert has U = groups * Q units (Q = in / 256), group-major. A unit of a
// trellis expert costs K (its bytes are proportional to K); an MXFP4 unit costs 1. With
// C = the total cost of the active experts, the first G' = min(G, C / largest unit cost)
// workgroups get work (so each owns at least one unit), workgroup w < G' owns the cost range
// [c0(w), c0(w + 1)), c0(w) = floor(w * C / G'), and every unit whose first cost lies in it.
// A workgroup's share of one expert's group is a "piece"; piece p of (expert, group) is the
// share of workgroup owner(group start) + p. Pieces are summed in that order, so results
// are independent of timing.
#pragma once

#include "tq_device.h"

namespace tq {

// One active expert (index a in the active list).
struct alignas(16) PlanRec {
  int32_t e;      // expert id
  int32_t start;  // first entry of its slots in the slot list
  int32_t cnt;    // number of slots routed to it
  int32_t k;      // cost of one unit
  int64_t off;    // byte offset of its unit
  int32_t p0;     // cost prefix: the expert's first cost
  int32_t pad;
};

// Per-slot record for the reduction: {expert id, p0, k, 0}, or code in .x:
constexpr int SLOT_EMPTY = -1;     // id -1: output 0
constexpr int SLOT_BAD_ID = -2;    // id outside [-1, E): NaN
constexpr int SLOT_BAD_UNIT = -3;  // expert with a bad width byte or offset: NaN

constexpr int PLAN_MAX_E = 4096;
constexpr int PLAN_THREADS = 1024;
constexpr int GEMV_MAX_G = 4096;   // bound on the GEMV grid (desc buffer size)

// First cost owned by workgroup w.
__device__ __forceinline__ int64_t plan_c0(int w, int64_t C, int G) {
  return (int64_t)w * C / G;
}
// The workgroup whose range holds cost c (0 <= c < C): the largest w with c0(w) <= c.
__device__ __forceinline__ int plan_owner(int64_t c, int64_t C, int G) {
  const int64_t w = ((c + 1) * G - 1) / C;
  return (int)(w < G - 1 ? w : G - 1);
}

}  // namespace tq

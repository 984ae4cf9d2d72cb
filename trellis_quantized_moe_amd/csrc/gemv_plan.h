// Decode-batch plan: which wave streams which part of which routed expert.
//
// The decode-batch path runs three launches:
//   1. plan + prep (gemv_plan.hip): one block buckets the routes by expert (slot lists,
//      the active experts in ascending id order, per-slot records) and splits the work
//      among the GEMV's waves; the other blocks prepare activations;
//   2. the grouped GEMV: single-wave workgroups, each streaming one piece;
//   3. the piece reduction (gemv_reduce.hip): per slot, the partial sums of the pieces its
//      expert was split into, added in piece order, then the epilogue (and the combine).
//
// Work is counted in steps: one step is 64 inputs of one group of 128 output channels, so
// a group has S = in / 64 steps. A step of a trellis expert of width K costs K (its bytes
// are proportional to K); an MXFP4 step costs 1. An expert's routed slots come in chunks of
// R (the rows one wave's matrix-core operations hold: 8 tokens for trellis, 16 for the
// E8M0-scaled stores), and each chunk of each group is its own work. Every active expert's
// group and chunk is split into W(k) pieces of consecutive steps (W depends only on the
// expert's cost k), piece j taking
// steps floor(j S / W) .. floor((j + 1) S / W) - 1, and every piece is one wave's whole
// work: no wave crosses from one expert or group into another, so a wave's load stream
// never restarts, and the pieces of a group differ by at most one step. W(k) =
// ceil(S / floor(T / k)) for the smallest per-wave cost bound T >= 4 * kmax (kmax the
// largest active cost) whose total number of waves fits the wave target (or the number of
// active groups and chunks, when that is larger); T >= 4 kmax keeps W(k) <= S / 4 =
// in / 256. A slot's pieces are the W(k) pieces of its group and chunk.
// Pieces are summed in piece order, so results are independent of timing, and the split
// depends only on which experts are active, never on the order of the tokens.
#pragma once

#include "tq_device.h"

namespace tq {

// One active expert (index a in the active list).
struct alignas(16) PlanRec {
  int32_t e;      // expert id
  int32_t start;  // first entry of its slots in the slot list
  int32_t cnt;    // number of slots routed to it
  int32_t k;      // cost of one step
  int64_t off;    // byte offset of its unit
  int32_t wave0;  // first wave of its pieces
  int32_t np;     // pieces per group, W(k)
};

// desc[w], the piece of wave w (int4): {active expert index, or -1 for no work; group |
// chunk << 16 (the chunk of the expert's slot list: slots c R .. c R + R - 1); piece index;
// its steps s0 .. s1 - 1 packed as s0 | s1 << 16}.

// Per-slot record for the reduction: {expert id, pieces per group, k, 0}, or code in .x:
constexpr int SLOT_EMPTY = -1;     // id -1: output 0
constexpr int SLOT_BAD_ID = -2;    // id outside [-1, E): NaN
constexpr int SLOT_BAD_UNIT = -3;  // expert with a bad width byte or offset: NaN

constexpr int PLAN_MAX_E = 4096;
constexpr int PLAN_THREADS = 1024;
// An expert with at most PLAN_OWN_PIECES pieces has them written by its own thread of the
// plan; larger ones (at most GEMV_MAX_G / PLAN_OWN_PIECES of them) by the whole block.
constexpr int PLAN_OWN_PIECES = 32;
// Bound on the GEMV grid (desc buffer size). It keeps a chunk index below 2^15 and the
// plan's per-cost chunk counts below 2^16 (the host checks groups * (E + N / R) against it).
constexpr int GEMV_MAX_G = 32768;
constexpr int PLAN_MAX_BIG = GEMV_MAX_G / PLAN_OWN_PIECES;
// Waves per compute unit the plan aims for, for waves of 8 strips (2 per SIMD). The trellis
// decode is bound by instruction issue: fewer, longer pieces spend less on each wave's setup
// and on the partial sums that the reduction reads, and the trellis GEMV doubles the waves
// by splitting each piece's strips over two of them (4 per SIMD). The MXFP4 GEMV, which
// waits on memory more than it issues, aims for 3 per SIMD.
constexpr int GEMV_TARGET_PER_CU = 8;

}  // namespace tq

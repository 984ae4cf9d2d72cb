// Shared pieces of the single-wave decode-batch GEMVs (trellis_gemv.hip, mxfp4.hip): buffer
// resources for the streaming loads, and the plan's records and pieces read through the
// scalar cache.
#pragma once

#include "gemv_plan.h"

namespace tq {

// The streaming loads address memory as a scalar buffer resource + one per-lane byte offset
// (fixed for the whole piece) + a scalar offset for the step and strip, so a load costs no
// vector address arithmetic and no 64-bit address registers. A load whose offset lies
// past the resource's size returns 0.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Plan records and pieces are read through the scalar cache (constant address space): their
// waits then count on the scalar counter and never on the vector-memory counter that the
// streaming loads keep busy.
typedef const __attribute__((address_space(4))) PlanRec* ConstRec;
__device__ __forceinline__ PlanRec load_rec(const PlanRec* rec, int i) {
  const ConstRec p = (ConstRec)rec + i;
  PlanRec r;
  r.e = p->e;
  r.start = p->start;
  r.cnt = p->cnt;
  r.k = p->k;
  r.off = p->off;
  r.wave0 = 0;
  r.np = 0;
  return r;
}

typedef const __attribute__((address_space(4))) int4* ConstDesc;

// The piece of wave w (see gemv_plan.h): false when the wave has none.
struct Piece {
  int ai, grp, chunk, idx, s0, s1;
};
__device__ __forceinline__ bool load_piece(const int4* desc, int w, Piece& p) {
  const ConstDesc dp = (ConstDesc)desc + w;
  p.ai = dp->x;
  if (p.ai < 0) return false;
  const int gc = dp->y;
  p.grp = gc & 0xFFFF;
  p.chunk = gc >> 16;
  p.idx = dp->z;
  const int span = dp->w;
  p.s0 = span & 0xFFFF;
  p.s1 = span >> 16;
  return true;
}

}  // namespace tq

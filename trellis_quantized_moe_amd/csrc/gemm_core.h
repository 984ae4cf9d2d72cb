// Pieces shared by the prefill grouped GEMMs (gfx950): the work-unit order of the grid,
// buffer resources, and the barrier and waits of the LDS rings that loads writing LDS fill.
#pragma once

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

// The work unit of this workgroup. Consecutive workgroups land on the 8 XCDs in turn
// (workgroup b on XCD b % 8), so the grid is read as 8 interleaved streams and stream x
// takes a contiguous range of the n_items * groups units: the units of one expert, which
// read the same weight unit, then share one L2. The grid has gemm_grid() workgroups.
__device__ inline bool gemm_unit(const int32_t* n_items, int groups, int* item, int* grp) {
  const int units = *n_items * groups;
  const int per = (units + 7) >> 3;
  const int j = blockIdx.x >> 3;
  const int u = (blockIdx.x & 7) * per + j;
  if (j >= per || u >= units) return false;
  *item = u / groups;
  *grp = u % groups;
  return true;
}
inline int gemm_grid(int max_items, int groups) { return (max_items * groups + 7) & ~7; }

// ---- LDS rings filled by loads that write LDS ----------------------------------------------
typedef __attribute__((address_space(3))) void* LdsPtr;

// s_waitcnt with only the vector-memory count limited (gfx9 encoding: vmcnt in bits 3:0
// and 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier with no memory fence. The loads that write LDS count on the vector
// memory counter, so an LDS fence would wait for all of them, including the ones meant to
// stay in flight; the waits are explicit instead (wait_vmcnt before the barrier). The wave's
// own LDS reads are waited for (lgkmcnt(0)) and no instruction moves across the barrier, so
// no wave can still be reading a stage when another starts refilling it after the barrier.
__device__ __forceinline__ void bare_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unlimited
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ---- buffer loads ------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t GemmRsrc;
__device__ __forceinline__ GemmRsrc gemm_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

}  // namespace tq

// Prefill work-item core shared by the trellis and MXFP4 grouped GEMMs (gfx950).
//
// One workgroup (4 waves, 2 x 2 over a 128 x 128 output tile) multiplies up to 128 routed
// rows of one expert by one group of up to 128 output channels over the whole K range, in
// steps of 32 inputs:
//   - a B producer (format-specific) decodes the step's 32 x 128 weights into operand
//     pairs, each thread one run of 16 inputs of one output channel;
//   - each thread copies 16 activations of one routed row into the A tile;
//   - each wave runs its 4 x 4 block of 16x16x32 bf16 matrix-core operations.
// Two LDS buffers alternate: while the waves multiply step kk, they decode and stage step
// kk + 1 into the other buffer, from registers loaded GEMM_RING steps earlier. Each output
// is written once by the workgroup owning its row.
#pragma once

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

constexpr int GEMM_THREADS = 256;
constexpr int GEMM_KS = 32;          // inputs per step
constexpr int GEMM_LDS_STRIDE = 40;  // bf16 per LDS row (32 + 8 padding against bank conflicts)

// 16-byte alignment lets every operand access be one ds_read_b128 / ds_write_b128 (with
// 2-byte alignment the compiler splits them into 32-bit accesses).
struct GemmShared {
  alignas(16) uint16_t a[2][GEMM_MT * GEMM_LDS_STRIDE];
  alignas(16) uint16_t b[2][128 * GEMM_LDS_STRIDE];
  int slot[GEMM_MT];
};

struct GemmItem {
  const void* x;           // bf16 x [T][in]
  uint32_t x_bytes;        // size of x in bytes (< 2^31)
  const float* gates;
  const uint16_t* scales;  // fp16 per output channel of this expert, or null
  float* y;
  int in, out, topk, grp, nrows, ns;
};

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

// Load slot indices of the item's rows into LDS (all threads; ends with a barrier).
__device__ inline void gemm_load_slots(GemmShared& sh, const int32_t* pairs, int row0,
                                       int nrows) {
  for (int m = threadIdx.x; m < GEMM_MT; m += GEMM_THREADS)
    sh.slot[m] = m < nrows ? pairs[row0 + m] : 0;
  lds_barrier();
}

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

// Producer interface (format-specific B operand, bf16 in natural input order):
//   typename Raw                  this thread's undecoded data of one step (registers)
//   void load(int kk, Raw& r)     issues the loads of step kk (any kk < steps)
//   void decode(const Raw& r, uint32_t nat[8])
//                                 the thread's run as 8 dwords of operand pairs
//   int o, h                      the run: output channel o (0..127 within the group),
//                                 inputs 32 kk + 16 h .. + 15
//
// The loads of step kk + GEMM_RING are issued as soon as step kk's raw data has been
// consumed, into the same registers, so GEMM_RING steps of loads are in flight while the
// matrix cores work; every load is unconditional (indices clamped to valid steps), so each
// path through the loop leaves the same loads in flight.
constexpr int GEMM_RING = 4;

template <class Producer>
__device__ __forceinline__ void gemm_item(const GemmItem& it, GemmShared& sh, Producer& prod) {
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int wm = w >> 1, wn = w & 1;
  const int nsteps = it.in / GEMM_KS;  // a multiple of 8 (in is a multiple of 256)
  // A staging: thread (a_m, a_h) copies inputs 16 a_h .. + 15 of the step for routed row
  // a_m. Both activation layouts keep these 16 inputs in 32 contiguous bytes at the same
  // offset. Rows past the item's count load from beyond the buffer's end (x_bytes < 2^31):
  // the hardware returns zeros without a memory access, and those rows are never stored.
  const int a_m = tid >> 1, a_h = tid & 1;
  const GemmRsrc ra = gemm_rsrc(it.x, it.x_bytes);
  const uint32_t a_vo =
      a_m < it.nrows ? 2u * (uint32_t)((size_t)(sh.slot[a_m] / it.topk) * it.in + 16 * a_h)
                     : 0x80000000u;

  typename Producer::Raw raw[GEMM_RING];
  u32x4 xa0[GEMM_RING], xa1[GEMM_RING];
  auto load_step = [&](int slot, int kk) {
    const int k = kk < nsteps ? kk : nsteps - 1;
    prod.load(k, raw[slot]);
    xa0[slot] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_vo, 64u * k, 0);
    xa1[slot] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_vo + 16, 64u * k, 0);
  };
  // decodes the slot into LDS buffer buf, then reuses its registers for step kk_next. The
  // stores come first: the new loads then write the very registers just read, and every
  // ring slot stays in the same registers from one loop iteration to the next (a slot
  // moved between registers would have to wait for all loads in flight).
  auto stage = [&](int slot, int buf, int kk_next) {
    uint32_t nat[8];
    prod.decode(raw[slot], nat);
    const u32x4 v0 = xa0[slot], v1 = xa1[slot];
    uint4* da = reinterpret_cast<uint4*>(&sh.a[buf][a_m * GEMM_LDS_STRIDE + 16 * a_h]);
    da[0] = make_uint4(v0.x, v0.y, v0.z, v0.w);
    da[1] = make_uint4(v1.x, v1.y, v1.z, v1.w);
    uint4* db = reinterpret_cast<uint4*>(&sh.b[buf][prod.o * GEMM_LDS_STRIDE + 16 * prod.h]);
    db[0] = make_uint4(nat[0], nat[1], nat[2], nat[3]);
    db[1] = make_uint4(nat[4], nat[5], nat[6], nat[7]);
    __builtin_amdgcn_sched_barrier(0);
    load_step(slot, kk_next);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  int mblocks = (it.nrows - 64 * wm + 15) / 16;
  mblocks = mblocks < 0 ? 0 : (mblocks > 4 ? 4 : mblocks);
  int nblocks = it.ns - 4 * wn;
  nblocks = nblocks < 0 ? 0 : (nblocks > 4 ? 4 : nblocks);

#pragma unroll
  for (int d = 0; d < GEMM_RING; ++d) load_step(d, d);
  stage(0, 0, GEMM_RING);
  lds_barrier();
  for (int kk = 0; kk < nsteps; kk += GEMM_RING) {
#pragma unroll
    for (int d = 0; d < GEMM_RING; ++d) {
      const int step = kk + d;
      const int buf = d & 1;  // = step & 1 (GEMM_RING is even)
      // the next step goes into the other buffer (after the last step: harmless, unread)
      stage((d + 1) % GEMM_RING, buf ^ 1, step + 1 + GEMM_RING);
      u32x4 bop[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        bop[nb] = *reinterpret_cast<const u32x4*>(
            &sh.b[buf][(64 * wn + 16 * nb + n) * GEMM_LDS_STRIDE + 8 * g]);
      // Row blocks past the item's rows are skipped (a wave-uniform branch). Column blocks
      // past the group's strips are multiplied anyway: their B rows hold a copy of the last
      // strip and their results are never stored.
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < mblocks) {
          const u32x4 aop = *reinterpret_cast<const u32x4*>(
              &sh.a[buf][(64 * wm + 16 * mb + n) * GEMM_LDS_STRIDE + 8 * g]);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_bf16(aop, bop[nb], acc[mb][nb]);
        }
      }
      lds_barrier();
    }
  }

#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      if (mb < mblocks && nb < nblocks) {
        const int o = it.grp * 128 + 64 * wn + 16 * nb + n;
        const float sc = it.scales ? f16_bits_to_f32(it.scales[o]) : 1.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 64 * wm + 16 * mb + 4 * g + i;
          if (row < it.nrows) {
            const int slot = sh.slot[row];
            float v = acc[mb][nb][i];
            v = v * sc;
            if (it.gates) v = v * it.gates[slot];
            it.y[(size_t)slot * it.out + o] = v;
          }
        }
      }
    }
  }
}

// NaN in every output of the item (bad unit descriptor).
__device__ inline void gemm_item_nan(const GemmItem& it, GemmShared& sh) {
  for (int v = threadIdx.x; v < it.nrows * it.ns * 16; v += GEMM_THREADS) {
    const int m = v / (it.ns * 16), o = it.grp * 128 + v % (it.ns * 16);
    it.y[(size_t)sh.slot[m] * it.out + o] = __builtin_nanf("");
  }
}

}  // namespace tq

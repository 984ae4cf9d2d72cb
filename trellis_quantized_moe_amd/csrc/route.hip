// Route bucketing for the prefill path (gfx950): a stable counting sort of the flat slot
// indices t * topk + k by expert id (FORMAT F11, F14), in three launches:
//   1. rank:    one wave per block of 1024 slots; slots are taken 64 at a time in index
//               order, lanes holding the same expert are found with one ballot per id bit,
//               and each slot's rank among the block's earlier slots of its expert comes
//               from a per-expert running count in LDS. The block's counts go to hist.
//   2. scan:    one workgroup turns hist into per-(block, expert) bases, per-expert counts
//               and offsets, and the list of (expert, row0, nrows) work items.
//   3. scatter: pairs[base[block][e] + rank] = slot; empty (-1) slots get zero outputs and
//               invalid ids NaN outputs plus a status bit.
// No step depends on timing, so the order is the same on every run.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr int RANK_BLOCK = ROUTE_CHUNK;  // slots per rank block (one wave, rounds of 64)
constexpr int MAX_E = 4096;

__global__ __launch_bounds__(64) void route_rank_kernel(const int32_t* __restrict__ ids, int N,
                                                        int E, int idbits,
                                                        int32_t* __restrict__ rank,
                                                        int32_t* __restrict__ hist) {
  __shared__ int cnt[MAX_E];
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  for (int round = 0; round < RANK_BLOCK / 64; ++round) {
    const int i = b * RANK_BLOCK + round * 64 + lane;
    const int id = i < N ? ids[i] : -1;
    const bool valid = id >= 0 && id < E;
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < idbits; ++bit) {
      const bool on = (id >> bit) & 1;
      const uint64_t bb = __ballot(on);
      m &= on ? bb : ~bb;
    }
    const int r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    const int size = __popcll(m);
    int base = 0;
    if (valid) base = cnt[id];
    __builtin_amdgcn_wave_barrier();
    if (valid && r == 0) cnt[id] = base + size;
    __builtin_amdgcn_wave_barrier();
    if (i < N) rank[i] = valid ? base + r : -1;
  }
  __syncthreads();
  for (int e = lane; e < E; e += 64) hist[(size_t)b * E + e] = cnt[e];
}

// Exclusive block scan of one int per thread (1024 threads); returns the prefix and
// stores the total in *total.
__device__ int block_scan_1024(int v, int* wave_sums, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  if (lane == 63) wave_sums[w] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int k = 0; k < 16; ++k) {
      const int t = wave_sums[k];
      wave_sums[k] = run;
      run += t;
    }
    *total = run;
  }
  __syncthreads();
  const int res = wave_sums[w] + incl - v;
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(1024) void route_scan_kernel(RouteArgs a) {
  __shared__ int wave_sums[16];
  __shared__ int total;
  __shared__ int carry[2];
  const int tid = threadIdx.x;
  if (tid == 0) {
    carry[0] = 0;
    carry[1] = 0;
  }
  __syncthreads();
  // per expert: count, then offsets (exclusive scan) and item bases, 1024 experts a pass
  for (int e0 = 0; e0 < a.E; e0 += 1024) {
    const int e = e0 + tid;
    int c = 0;
    if (e < a.E)
      for (int b = 0; b < a.blocks; ++b) c += a.hist[(size_t)b * a.E + e];
    const int ni = a.items ? (c + a.item_rows - 1) / a.item_rows : 0;
    const int off = block_scan_1024(c, wave_sums, &total) + carry[0];
    const int tc = total;
    const int ib = block_scan_1024(ni, wave_sums, &total) + carry[1];
    const int ti = total;
    if (e < a.E) {
      a.counts[e] = c;
      a.offsets[e] = off;
      int run = off;
      for (int b = 0; b < a.blocks; ++b) {
        const int h = a.hist[(size_t)b * a.E + e];
        a.hist[(size_t)b * a.E + e] = run;
        run += h;
      }
      if (a.items) {
        for (int k = 0; k < ni; ++k) {
          const int r0 = k * a.item_rows;
          const int rows = min(a.item_rows, c - r0);
          reinterpret_cast<int4*>(a.items)[ib + k] = make_int4(e, off + r0, rows, 0);
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      carry[0] += tc;
      carry[1] += ti;
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.offsets[a.E] = carry[0];
    if (a.n_items) *a.n_items = carry[1];
  }
}

__global__ __launch_bounds__(256) void route_scatter_kernel(RouteArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.N) return;
  const int id = a.ids[i];
  if (id >= 0 && id < a.E) {
    const int b = i / RANK_BLOCK;
    a.pairs[a.hist[(size_t)b * a.E + id] + a.rank[i]] = i;
    return;
  }
  if (id != -1) set_status(a.status, STATUS_BAD_EXPERT);
  if (a.y_special) {
    const float v = (id == -1) ? 0.0f : __builtin_nanf("");
    float4* row = reinterpret_cast<float4*>(a.y_special + (size_t)i * a.out);
    for (int o = 0; o < a.out / 4; ++o) row[o] = make_float4(v, v, v, v);
  }
}

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ slots,
                                                      float* __restrict__ y, int64_t T,
                                                      int topk, int out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * out) return;
  const int64_t t = idx / out;
  const int o = (int)(idx % out);
  const float* src = slots + (size_t)t * topk * out + o;
  float acc = 0.0f;
  for (int k = 0; k < topk; ++k) acc += src[(size_t)k * out];
  y[idx] = acc;
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n,
                                                       int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  int idbits = 1;
  while ((1 << idbits) < a.E) ++idbits;
  hipLaunchKernelGGL(route_rank_kernel, dim3(a.blocks), dim3(64), 0, s, a.ids, (int)a.N, a.E,
                     idbits, a.rank, a.hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, s, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)((a.N + 255) / 256)), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_combine(const float* slots, float* y, int64_t T, int topk, int out,
                          hipStream_t s) {
  const int64_t total = T * out;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     slots, y, T, topk, out);
  return hipGetLastError();
}

}  // namespace tq

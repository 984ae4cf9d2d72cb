// Route bucketing for the prefill path (gfx950): a stable counting sort of the flat slot
// indices t * topk + k by expert id (FORMAT F11, F14), in three launches:
//   1. rank:    blocks of ROUTE_CHUNK slots, four waves each; every wave ranks its quarter
//               64 slots at a time in index order (lanes holding the same expert are found
//               with one ballot per id bit, counts run in LDS), then the block adds the
//               earlier waves' counts. The block's counts go to hist.
//   2. scan:    one workgroup turns hist into per-(block, expert) bases, per-expert counts
//               and offsets, and the list of (expert, row0, nrows) work items.
//   3. scatter: pairs[base[block][e] + rank] = slot; empty (-1) slots get zero outputs and
//               invalid ids NaN outputs plus a status bit.
// No step depends on timing, so the order is the same on every run.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr int RANK_BLOCK = ROUTE_CHUNK;        // slots per rank block
constexpr int RANK_WAVES = 4;                  // waves per rank block
constexpr int RANK_ROUNDS = RANK_BLOCK / (64 * RANK_WAVES);  // 64-slot rounds per wave
constexpr int MAX_E = 4096;

// Wave w of rank block b ranks slots b * RANK_BLOCK + w * (RANK_BLOCK / RANK_WAVES) .. in
// rounds of 64: the lanes holding the same expert are found with one ballot per id bit, and a
// slot's rank among the wave's earlier slots of its expert comes from the wave's running count
// in LDS. The block then turns the per-wave counts into per-wave bases (exclusive prefix over
// the waves, in order), adds them, and writes its per-expert totals to hist.
__global__ __launch_bounds__(64 * RANK_WAVES) void route_rank_kernel(
    const int32_t* __restrict__ ids, int N, int E, int idbits, int32_t* __restrict__ rank,
    int32_t* __restrict__ hist) {
  __shared__ int cnt[RANK_WAVES][MAX_E];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const int first = b * RANK_BLOCK + w * (RANK_BLOCK / RANK_WAVES);
  // all of the wave's ids are loaded first, so their latencies overlap
  int idv[RANK_ROUNDS], rk[RANK_ROUNDS];
#pragma unroll
  for (int round = 0; round < RANK_ROUNDS; ++round) {
    const int i = first + round * 64 + lane;
    idv[round] = i < N ? ids[i] : -1;
  }
  for (int e = lane; e < E; e += 64) cnt[w][e] = 0;
  __syncthreads();
#pragma unroll
  for (int round = 0; round < RANK_ROUNDS; ++round) {
    const int id = idv[round];
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
    if (valid) base = cnt[w][id];
    __builtin_amdgcn_wave_barrier();
    if (valid && r == 0) cnt[w][id] = base + size;
    __builtin_amdgcn_wave_barrier();
    rk[round] = base + r;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 64 * RANK_WAVES) {
    int run = 0;
#pragma unroll
    for (int v = 0; v < RANK_WAVES; ++v) {
      const int c = cnt[v][e];
      cnt[v][e] = run;
      run += c;
    }
    hist[(size_t)b * E + e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int round = 0; round < RANK_ROUNDS; ++round) {
    const int i = first + round * 64 + lane;
    const int id = idv[round];
    if (i < N) rank[i] = (id >= 0 && id < E) ? cnt[w][id] + rk[round] : -1;
  }
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

// Thread e reads its column of hist (the count of expert e in each rank block) in batches
// of SCAN_BATCH independent loads, once for the count and once more for the bases. The loads
// take one per-thread offset (4 e) and a scalar one per block, so a batch in flight costs
// one register per load.
constexpr int SCAN_BATCH = 32;

__device__ __forceinline__ void hist_batch(__amdgpu_buffer_rsrc_t rh, int E, int e, int b0,
                                           int blocks, int t[SCAN_BATCH]) {
#pragma unroll
  for (int j = 0; j < SCAN_BATCH; ++j)
    t[j] = b0 + j < blocks
               ? (int)__builtin_amdgcn_raw_buffer_load_b32(rh, 4u * e, 4u * (uint32_t)((b0 + j) * E), 0)
               : 0;
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
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      a.hist, (short)0, (int)((size_t)a.blocks * a.E * 4), 0x00020000);
  // per expert: count, then offsets (exclusive scan) and item bases, 1024 experts a pass
  for (int e0 = 0; e0 < a.E; e0 += 1024) {
    const int e = e0 + tid;
    const bool mine = e < a.E;
    int c = 0;
    if (mine) {
      for (int b0 = 0; b0 < a.blocks; b0 += SCAN_BATCH) {
        int t[SCAN_BATCH];
        hist_batch(rh, a.E, e, b0, a.blocks, t);
#pragma unroll
        for (int j = 0; j < SCAN_BATCH; ++j) c += t[j];
      }
    }
    const int ni = a.items ? (c + a.item_rows - 1) / a.item_rows : 0;
    const int off = block_scan_1024(c, wave_sums, &total) + carry[0];
    const int tc = total;
    const int ib = block_scan_1024(ni, wave_sums, &total) + carry[1];
    const int ti = total;
    if (mine) {
      a.counts[e] = c;
      a.offsets[e] = off;
      int run = off;
      for (int b0 = 0; b0 < a.blocks; b0 += SCAN_BATCH) {
        int t[SCAN_BATCH];
        hist_batch(rh, a.E, e, b0, a.blocks, t);
#pragma unroll
        for (int j = 0; j < SCAN_BATCH; ++j) {
          if (b0 + j < a.blocks) a.hist[(size_t)(b0 + j) * a.E + e] = run;
          run += t[j];
        }
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
  // the scan addresses hist with 32-bit byte offsets
  if ((int64_t)a.blocks * a.E * 4 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  int idbits = 1;
  while ((1 << idbits) < a.E) ++idbits;
  hipLaunchKernelGGL(route_rank_kernel, dim3(a.blocks), dim3(64 * RANK_WAVES), 0, s, a.ids,
                     (int)a.N, a.E, idbits, a.rank, a.hist);
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

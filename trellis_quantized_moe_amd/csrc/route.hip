// Route bucketing for the prefill path (gfx950): a stable counting sort of the flat slot
// indices t * topk + k by expert id (FORMAT F11, F14), in three launches:
//   1. rank:    blocks of ROUTE_CHUNK slots, four waves each; every wave ranks its quarter
//               64 slots at a time in index order (lanes holding the same expert are found
//               with one ballot per id bit, counts run in LDS), then the block adds the
//               earlier waves' counts. The block's counts go to hist.
//   2. scan:    one workgroup turns hist into per-(block, expert) bases, per-expert counts
//               and offsets, and the list of (expert, row0, nrows) work items, laid out for
//               the 8 XCDs (below).
//   3. scatter: pairs[base[block][e] + rank] = slot; empty (-1) slots get zero outputs and
//               invalid ids NaN outputs plus a status bit.
// No step depends on timing, so the order is the same on every run.
//
// Work items and the XCDs. The prefill GEMMs give the 8 XCDs (each with its own L2) 8
// contiguous, equal segments of the item list. Every item gathers its rows' activations, and
// a token's rows sit in topk experts' items: rows gathered on the same XCD at about the same
// time come from its L2. The slot order is token-major, so the rank blocks cut it into 8
// token ranges (block b in range 8 b / blocks), and an expert's slots, in slot order, run
// through the ranges in turn. With split_rows > 0, the items of an expert with at least
// split_rows slots go to the segment of the range that holds their middle row (row 64 of the
// item, or its last row), opening that segment; the other experts' items, in expert order,
// fill the segments up to an equal share. The items are the same either way (each expert's
// slots in runs of item_rows); without a split the list is in expert order. Which item
// computes a slot changes nothing in its result.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr int RANK_BLOCK = ROUTE_CHUNK;        // slots per rank block
constexpr int RANK_WAVES = 4;                  // waves per rank block
constexpr int RANK_ROUNDS = RANK_BLOCK / (64 * RANK_WAVES);  // 64-slot rounds per wave
constexpr int MAX_E = 4096;
constexpr int SCAN_PASSES = MAX_E / 1024;  // experts per scan thread
constexpr int XCDS = 8;
constexpr int XCD_CUS = 32;        // compute units per XCD
constexpr int ORDER_ROUNDS = 4;    // item lists of up to 4096 are put in snake order

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

// The same for XCDS ints per thread at once: res[x] is the exclusive prefix of v[x], tot[x]
// (shared) its total.
__device__ void block_scan8_1024(const int v[XCDS], int res[XCDS], int (*sums)[XCDS], int* tot) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl[XCDS];
#pragma unroll
  for (int x = 0; x < XCDS; ++x) incl[x] = v[x];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int x = 0; x < XCDS; ++x) {
      const int t = __shfl_up(incl[x], d, 64);
      if (lane >= d) incl[x] += t;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int x = 0; x < XCDS; ++x) sums[w][x] = incl[x];
  }
  __syncthreads();
  if (tid < XCDS) {
    int run = 0;
    for (int k = 0; k < 16; ++k) {
      const int t = sums[k][tid];
      sums[k][tid] = run;
      run += t;
    }
    tot[tid] = run;
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < XCDS; ++x) res[x] = sums[w][x] + incl[x] - v[x];
  __syncthreads();
}

// The token range of an expert's slot row r, given the first row of each range (start[0] =
// 0, non-decreasing).
__device__ __forceinline__ int item_range(const int start[XCDS], int r) {
  int x = 0;
#pragma unroll
  for (int j = 1; j < XCDS; ++j) x += r >= start[j] ? 1 : 0;
  return x;
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

// Snake order within each segment of a list of one-group items. The workgroups of an XCD go
// to its XCD_CUS compute units in turn, so items j, j + 32 and j + 64 of a segment share a
// unit. The items of a segment are ranked by their row blocks of 32 (the products' work,
// heaviest first; ties in list order) and dealt out in rounds of 32 that alternate
// direction, so that every unit gets a similar amount. Every thread holds up to
// ORDER_ROUNDS items (positions tid + 1024 m) between reading and writing the list.
__device__ void snake_order(int4* items, int all, const int seg[XCDS], const int B[XCDS],
                            const int S[XCDS]) {
  __shared__ int sums8[16][XCDS];
  __shared__ int tot8[XCDS];
  __shared__ int cnt[XCDS][4];     // items per segment and class
  __shared__ int segp[XCDS][4];    // items of each class before each segment's start
  __shared__ int carry[4];
  const int tid = threadIdx.x;
  if (tid < XCDS * 4) {
    cnt[tid >> 2][tid & 3] = 0;
    segp[tid >> 2][tid & 3] = -1;
  }
  if (tid < 4) carry[tid] = 0;
  __threadfence();  // the list, as written, is visible to every thread of the workgroup
  __syncthreads();
  int4 it[ORDER_ROUNDS];
  int cl[ORDER_ROUNDS], sx[ORDER_ROUNDS], pk[ORDER_ROUNDS];
#pragma unroll
  for (int m = 0; m < ORDER_ROUNDS; ++m) {
    const int i = m * 1024 + tid;
    const bool valid = i < all;
    it[m] = valid ? items[i] : make_int4(0, 0, 0, 0);
    // class 0: 4 blocks of 32 rows (the heaviest) .. class 3: 1 block
    cl[m] = valid ? 4 - min(4, (it[m].z + 31) >> 5) : -1;
    sx[m] = 0;
#pragma unroll
    for (int x = 1; x < XCDS; ++x) sx[m] += i >= seg[x] ? 1 : 0;
    int v[XCDS], pr[XCDS];
#pragma unroll
    for (int q = 0; q < XCDS; ++q) v[q] = q == cl[m] ? 1 : 0;
    block_scan8_1024(v, pr, sums8, tot8);
    pk[m] = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pr[q] += carry[q];
      if (q == cl[m]) pk[m] = pr[q];
    }
    if (valid) atomicAdd(&cnt[sx[m]][cl[m]], 1);
#pragma unroll
    for (int x = 0; x < XCDS; ++x) {
      if (i == seg[x]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) segp[x][q] = pr[q];
      }
    }
    __syncthreads();
    if (tid < 4) carry[tid] += tot8[tid];
    __syncthreads();
  }
  // a segment that starts at the end of the list has every item before it
  if (tid < XCDS * 4 && segp[tid >> 2][tid & 3] < 0) segp[tid >> 2][tid & 3] = carry[tid & 3];
  __syncthreads();
#pragma unroll
  for (int m = 0; m < ORDER_ROUNDS; ++m) {
    if (m * 1024 + tid >= all) break;
    int x0 = 0, n = 0, r = 0;
#pragma unroll
    for (int x = 0; x < XCDS; ++x) {
      if (x == sx[m]) {
        x0 = seg[x];
        n = B[x] + S[x];
        r = pk[m] - segp[x][cl[m]];
#pragma unroll
        for (int q = 0; q < 4; ++q) r += q < cl[m] ? cnt[x][q] : 0;
      }
    }
    const int round = r / XCD_CUS, j = r % XCD_CUS;
    const int len = min(XCD_CUS, n - round * XCD_CUS);
    items[x0 + round * XCD_CUS + ((round & 1) ? len - 1 - j : j)] = it[m];
  }
}

// SPLIT: items placed by token range (a.E <= 1024, one expert per thread); else the
// experts' items in expert order, up to MAX_E experts.
template <bool SPLIT>
__global__ __launch_bounds__(1024) void route_scan_kernel(RouteArgs a) {
  constexpr int PASSES = SPLIT ? 1 : SCAN_PASSES;
  __shared__ int wave_sums[16];
  __shared__ int total;
  __shared__ int sums8[16][XCDS];
  __shared__ int tot8[XCDS];
  __shared__ int carry[2 + XCDS];  // slots, other experts' items, split items per range
  const int tid = threadIdx.x;
  if (tid < 2 + XCDS) carry[tid] = 0;
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      a.hist, (short)0, (int)((size_t)a.blocks * a.E * 4), 0x00020000);
  const int R = a.item_rows;
  // per expert of this thread (e = 1024 p + tid): slots and offset, whether it is placed by
  // range, the first row of each range among its slots and the list position of its first
  // item placed in range x among all items placed in range x, or the position of its first
  // item among the other experts' items
  int cnt[PASSES], eoff[PASSES], psm[PASSES];
  int cx[PASSES][XCDS], pbx[PASSES][XCDS];
  bool big[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    cnt[p] = eoff[p] = psm[p] = 0;
    big[p] = false;
#pragma unroll
    for (int x = 0; x < XCDS; ++x) cx[p][x] = pbx[p][x] = 0;
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    if (p * 1024 >= a.E) break;
    const int e = p * 1024 + tid;
    const bool mine = e < a.E;
    int c = 0;
    if (mine) {
      for (int b0 = 0; b0 < a.blocks; b0 += SCAN_BATCH) {
        int t[SCAN_BATCH];
        hist_batch(rh, a.E, e, b0, a.blocks, t);
#pragma unroll
        for (int j = 0; j < SCAN_BATCH; ++j) {
          c += t[j];
          if constexpr (SPLIT) {
            const int xr = ((b0 + j) * XCDS) / a.blocks;
#pragma unroll
            for (int x = 0; x < XCDS; ++x) cx[p][x] += xr == x ? t[j] : 0;
          }
        }
      }
    }
    const int off = block_scan_1024(c, wave_sums, &total) + carry[0];
    const int tc = total;
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
    }
    cnt[p] = c;
    eoff[p] = off;
    big[p] = SPLIT && mine && c >= a.split_rows;
    if constexpr (SPLIT) {
      // cx becomes the first row of each range among the expert's slots
      int run_r = 0;
#pragma unroll
      for (int x = 0; x < XCDS; ++x) {
        const int t = cx[p][x];
        cx[p][x] = run_r;
        run_r += t;
      }
      int nb[XCDS], pb[XCDS];
#pragma unroll
      for (int x = 0; x < XCDS; ++x) nb[x] = 0;
      if (big[p]) {
        for (int r0 = 0; r0 < c; r0 += R) {
          const int xi = item_range(cx[p], min(r0 + R / 2, c - 1));
#pragma unroll
          for (int x = 0; x < XCDS; ++x) nb[x] += xi == x ? 1 : 0;
        }
      }
      block_scan8_1024(nb, pb, sums8, tot8);
#pragma unroll
      for (int x = 0; x < XCDS; ++x) pbx[p][x] = pb[x] + carry[2 + x];
    }
    const int ns = (a.items && mine && !big[p]) ? (c + R - 1) / R : 0;
    psm[p] = block_scan_1024(ns, wave_sums, &total) + carry[1];
    const int ts = total;
    __syncthreads();
    if (tid == 0) {
      carry[0] += tc;
      carry[1] += ts;
    }
    if (SPLIT && tid < XCDS) carry[2 + tid] += tot8[tid];
    __syncthreads();
  }
  if (tid == 0) a.offsets[a.E] = carry[0];
  if (!a.items) return;

  // segments: x holds the items placed in range x, then its share of the others' items
  int B[XCDS], S[XCDS], seg[XCDS], ps0[XCDS];
  const int small = carry[1];
  int all = small;
#pragma unroll
  for (int x = 0; x < XCDS; ++x) {
    B[x] = carry[2 + x];
    all += B[x];
  }
  const int share = (all + XCDS - 1) / XCDS;
  int rem = small, run = 0, runs = 0;
#pragma unroll
  for (int x = 0; x < XCDS; ++x) {
    S[x] = min(rem, max(0, share - B[x]));
    rem -= S[x];
  }
  S[XCDS - 1] += rem;
#pragma unroll
  for (int x = 0; x < XCDS; ++x) {
    seg[x] = run;
    ps0[x] = runs;
    run += B[x] + S[x];
    runs += S[x];
  }
  int4* items = reinterpret_cast<int4*>(a.items);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int e = p * 1024 + tid;
    if (p * 1024 >= a.E || e >= a.E) break;
    const int c = cnt[p];
    if (big[p]) {
      // the ranges of successive items never decrease: k counts the items placed in the
      // current one
      int xprev = -1, k = 0;
      for (int r0 = 0; r0 < c; r0 += R) {
        const int xi = item_range(cx[p], min(r0 + R / 2, c - 1));
        k = xi == xprev ? k + 1 : 0;
        xprev = xi;
        int base = 0;
#pragma unroll
        for (int x = 0; x < XCDS; ++x)
          if (x == xi) base = seg[x] + pbx[p][x];
        items[base + k] = make_int4(e, eoff[p] + r0, min(R, c - r0), 0);
      }
    } else {
      for (int k = 0; k * R < c; ++k) {
        const int g = psm[p] + k;  // its place among the other experts' items
        int pos = 0;
#pragma unroll
        for (int x = 0; x < XCDS; ++x)
          if (g >= ps0[x] && g < ps0[x] + S[x]) pos = seg[x] + B[x] + (g - ps0[x]);
        items[pos] = make_int4(e, eoff[p] + k * R, min(R, c - k * R), 0);
      }
    }
  }
  if (tid == 0) *a.n_items = all;
  if constexpr (SPLIT) {
    if ((a.out + 127) / 128 == 1 && all <= 1024 * ORDER_ROUNDS)
      snake_order(items, all, seg, B, S);
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
  if (a.items && a.split_rows > 0 && a.E <= 1024)
    hipLaunchKernelGGL(route_scan_kernel<true>, dim3(1), dim3(1024), 0, s, a);
  else
    hipLaunchKernelGGL(route_scan_kernel<false>, dim3(1), dim3(1024), 0, s, a);
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

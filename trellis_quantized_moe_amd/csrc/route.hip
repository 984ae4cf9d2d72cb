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
constexpr int XCDS = 8;
constexpr int XCD_CUS = 32;        // compute units per XCD
constexpr int ORDER_ROUNDS = 2;    // item lists of up to 2048 are put in snake order

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

// Inclusive sums within each row of 16 lanes by DPP (row_shr 1, 2, 4, 8; a lane with no
// source adds 0).
__device__ __forceinline__ int row_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  return v;
}
// Inclusive sums over the 64 lanes: the rows', then lane 15 of rows 0 and 2 added to rows 1
// and 3 (row_bcast 15), then lane 31 to rows 2 and 3 (row_bcast 31).
__device__ __forceinline__ int wave_scan_incl(int v) {
  v = row_scan_incl(v);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}

// Exclusive block scan of one int per thread (1024 threads); returns the prefix and
// stores the total in *total. Wave 0 scans the 16 wave totals.
__device__ int block_scan_1024(int v, int* wave_sums, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int incl = wave_scan_incl(v);
  if (lane == 63) wave_sums[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int t = lane < 16 ? wave_sums[lane] : 0;
    const int ti = row_scan_incl(t);
    if (lane < 16) wave_sums[lane] = ti - t;
    if (lane == 15) *total = ti;
  }
  __syncthreads();
  const int res = wave_sums[w] + incl - v;
  __syncthreads();
  return res;
}

// The same for XCDS ints per thread at once: res[x] is the exclusive prefix of v[x], tot[x]
// (shared) its total. Wave 0 scans the wave totals of four columns per pass, one row of
// 16 lanes each.
__device__ void block_scan8_1024(const int v[XCDS], int res[XCDS], int (*sums)[XCDS], int* tot) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl[XCDS];
#pragma unroll
  for (int x = 0; x < XCDS; ++x) incl[x] = wave_scan_incl(v[x]);
  if (lane == 63) {
#pragma unroll
    for (int x = 0; x < XCDS; ++x) sums[w][x] = incl[x];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int h = 0; h < XCDS / 4; ++h) {
      const int x = 4 * h + (lane >> 4), k = lane & 15;
      const int t = sums[k][x];
      const int ti = row_scan_incl(t);
      sums[k][x] = ti - t;
      if (k == 15) tot[x] = ti;
    }
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < XCDS; ++x) res[x] = sums[w][x] + incl[x] - v[x];
  __syncthreads();
}

// An expert's items are its slot rows in runs of R; the anchor of item i is row
// min(R i + R / 2, c - 1). first_items(Y) = the items i < ni - 1 with R i + R / 2 < Y (for
// those items the anchor is R i + R / 2); the last item is counted on its own.
__device__ __forceinline__ int first_items(int Y, int R, int ni) {
  const int n = Y <= R / 2 ? 0 : (Y - R / 2 + R - 1) / R;
  return min(n, ni - 1);
}
// The token range of row r, given the first row of each range (start[0] = 0, ascending).
__device__ __forceinline__ int row_range(const int start[XCDS], int r) {
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
  __shared__ int sseg[XCDS], slen[XCDS];
  const int tid = threadIdx.x;
  if (tid < XCDS * 4) {
    cnt[tid >> 2][tid & 3] = 0;
    segp[tid >> 2][tid & 3] = -1;
  }
  if (tid < 4) carry[tid] = 0;
  if (tid < XCDS) {
#pragma unroll
    for (int x = 0; x < XCDS; ++x) {
      if (x == tid) {
        sseg[x] = seg[x];
        slen[x] = B[x] + S[x];
      }
    }
  }
  __syncthreads();  // the list, as written, is visible to every thread of the workgroup
  int4 it[ORDER_ROUNDS];
  int cl[ORDER_ROUNDS], sx[ORDER_ROUNDS], pk[ORDER_ROUNDS];
#pragma unroll
  for (int m = 0; m < ORDER_ROUNDS; ++m) {
    if (m * 1024 >= all) break;
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
    const int x = sx[m];
    const int x0 = sseg[x], n = slen[x];
    int r = pk[m] - segp[x][cl[m]];
    for (int q = 0; q < cl[m]; ++q) r += cnt[x][q];
    const int round = r / XCD_CUS, j = r % XCD_CUS;
    const int len = min(XCD_CUS, n - round * XCD_CUS);
    items[x0 + round * XCD_CUS + ((round & 1) ? len - 1 - j : j)] = it[m];
  }
}

// Per-expert counts and offsets and the bases of every (block, expert) in hist; items (when
// asked) in expert order. Up to MAX_E experts, 1024 a pass.
// Thread e writes the bases of its column of hist (off + the slots of the earlier blocks),
// by buffer stores (those past the last block are dropped). With st, also the first row of
// each token range x among its slots: the slots of the blocks before the range's first
// block, the first b with 8 b >= x blocks.
template <bool ST>
__device__ __forceinline__ void hist_bases(__amdgpu_buffer_rsrc_t rh, int E, int e, int blocks,
                                           int off, int (&st)[XCDS]) {
  int lo[XCDS];
#pragma unroll
  for (int x = 0; x < XCDS; ++x) {
    lo[x] = (x * blocks + XCDS - 1) / XCDS;
    if constexpr (ST) st[x] = 0;
  }
  typedef int i32x32 __attribute__((ext_vector_type(SCAN_BATCH)));
  int run = off;
  for (int b0 = 0; b0 < blocks; b0 += SCAN_BATCH) {
    int t[SCAN_BATCH];
    hist_batch(rh, E, e, b0, blocks, t);
    i32x32 pre;  // the base of each block of the batch
#pragma unroll
    for (int j = 0; j < SCAN_BATCH; ++j) {
      pre[j] = run;
      __builtin_amdgcn_raw_buffer_store_b32(run, rh, 4u * e, 4u * (uint32_t)((b0 + j) * E), 0);
      run += t[j];
    }
    if constexpr (ST) {
      // a range's first block in this batch: its base (a uniform index into pre)
#pragma unroll
      for (int x = 1; x < XCDS; ++x) {
        const int j = lo[x] - b0;
        if (j >= 0 && j < SCAN_BATCH) st[x] = pre[j] - off;
      }
    }
  }
  if constexpr (ST) {
#pragma unroll
    for (int x = 1; x < XCDS; ++x)
      if (lo[x] >= blocks) st[x] = run - off;  // a range with no block starts after them all
  }
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
  const int R = a.item_rows;
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
    const int ni = (a.items && mine) ? (c + R - 1) / R : 0;
    const int off = block_scan_1024(c, wave_sums, &total) + carry[0];
    const int tc = total;
    const int ib = block_scan_1024(ni, wave_sums, &total) + carry[1];
    const int ti = total;
    if (mine) {
      a.counts[e] = c;
      a.offsets[e] = off;
      int unused[XCDS];
      hist_bases<false>(rh, a.E, e, a.blocks, off, unused);
      for (int k = 0; k < ni; ++k)
        reinterpret_cast<int4*>(a.items)[ib + k] =
            make_int4(e, off + k * R, min(R, c - k * R), 0);
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

// The same with the items placed by token range (a.items set, a.split_rows > 0, a.E <=
// 1024: one expert per thread).
__global__ __launch_bounds__(1024) void route_scan_split_kernel(RouteArgs a) {
  __shared__ int wave_sums[16];
  __shared__ int total;
  __shared__ int sums8[16][XCDS];
  __shared__ int tot8[XCDS];
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      a.hist, (short)0, (int)((size_t)a.blocks * a.E * 4), 0x00020000);
  const int R = a.item_rows;
  const int e = tid;
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
  const int off = block_scan_1024(c, wave_sums, &total);
  const int all_slots = total;
  // st[x]: the first row of token range x among the expert's slots (the slots of the
  // blocks before the range's first block)
  int st[XCDS] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (mine) {
    a.counts[e] = c;
    a.offsets[e] = off;
    hist_bases<true>(rh, a.E, e, a.blocks, off, st);
  }
  const bool big = mine && c >= a.split_rows;
  // items per range: the counts of first_items between the range starts, and the last item
  const int ni = (c + R - 1) / R;
  const int last = (ni - 1) * R;
  int nb[XCDS], pb[XCDS];
  int xl = 0;
  if (big) {
    xl = row_range(st, min(last + R / 2, c - 1));
#pragma unroll
    for (int x = 0; x < XCDS; ++x)
      nb[x] = first_items(x + 1 < XCDS ? st[x + 1] : c, R, ni) - first_items(st[x], R, ni) +
              (x == xl ? 1 : 0);
  } else {
#pragma unroll
    for (int x = 0; x < XCDS; ++x) nb[x] = 0;
  }
  block_scan8_1024(nb, pb, sums8, tot8);
  const int ns = (mine && !big) ? ni : 0;
  const int psm = block_scan_1024(ns, wave_sums, &total);
  const int small = total;
  if (tid == 0) a.offsets[a.E] = all_slots;

  // segments: x holds the items placed in range x, then its share of the others' items
  int B[XCDS], S[XCDS], seg[XCDS], ps0[XCDS];
  int all = small;
#pragma unroll
  for (int x = 0; x < XCDS; ++x) {
    B[x] = tot8[x];
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
  if (big) {
    // range x takes items first_items(start x) .. first_items(start x + 1) - 1, then the
    // last item joins the range of its anchor, after them
    int lpos = 0;
#pragma unroll
    for (int x = 0; x < XCDS; ++x) {
      const int i0 = first_items(st[x], R, ni);
      const int i1 = first_items(x + 1 < XCDS ? st[x + 1] : c, R, ni);
      const int base = seg[x] + pb[x];
      for (int i = i0; i < i1; ++i) items[base + (i - i0)] = make_int4(e, off + i * R, R, 0);
      if (x == xl) lpos = base + (i1 - i0);
    }
    items[lpos] = make_int4(e, off + last, c - last, 0);
  } else if (mine) {
    for (int k = 0; k < ni; ++k) {
      const int g = psm + k;  // its place among the other experts' items
      int pos = 0;
#pragma unroll
      for (int x = 0; x < XCDS; ++x)
        if (g >= ps0[x] && g < ps0[x] + S[x]) pos = seg[x] + B[x] + (g - ps0[x]);
      items[pos] = make_int4(e, off + k * R, min(R, c - k * R), 0);
    }
  }
  if (tid == 0) *a.n_items = all;
  if ((a.out + 127) / 128 == 1 && all <= 1024 * ORDER_ROUNDS) snake_order(items, all, seg, B, S);
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
    hipLaunchKernelGGL(route_scan_split_kernel, dim3(1), dim3(1024), 0, s, a);
  else
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

// Prefill grouped GEMM over trellis-coded experts (gfx950): the work-item core of
// gemm_core.h with a T16 B producer. Each thread decodes one tile column (16 weights of
// one output channel) per step; the step's 32 inputs are two tile columns of each of the
// group's 8 strips (256 columns, one per thread). The decoded q are exact in bf16.
#include "gemm_core.h"
#include "trellis_decode.h"

namespace tq {

namespace {

template <int K>
struct TrellisProducer {
  const uint32_t* unit;
  int n_ti, grp, ns;
  int s8, c, n, o0, o1, o2;
  uint32_t sh3;

  __device__ TrellisProducer(const uint32_t* u, int in, int grp_, int ns_)
      : unit(u), n_ti(in / 16), grp(grp_), ns(ns_) {
    const int tid = threadIdx.x;
    s8 = tid >> 5;
    c = (tid >> 4) & 1;
    n = tid & 15;
    o0 = o1 = o2 = 0;
    sh3 = 0;
    if constexpr (K == 3) k3_column_words(n, &o0, &o1, &o2, &sh3);
  }

  __device__ __forceinline__ void operator()(int kk, int* o, int* h, uint32_t nat[8]) {
    *o = 16 * s8 + n;
    *h = c;
#pragma unroll
    for (int t = 0; t < 8; ++t) nat[t] = 0u;
    if (s8 < ns) {
      const uint32_t* tile = unit + (size_t)((grp * 8 + s8) * n_ti + 2 * kk + c) * (8 * K);
      uint32_t M[8];
      if constexpr (K == 2) {
        const uint32_t w = tile[n];
        col_mpairs_k2(w, row_next(w), M);
      } else if constexpr (K == 4) {
        const uint2 ww = *reinterpret_cast<const uint2*>(tile + 2 * n);
        col_mpairs_k4(ww.x, ww.y, row_next(ww.x), M);
      } else {
        col_mpairs_k3(tile[o0], tile[o1], tile[o2], sh3, M);
      }
      mpairs_to_bf16_natural<K>(M, nat);
    }
  }
};

__global__ __launch_bounds__(GEMM_THREADS) void trellis_gemm_kernel(TrellisGemmArgs a) {
  __shared__ GemmShared sh;
  const int item = blockIdx.x / a.groups;
  const int grp = blockIdx.x % a.groups;
  if (item >= *a.n_items) return;
  const int4 itd = reinterpret_cast<const int4*>(a.items)[item];
  const int e = itd.x;
  gemm_load_slots(sh, a.pairs, itd.y, itd.z);
  GemmItem it;
  it.x = a.x;
  it.gates = a.gates;
  it.scales = a.scales + (size_t)e * a.out;
  it.y = a.y;
  it.in = a.in;
  it.out = a.out;
  it.topk = a.topk;
  it.grp = grp;
  it.nrows = itd.z;
  it.ns = min(8, a.out / 16 - grp * 8);
  const int K = a.bits[e];
  const int64_t off = a.code_off[e];
  if ((K < 2 || K > 4) || (off & 15)) {
    gemm_item_nan(it, sh);
    if (threadIdx.x == 0) set_status(a.status, STATUS_BAD_UNIT);
    return;
  }
  const uint32_t* unit = a.codes + off / 4;
  if (K == 2) {
    TrellisProducer<2> p(unit, a.in, grp, it.ns);
    gemm_item(it, sh, p);
  } else if (K == 3) {
    TrellisProducer<3> p(unit, a.in, grp, it.ns);
    gemm_item(it, sh, p);
  } else {
    TrellisProducer<4> p(unit, a.in, grp, it.ns);
    gemm_item(it, sh, p);
  }
}

}  // namespace

hipError_t launch_trellis_gemm(const TrellisGemmArgs& a, hipStream_t s) {
  const int blocks = a.max_items * a.groups;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(trellis_gemm_kernel, dim3(blocks), dim3(GEMM_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq

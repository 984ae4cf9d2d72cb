// Prefill grouped GEMM over trellis-coded experts (gfx950): the work-item core of
// gemm_core.h with a T16 B producer. Each thread decodes one tile column (16 weights of
// one output channel) per step; the step's 32 inputs are two tile columns of each of the
// group's 8 strips (256 columns, one per thread). Each weight enters the matrix cores as
// the f16 subnormal (q + 255) * 2^-24 (trellis_decode.h), against the prepared f16
// activations; the epilogue scales by 2^24 and removes 255 * sum(x) per token.
#include "gemm_core.h"
#include "trellis_decode.h"

namespace tq {

namespace {

// Thread t decodes, each step, tile column 2 kk + c of strip s8 (s8 = t / 32, c = t / 16 % 2)
// for output channel n = t % 16: 16 weights of channel 16 s8 + n. The 16 lanes of a tile
// read its words once; the neighbour word comes from the next lane (row rotation).
template <int K>
struct TrellisProducer {
  static constexpr bool kF16 = true;
  struct Raw {
    uint32_t w[K == 2 ? 1 : (K == 4 ? 2 : 3)];
  };
  GemmRsrc rc;
  uint32_t vo[3];
  uint32_t sh3;
  int o, h;

  __device__ TrellisProducer(const uint32_t* unit, int out, int in, int grp, int ns) {
    constexpr int TW = 8 * K;
    const int tid = threadIdx.x;
    const int s8 = tid >> 5, c = (tid >> 4) & 1, n = tid & 15;
    const int n_ti = in / 16;
    o = 16 * s8 + n;
    h = c;
    rc = gemm_rsrc(unit, (uint32_t)((size_t)out * in * K / 8));
    // strips past the group read its last strip (their rows of the B tile are never used)
    const int strip = grp * 8 + (s8 < ns ? s8 : ns - 1);
    const uint32_t base = (uint32_t)((strip * n_ti + c) * TW);
    sh3 = 0;
    vo[0] = vo[1] = vo[2] = 0;
    if constexpr (K == 2) {
      vo[0] = 4u * (base + n);
    } else if constexpr (K == 4) {
      vo[0] = 4u * (base + 2 * n);
    } else {
      int a, b, d;
      k3_column_words(n, &a, &b, &d, &sh3);
      vo[0] = 4u * (base + a);
      vo[1] = 4u * (base + b);
      vo[2] = 4u * (base + d);
    }
  }

  __device__ __forceinline__ void load(int kk, Raw& r) const {
    constexpr int TW = 8 * K;
    const uint32_t so = 4u * (uint32_t)(2 * kk * TW);  // two tile columns per step
    if constexpr (K == 2) {
      r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rc, vo[0], so, 0);
    } else if constexpr (K == 4) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, vo[0], so, 0);
      r.w[0] = v.x;
      r.w[1] = v.y;
    } else {
      r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rc, vo[0], so, 0);
      r.w[1] = __builtin_amdgcn_raw_buffer_load_b32(rc, vo[1], so, 0);
      r.w[2] = __builtin_amdgcn_raw_buffer_load_b32(rc, vo[2], so, 0);
    }
  }

  __device__ __forceinline__ void decode(const Raw& r, uint32_t nat[8]) const {
    uint32_t M[8];
    if constexpr (K == 2)
      col_mpairs_k2(r.w[0], row_next(r.w[0]), M);
    else if constexpr (K == 4)
      col_mpairs_k4(r.w[0], r.w[1], row_next(r.w[0]), M);
    else
      col_mpairs_k3(r.w[0], r.w[1], r.w[2], sh3, M);
    byte_sums<K>(M, nat);  // [lo: v[r + 8], hi: v[r]], the layout of the prepared activations
  }
};

// One launch per width KW (each needs its own register budget): workgroups whose item has
// another width leave at once; the KW = 2 launch also handles bad unit descriptors.
template <int KW>
__global__ __launch_bounds__(GEMM_THREADS, 2) void trellis_gemm_kernel(TrellisGemmArgs a) {
  __shared__ GemmShared sh;
  const int item = blockIdx.x / a.groups;
  const int grp = blockIdx.x % a.groups;
  if (item >= *a.n_items) return;
  const int4 itd = reinterpret_cast<const int4*>(a.items)[item];
  const int e = itd.x;
  const int K = a.bits[e];
  const int64_t off = a.code_off[e];
  const bool bad = (K < 2 || K > 4) || (off & 15);
  if (bad ? KW != 2 : K != KW) return;
  gemm_load_slots(sh, a.pairs, itd.y, itd.z);
  GemmItem it;
  it.x = a.xp;
  it.x_bytes = a.x_bytes;
  it.rowsum = a.rowsum;
  it.gates = a.gates;
  it.scales = a.scales + (size_t)e * a.out;
  it.y = a.y;
  it.in = a.in;
  it.out = a.out;
  it.topk = a.topk;
  it.grp = grp;
  it.nrows = itd.z;
  it.ns = min(8, a.out / 16 - grp * 8);
  if (bad) {
    gemm_item_nan(it, sh);
    if (threadIdx.x == 0) set_status(a.status, STATUS_BAD_UNIT);
    return;
  }
  TrellisProducer<KW> p(a.codes + off / 4, a.out, a.in, grp, it.ns);
  gemm_item(it, sh, p);
}

}  // namespace

hipError_t launch_trellis_gemm(const TrellisGemmArgs& a, hipStream_t s) {
  const int blocks = a.max_items * a.groups;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(trellis_gemm_kernel<2>, dim3(blocks), dim3(GEMM_THREADS), 0, s, a);
  hipLaunchKernelGGL(trellis_gemm_kernel<3>, dim3(blocks), dim3(GEMM_THREADS), 0, s, a);
  hipLaunchKernelGGL(trellis_gemm_kernel<4>, dim3(blocks), dim3(GEMM_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq

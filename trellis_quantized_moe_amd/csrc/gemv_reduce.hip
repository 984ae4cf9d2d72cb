// Piece reduction: the third launch of the planned decode batches (gemv_plan.h), trellis and
// the E8M0-scaled stores. A slot's expert group was split into pieces by the plan; their
// partial sums are added in piece order.
//   - Trellis pieces are exact int64 sums of x * (q - 1), x the token's 16-bit integers.
//     They are added exactly, so the sum does not depend on where the plan cut the inputs
//     (a slot gets the same bits whatever else the batch routes). The token's sum of x is
//     added back (making it the exact sum of x * q), the total is rounded to fp32 once, and
//     the token's 2^-e, the per-channel fp16 scale and the gate are applied.
//   - MXFP4 / fp8b32 pieces are fp32 sums; they are added in piece order.
// Empty slots give 0, bad ids and bad units NaN (their status bits were set by the plan).
// Without combine, one thread per 4 outputs of a slot; with combine, one block per (token,
// 128 outputs) puts the slot values in LDS and adds them over k = 0..topk-1 in order.
#include "gemv_reduce.h"

namespace tq {

namespace {

template <bool EXACT>
__global__ __launch_bounds__(256) void piece_reduce_kernel(PieceReduceArgs a) {
  const int per_row = a.out / 4;
  if (!a.combine) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)a.N * per_row) return;
    const int r = (int)(idx / per_row), o = (int)(idx % per_row) * 4;
    *reinterpret_cast<float4*>(a.y + (size_t)r * a.out + o) = piece_slot<EXACT>(a, r, o);
    return;
  }
  // block = (token t, outputs o0 .. o0 + 127); LDS holds the topk slot values
  __shared__ float4 vals[PIECE_MAX_TOPK * 32];
  const int chunks = (a.out + 127) / 128;
  const int t = blockIdx.x / chunks, o0 = (blockIdx.x % chunks) * 128;
  const int w4 = min(128, a.out - o0) / 4;  // float4 columns in this chunk
  for (int v = threadIdx.x; v < a.topk * 32; v += 256) {
    const int k = v / 32, c = v % 32;
    if (c < w4) vals[v] = piece_slot<EXACT>(a, t * a.topk + k, o0 + 4 * c);
  }
  lds_barrier();
  if ((int)threadIdx.x < w4) {
    float4 acc = vals[threadIdx.x];
    for (int k = 1; k < a.topk; ++k) add4(acc, vals[k * 32 + threadIdx.x]);
    *reinterpret_cast<float4*>(a.y + (size_t)t * a.out + o0 + 4 * threadIdx.x) = acc;
  }
}

}  // namespace

hipError_t launch_piece_reduce(const PieceReduceArgs& a, hipStream_t s) {
  unsigned blocks;
  if (a.combine) {
    blocks = (unsigned)((int64_t)(a.N / a.topk) * ((a.out + 127) / 128));
  } else {
    const int64_t total = (int64_t)a.N * (a.out / 4);
    blocks = (unsigned)((total + 255) / 256);
  }
  if (blocks == 0) return hipSuccess;
  if (a.exact)
    hipLaunchKernelGGL(piece_reduce_kernel<true>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(piece_reduce_kernel<false>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq

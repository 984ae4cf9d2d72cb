// Piece reduction: the third launch of the planned decode batches (gemv_plan.h), trellis and
// MXFP4. A slot's expert group was split into pieces by the plan; their partial sums are
// added in piece order. For trellis layers those sums are of x * (q - 1) with x the
// token's 16-bit integers: the token's sum of x is added back and the token's 2^-e
// applied, then the per-channel fp16 scale; MXFP4 sums are final. Then the gate. Empty
// slots give 0, bad ids and bad units NaN (their status bits were set by the plan). Without
// combine, one thread per 4 outputs of a slot; with combine, one block per (token, 128
// outputs) puts the slot values in LDS and adds them over k = 0..topk-1 in order.
#include "gemv_plan.h"
#include "tq_internal.h"

namespace tq {

namespace {

__device__ __forceinline__ void add4(float4& s, const float4& v) {
  s.x += v.x;
  s.y += v.y;
  s.z += v.z;
  s.w += v.w;
}

__device__ __forceinline__ float4 piece_slot(const PieceReduceArgs& a, int slot, int o) {
  const int t = slot / a.topk;
  const size_t stride = (size_t)a.N * a.out;
  const float* p = a.partial + (size_t)slot * a.out + o;
  // The slot's record, its token's values and gate and its first a.pre pieces are
  // requested together (indices clamped to the buffer's qmax pieces; the ones past the
  // slot's count are dropped); pieces pre .. 7 only once the record gives the slot's count.
  // The host takes pre = 1 when the split is expected to give one piece per slot: a plane
  // past the count holds no partial and would be read from HBM for nothing. Further pieces
  // follow eight at a time; all are added in piece order.
  const int4 inf = a.slot_info[slot];
  const float add = a.xsum ? (float)a.xsum[t] : 0.0f;
  const float mul = a.xscale ? a.xscale[t] : 1.0f;
  const float gate = a.gates ? a.gates[slot] : 1.0f;
  float4 v[8];
  v[0] = *reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int q = 1; q < 8; ++q)
    if (q < a.pre) v[q] = *reinterpret_cast<const float4*>(p + (size_t)min(q, a.qmax - 1) * stride);
  if (inf.x == SLOT_EMPTY) return make_float4(0.f, 0.f, 0.f, 0.f);
  if (inf.x < 0) {
    const float nan = __builtin_nanf("");
    return make_float4(nan, nan, nan, nan);
  }
  const int e = inf.x, np = inf.y;
#pragma unroll
  for (int q = 1; q < 8; ++q)
    if (q >= a.pre && q < np) v[q] = *reinterpret_cast<const float4*>(p + (size_t)q * stride);
  const uint2 sc = a.scales ? *reinterpret_cast<const uint2*>(a.scales + (size_t)e * a.out + o)
                           : make_uint2(0x3C003C00u, 0x3C003C00u);  // fp16 1.0
  float4 s = v[0];
#pragma unroll
  for (int q = 1; q < 8; ++q)
    if (q < np) add4(s, v[q]);
  for (int q0 = 8; q0 < np; q0 += 8) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      v[q] = *reinterpret_cast<const float4*>(p + (size_t)min(q0 + q, np - 1) * stride);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q0 + q < np) add4(s, v[q]);
  }
  const uint32_t sw[2] = {sc.x, sc.y};
  float r[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = (r[j] + add) * mul;
    r[j] = r[j] * f16_bits_to_f32(sw[j >> 1] >> (16 * (j & 1)));
    if (a.gates) r[j] = r[j] * gate;
  }
  return make_float4(r[0], r[1], r[2], r[3]);
}

__global__ __launch_bounds__(256) void piece_reduce_kernel(PieceReduceArgs a) {
  const int per_row = a.out / 4;
  if (!a.combine) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)a.N * per_row) return;
    const int r = (int)(idx / per_row), o = (int)(idx % per_row) * 4;
    *reinterpret_cast<float4*>(a.y + (size_t)r * a.out + o) = piece_slot(a, r, o);
    return;
  }
  // block = (token t, outputs o0 .. o0 + 127); LDS holds the topk slot values
  __shared__ float4 vals[PIECE_MAX_TOPK * 32];
  const int chunks = (a.out + 127) / 128;
  const int t = blockIdx.x / chunks, o0 = (blockIdx.x % chunks) * 128;
  const int w4 = min(128, a.out - o0) / 4;  // float4 columns in this chunk
  for (int v = threadIdx.x; v < a.topk * 32; v += 256) {
    const int k = v / 32, c = v % 32;
    if (c < w4) vals[v] = piece_slot(a, t * a.topk + k, o0 + 4 * c);
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
  hipLaunchKernelGGL(piece_reduce_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tq

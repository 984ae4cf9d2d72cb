// The piece reduction of one slot's four outputs (the decode batches' third launch, and the
// routed FFN's intermediate step). See gemv_reduce.hip for the scheme.
#pragma once

#include "gemv_plan.h"
#include "tq_internal.h"

namespace tq {

__device__ __forceinline__ void add4(float4& s, const float4& v) {
  s.x += v.x;
  s.y += v.y;
  s.z += v.z;
  s.w += v.w;
}

// Four outputs of one piece: fp32, or the exact int64 sums.
template <bool EXACT>
struct Quad;
template <>
struct Quad<false> {
  float4 v;
  __device__ void load(const void* p, size_t i) {
    v = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
  }
  __device__ void zero() { v = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ void add(const Quad& o) { add4(v, o.v); }
};
template <>
struct Quad<true> {
  int64_t v[4];
  __device__ void load(const void* p, size_t i) {
    const longlong2* q = reinterpret_cast<const longlong2*>(static_cast<const int64_t*>(p) + i);
    const longlong2 a = q[0], b = q[1];
    v[0] = a.x;
    v[1] = a.y;
    v[2] = b.x;
    v[3] = b.y;
  }
  __device__ void zero() { v[0] = v[1] = v[2] = v[3] = 0; }
  __device__ void add(const Quad& o) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] += o.v[j];
  }
};

template <bool EXACT>
__device__ __forceinline__ float4 piece_slot(const PieceReduceArgs& a, int slot, int o) {
  const int t = slot / a.xdiv;  // the slot's activation row
  const size_t stride = (size_t)a.N * a.out;
  const size_t base = (size_t)slot * a.out + o;
  // The slot's record, its token's values and gate and its first a.pre pieces are
  // requested together (indices clamped to the buffer's qmax pieces; the ones past the
  // slot's count are dropped); pieces pre .. 7 only once the record gives the slot's count.
  // The host takes pre = 1 when the split is expected to give one piece per slot: a plane
  // past the count holds no partial and would be read from memory for nothing. Further
  // pieces follow eight at a time; all are added in piece order.
  const int4 inf = a.slot_info[slot];
  const int32_t add = a.xsum ? a.xsum[t] : 0;
  const float mul = a.xscale ? a.xscale[t] : 1.0f;
  const float gate = a.gates ? a.gates[slot] : 1.0f;
  Quad<EXACT> v[8];
  v[0].load(a.partial, base);
#pragma unroll
  for (int q = 1; q < 8; ++q)
    if (q < a.pre) v[q].load(a.partial, base + (size_t)min(q, a.qmax - 1) * stride);
  if (inf.x == SLOT_EMPTY) return make_float4(0.f, 0.f, 0.f, 0.f);
  if (inf.x < 0) {
    const float nan = __builtin_nanf("");
    return make_float4(nan, nan, nan, nan);
  }
  const int e = inf.x, np = inf.y;
#pragma unroll
  for (int q = 1; q < 8; ++q)
    if (q >= a.pre && q < np) v[q].load(a.partial, base + (size_t)q * stride);
  const uint2 sc = a.scales ? *reinterpret_cast<const uint2*>(a.scales + (size_t)e * a.out + o)
                           : make_uint2(0x3C003C00u, 0x3C003C00u);  // fp16 1.0
  Quad<EXACT> s = v[0];
#pragma unroll
  for (int q = 1; q < 8; ++q)
    if (q < np) s.add(v[q]);
  for (int q0 = 8; q0 < np; q0 += 8) {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q].load(a.partial, base + (size_t)min(q0 + q, np - 1) * stride);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q0 + q < np) s.add(v[q]);
  }
  float r[4];
  if constexpr (EXACT) {
    // the exact sum of x * q, rounded to fp32 once (|sum| < 2^63 for any in < 2^31 / 255)
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (float)(s.v[j] + (int64_t)add) * mul;
  } else {
    r[0] = s.v.x;
    r[1] = s.v.y;
    r[2] = s.v.z;
    r[3] = s.v.w;
  }
  const uint32_t sw[2] = {sc.x, sc.y};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = r[j] * f16_bits_to_f32(sw[j >> 1] >> (16 * (j & 1)));
    if (a.gates) r[j] = r[j] * gate;
  }
  return make_float4(r[0], r[1], r[2], r[3]);
}

}  // namespace tq

// Host-side internal interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tq {

// ---- workspace layout -------------------------------------------------------------------
// [status 256 B][gemv partials][route: counts, offsets, hist, rank, pairs, items, n_items]
// [combine slot buffer]. Offsets are 256-byte aligned.
struct WsLayout {
  size_t status = 0;
  size_t partial = 0, partial_bytes = 0;
  size_t counts = 0, offsets = 0, hist = 0, rank = 0, pairs = 0, items = 0, n_items = 0;
  size_t route_bytes = 0;
  size_t slots = 0, slots_bytes = 0;
  size_t xprep = 0, rowsum = 0, xq = 0, xscale = 0, xsum = 0;
  size_t xa = 0, xs = 0;  // MXFP8 activation codes and block scales (TQ_FP8)
  size_t info = 0, rec = 0, desc = 0, list = 0, slot_info = 0, prank = 0;
  size_t total = 0;
  int groups = 1, route_blocks = 1, max_items = 0;
  int split_rows = 0;  // experts with at least this many slots have items placed by token range
  bool gemm = false;
};

constexpr int ROUTE_CHUNK = 2048;  // ids per route-count block
constexpr int GEMM_MT = 128;       // token rows per prefill work item
constexpr int GEMM_SPLIT = 256;    // slots from which an expert's items follow the token ranges
constexpr int GEMV_MAXK = 16;      // tokens per decode-batch chunk (one MFMA row block)

// ---- measurement hook (tq_time_kernel) -------------------------------------------------
// The hook's events for the main kernel about to be launched: both null unless the hook is
// armed (outside stream capture); taking them disarms it.
void take_kernel_events(hipEvent_t* start, hipEvent_t* stop);

// A main kernel's launch: with the hook armed, through hipExtLaunchKernelGGL, whose events
// take the dispatch's own start and end times (the kernel's duration, as a profiler reports
// it); else a plain launch.
template <typename F, typename... Args>
hipError_t launch_timed(F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  take_kernel_events(&e0, &e1);
  if (e0)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError();
}

// Records `msg` as this thread's last error (tq_last_error) and returns `code`.
int set_error(int code, const char* msg);

WsLayout ws_layout(int64_t T, int topk, int E, int out, int in, uint32_t flags,
                   bool mxfp4);

// ---- kernel launchers (return hipError_t) -------------------------------------------------
// Decode-batch plan + activation prep (gemv_plan.h, gemv_plan.hip).
struct PlanRec;
struct PlanArgs {
  const int32_t* ids;
  int N, E, topk;
  const uint8_t* bits;      // trellis widths, or null: every step costs 1 (MXFP4)
  const int64_t* code_off;  // trellis unit offsets (with bits)
  int64_t codes_bytes;      // trellis: size of the code buffer (a unit must lie inside)
  int64_t unit_bytes;       // MXFP4: expert e's unit is at e * unit_bytes; trellis: a
                            // unit's bytes per bit of width (out * in / 8)
  int groups, S;            // output groups per expert, steps per group (in / 64)
  int R;                    // routed slots one wave takes at most (a chunk of a slot
                            // list): a power of two
  int G;                    // the split's wave target
  int Gl;                   // launched GEMV waves (desc entries written)
  int32_t* info;            // [0] active experts, [1] waves with work, [2] cost bound T,
                            // [3] chunks
  PlanRec* rec;             // [E]
  int4* desc;               // [Gl]
  int32_t* list;            // [N]
  int4* slot_info;          // [N]
  int32_t* rank;            // [N] (used when N exceeds what the plan keeps in registers)
  uint32_t* status;
  // activation prep: x null = none
  const uint16_t* x;
  bool rotate;              // apply the 128-wide Hadamard (FORMAT F8) first
  const int8_t* signs;      // its signs, or null
  int T, in;
  uint32_t* xp;             // f16 pairs [T][in/16][8] (prefill GEMM operands)
  float2* rowsum;           // [T]: sum of the token's f16 values, and 2^-s
  uint32_t* xq;             // or int8 halves [T][2][in/16][8] (decode GEMV operands)
  float* xscale;            // [T]: 2^-e of each token
  int32_t* xsum;            // [T]: sum of each token's 16-bit integers
};
hipError_t launch_gemv_plan(const PlanArgs& a, hipStream_t s);
// x~ (bf16 [T][in]) times a per-token power of two 2^s -> f16 pairs [T][in/16][8] (word r of
// tile column c = [lo: x[16c + r + 8], hi: x[16c + r]]), and per token {sum of its f16
// values, 2^-s}: the activations of the trellis prefill GEMM. With rotate, x is first
// rotated as hadamard128 would (FORMAT F8).
hipError_t launch_activation_prep(const uint16_t* x, int64_t T, int in, uint32_t* xp,
                                  float2* rowsum, bool rotate, const int8_t* signs,
                                  hipStream_t s);

struct TrellisGemvArgs {
  int layout;           // 0: store order (F2); 1: read order (trellis_repack); 2: F2b units
  const uint32_t* codes;
  const uint32_t* xq;   // int8 halves [T][2][in/16][8] (the plan's prep)
  const PlanRec* rec;
  const int4* desc;     // [G]
  const int32_t* list;
  int64_t* partial;     // [in / 256][N][out]: the pieces' exact sums of each slot
  uint32_t x_bytes;     // size of xq in bytes (< 2^31)
  int N, out, in, topk;
  int G;                // pieces (desc entries) launched; two waves each
};
// The trellis GEMV's piece target (the plan's G): half the waves the GPU holds at once, up
// to 4 per SIMD; 0 on a HIP error.
int trellis_gemv_grid();
hipError_t launch_trellis_gemv(const TrellisGemvArgs& a, hipStream_t s);

struct PieceReduceArgs {
  const int4* slot_info;  // {expert, pieces, k, 0} or a SLOT_ code
  const void* partial;     // pieces: int64 exact sums (trellis) or fp32 (E8M0 stores)
  int exact;               // 1: int64 pieces of x * (q - 1), 0: fp32 pieces
  const uint16_t* scales;  // fp16 per output channel, or null
  const float* gates;   // or null
  const int32_t* xsum;  // [T]: added to each slot's sum (the signed-byte correction), or null
  const float* xscale;  // [T]: then multiplied, or null
  float* y;
  int N, out, topk, combine;
  int xdiv;  // a slot's activation row (xsum, xscale) is slot / xdiv: topk, or 1 when every
             // slot is a row of its own (the FFN's down projection)
  int qmax;  // pieces the partial buffer holds per slot
  int pre;   // pieces loaded before the slot's record arrives, 1 .. min(8, qmax)
};
constexpr int PIECE_MAX_TOPK = 64;  // largest topk (checked by the C ABI)
hipError_t launch_piece_reduce(const PieceReduceArgs& a, hipStream_t s);

struct TrellisGemmArgs {
  int layout;           // 0: store order (F2); 1: read order (trellis_repack); 2: F2b units
  const uint8_t* bits;
  const int64_t* code_off;
  const uint32_t* codes;
  int64_t codes_bytes;
  const uint16_t* scales;
  const uint32_t* xp;     // prepared activations: f16 pairs [T][in/16][8]
  const float2* rowsum;   // [T]: {sum of the token's f16 activations, 2^-s}
  uint32_t x_bytes;       // size of xp in bytes (< 2^31)
  const float* gates;
  const int32_t* pairs;
  const int32_t* items;
  const int32_t* n_items;
  float* y;
  uint32_t* status;
  int E, out, in, topk, groups, max_items;
};
hipError_t launch_trellis_gemm(const TrellisGemmArgs& a, hipStream_t s);

// FP8 trellis prefill (trellis_fp8.hip): MXFP8 activations (codes in the weight decoder's
// chunk order) times T16 values rounded to E4M3.
struct TrellisFp8GemmArgs {
  int layout;             // 0: store order (F2); 1: read order (trellis_repack); 2: F2b units
  const uint8_t* bits;
  const int64_t* code_off;
  const uint32_t* codes;
  int64_t codes_bytes;
  const uint16_t* scales;
  const uint8_t* xa;      // E4M3 codes [T][in] (tf8_prep order)
  uint32_t xa_bytes;      // < 2^31
  const uint8_t* xs;      // E8M0 scales [T][in / 32]
  uint32_t xs_bytes;
  const float* gates;
  const int32_t* pairs;
  const int32_t* items;
  const int32_t* n_items;
  float* y;
  uint32_t* status;
  int codebook;           // 0 T16 (F19), 1 mul1 (F20), 2 pmcgx (F21)
  int E, out, in, topk, groups, max_items;
};
hipError_t launch_tf8_prep(const uint16_t* x, int64_t rows, int n, bool rotate,
                           const int8_t* signs, uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_tf8_gemm(const TrellisFp8GemmArgs& a, hipStream_t s);
hipError_t launch_tf8_decode(const uint32_t* codes, int K, int out, int in, int16_t* q,
                             int codebook, hipStream_t s);

// Unit formats of the E8M0-scaled stores (mxfp4.hip).
constexpr int MX_FP4 = 0;     // MXFP4: E2M1 codes, a scale per row and 32 inputs
constexpr int MX_FP8B32 = 1;  // fp8b32: E4M3 codes, a scale per 32 x 32 block

struct Mxfp4GemvArgs {
  int fmt;               // MX_FP4 or MX_FP8B32
  int layout;            // 0: codes in store order; 1: repacked (mx_repack_kernel)
  const uint8_t* units;
  const uint16_t* x;     // bf16 [T][in]
  uint32_t x_bytes;      // size of x in bytes (< 2^31)
  const PlanRec* rec;
  const int4* desc;      // [G]
  const int32_t* list;
  float* partial;        // [in / 512][N][out]: the pieces of each slot
  int N, out, in, topk, G;
};
// The plan's wave target for the MXFP4 / fp8b32 GEMV (2 per SIMD, or fewer if the GPU
// holds fewer); 0 on a HIP error.
int mxfp4_gemv_grid(int fmt);
hipError_t launch_mxfp4_gemv(const Mxfp4GemvArgs& a, hipStream_t s);

struct Mxfp4GemmArgs {
  int fmt;     // MX_FP4 or MX_FP8B32
  int layout;  // 0: codes in store order; 1: repacked
  const uint8_t* units;
  const uint16_t* x;
  uint32_t x_bytes;  // size of x in bytes (< 2^31)
  const float* gates;
  const int32_t* pairs;
  const int32_t* items;
  const int32_t* n_items;
  float* y;
  int E, out, in, topk, groups, max_items;
};
// The prefill GEMM on the bf16 matrix cores, both formats (mxfp4_prefill.hip).
hipError_t launch_mxfp4_gemm(const Mxfp4GemmArgs& a, hipStream_t s);

// MXFP8 activations (FORMAT F18): bf16 [rows][n] -> E4M3 codes [rows][n] and E8M0 block scales
// [rows][n / 32].
hipError_t launch_mxfp8_prep(const uint16_t* x, int64_t rows, int n, uint8_t* codes,
                             uint8_t* scales, hipStream_t s);
// The MXFP4 prefill GEMM on the block-scaled fp8 x fp4 matrix cores (mx8.hip).
struct Mx8GemmArgs {
  int layout;            // 0: codes in store order; 1: repacked
  const uint8_t* units;
  const uint8_t* xa;     // E4M3 codes [T][in]
  uint32_t xa_bytes;     // < 2^31
  const uint8_t* xs;     // E8M0 scales [T][in / 32]
  uint32_t xs_bytes;
  const float* gates;
  const int32_t* pairs;
  const int32_t* items;
  const int32_t* n_items;
  float* y;
  int E, out, in, topk, groups, max_items;
};
hipError_t launch_mx8_gemm(const Mx8GemmArgs& a, hipStream_t s);

struct RouteArgs {
  const int32_t* ids;
  int64_t N;
  int E, out;
  int32_t* counts;    // [E]
  int32_t* offsets;   // [E+1]
  int32_t* hist;      // [blocks][E]
  int32_t* rank;      // [N]
  int32_t* pairs;     // [N]
  int32_t* items;     // [max_items][4] or null
  int32_t* n_items;   // [1] or null
  int split_rows;     // 0: items in expert order
  float* y_special;   // per-slot output rows for empty / invalid slots, or null
  uint32_t* status;
  int blocks, item_rows, max_items;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

hipError_t launch_combine(const float* slots, float* y, int64_t T, int topk, int out,
                          hipStream_t s);

hipError_t launch_hadamard(const uint16_t* x, uint16_t* y, int64_t rows, int64_t n,
                           const int8_t* signs, hipStream_t s);
// Output-side rotation (FORMAT F17) of fp32 rows [rows][out], in place; out % 128 == 0.
hipError_t launch_rotate_out(float* y, int64_t rows, int out, const int8_t* signs,
                             hipStream_t s);

// Copies every good unit of a trellis layer (width 2..4, inside codes_bytes, 16-byte
// aligned) from store order into the read order, at the same offset of dst.
hipError_t launch_trellis_repack(const uint8_t* bits, const int64_t* code_off,
                                 const uint32_t* codes, int64_t codes_bytes, int E, int out,
                                 int in, int from, uint32_t* dst, hipStream_t s);
hipError_t launch_trellis_decode(const uint32_t* codes, int K, int out, int in, int16_t* q,
                                 int path, hipStream_t s);
hipError_t launch_mxfp4_decode(const uint8_t* unit, int out, int in, uint16_t* w,
                               hipStream_t s);
// Copies E units of an E8M0-scaled store from store order into the GEMV's read order.
hipError_t launch_mx_repack(int fmt, const uint8_t* src, uint8_t* dst, int E, int out, int in,
                            hipStream_t s);
hipError_t launch_fp8b32_decode(const uint8_t* unit, int out, int in, uint16_t* w,
                                hipStream_t s);
// The routed FFN's middle step (ffn.hip): per slot, h = silu(g) * u from the fused gate/up
// outputs, rotated with the down layer's signs, converted to the down projection's operands.
struct FfnMidArgs {
  PieceReduceArgs gu;          // decode: the gate/up GEMV's pieces (xdiv = topk, no gates)
  const float* gu_rows;        // prefill: the gate/up GEMM's fp32 rows [N][2I]
  const int8_t* gu_out_signs;  // the gate/up output-side rotation still to apply, or null
  const int8_t* down_signs;    // the down projection's input signs, or null (all +1)
  int N, I;
  uint32_t* xq;                // decode: int8 halves [N][2][I/16][8]
  float* xscale;               // [N]: 2^-e
  int32_t* xsum;               // [N]: sum of the row's 16-bit integers
  uint32_t* xp;                // prefill: f16 pairs [N][I/16][8]
  float2* rowsum;              // [N]: {sum of the row's f16 values, 2^-e}
};
hipError_t launch_ffn_mid(const FfnMidArgs& a, bool decode, hipStream_t s);
// The FFN's two decode-batch plans (gate/up over T tokens, down over the T * topk slots as
// rows) and the gate/up activation prep, in one launch.
hipError_t launch_ffn_plan(const PlanArgs& gate_up, const PlanArgs& down, hipStream_t s);
hipError_t launch_nvfp4_transcode(const uint8_t* units, int E, int out, int in,
                                  uint8_t* codes, uint8_t* scales, float* scale2,
                                  uint8_t* status, hipStream_t s);

}  // namespace tq

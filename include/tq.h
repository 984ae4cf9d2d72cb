/*
 * tq.h — C ABI of the trellis / MXFP4 routed-expert library for AMD MI355X (gfx950).
 *
 * The library multiplies token activations by routed mixture-of-experts weights that stay
 * compressed in device memory and are decoded on the fly:
 *   - T16 bitshift-trellis codes, K = 2, 3 or 4 bits per weight (DeepSeek-V4.1-Flash-1017
 *     · dsx T16 page, "How T16 works": 16-bit window, multiply by 0x3A2F, add the
 *     product's two bytes; column-major positions in 16 x 16 tiles; per-output scales;
 *     128-wide Hadamard rotation of the inputs);
 *   - MXFP4 (E2M1 elements, one E8M0 scale per 32 inputs), the official expert store
 *     (DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores").
 * Every bit-level rule (tile order, bit order, tail-biting windows, nibble order, rounding)
 * is the one in FORMAT.md, rules F1-F14.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are device memory owned by the caller; the library never
 *     frees, allocates or retains them. Pointers marked "host" are read during the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is
 *     enqueued asynchronously on it. The compute entry points never synchronise, never
 *     allocate and never read routes back to the host, so they can be captured in a graph.
 *   - All host-side argument checks run before any HIP call. Return value 0 = success;
 *     a negative TQ_E* code otherwise, with a message from tq_last_error() (thread-local).
 *   - Device-side data errors (an expert id outside [-1, E), a width byte not in {2,3,4},
 *     a unit offset that is misaligned or puts the unit outside the code buffer) do not
 *     fault: the affected output slot is set to NaN and a sticky bit is set in the
 *     workspace status word (read with tq_device_status).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------------------ */
#define TQ_OK 0
#define TQ_EINVAL (-1)       /* bad shape, null pointer, bad K, bad flag                */
#define TQ_EUNSUPPORTED (-2) /* device is not gfx950                                    */
#define TQ_EALIGN (-3)       /* a pointer is not aligned as documented                  */
#define TQ_EWORKSPACE (-4)   /* workspace missing or smaller than tq_workspace_bytes()  */
#define TQ_EHIP (-5)         /* a HIP runtime call failed                               */

/* ---- flags of the expert GEMM calls -------------------------------------------------- */
#define TQ_AUTO 0u     /* prefill when T*topk > 16*E and its items, groups*ceil(T*topk/128),
                          number at least 256; else the decode batch (when it fits) */
#define TQ_GEMV 1u     /* force the decode-batch kernel (grouped GEMV, tokens in 8s)       */
#define TQ_GEMM 2u     /* force the prefill kernel (route bucketing + grouped MFMA GEMM)   */
#define TQ_COMBINE 4u  /* write y[T][out] = sum over k = 0..topk-1 (in order) of the slots */
#define TQ_ROTATE 8u   /* trellis only: x is not rotated; the call applies hadamard128 with */
                       /* the layer's signs first (same bits as calling hadamard128)        */
#define TQ_FP8 16u     /* trellis and MXFP4: FP8 matrix cores. The activations are         */
                       /* converted to MXFP8 (E4M3, one E8M0 scale per 32 inputs, as       */
                       /* mxfp8_quantize; FORMAT F18) and multiplied on the block-scaled    */
                       /* fp8 matrix cores with the stored E2M1 codes and their scales      */
                       /* (MXFP4), or with the T16 values rounded to E4M3 (trellis, FORMAT  */
                       /* F19); prefill mode (TQ_AUTO takes it; with TQ_GEMV an error)      */

/* ---- device status bits (tq_device_status) ------------------------------------------ */
#define TQ_STATUS_BAD_EXPERT 1u  /* an id outside [-1, E): that slot's output is NaN    */
#define TQ_STATUS_BAD_UNIT 2u    /* a width byte not in {2,3,4}, or an offset that is   */
                                 /* misaligned or puts the unit outside codes_bytes     */

/*
 * Code layouts. TQ_LAYOUT_STORE is the store order of the pages' units (trellis: FORMAT F2;
 * MXFP4 / fp8b32: HF orientation, rows of in/32 blocks). TQ_LAYOUT_GEMV is the same units
 * repacked once (trellis_repack, mxfp4_repack, fp8b32_repack) into the order the kernels
 * read them, so that a wave's loads stream contiguous memory. Both layouts give the same
 * results bit for bit.
 *   - trellis: the runs of 4 tiles that one 64-input step takes from each strip are
 *     step-major within each group of 8 strips (128 output channels): the 8 runs of a
 *     step, then the next step's; groups follow each other.
 *   - MXFP4 / fp8b32: every 128-input step of every strip of 16 output channels is one
 *     contiguous chunk (16 rows x 4 blocks); the scales keep their store order.
 */
#define TQ_LAYOUT_STORE 0
#define TQ_LAYOUT_GEMV 1
#define TQ_LAYOUT_UNIT128 2 /* trellis only: FORMAT F2b, the exlr8 page's units of 128     */
                            /* input channels (the down projection's units, "Layout"):    */
                            /* in/128 units of out x 128, each strip-major over its own   */
                            /* 8 tile columns, back to back                               */

/*
 * Trellis codebooks: how a state of the bit stream becomes a weight. One per layer (the
 * exlr8 page, "Stores": all encodes of a layer share its codebook).
 *   TQ_CODEBOOK_T16    the dsx T16 page's codebook ("How T16 works", item 1; FORMAT F5):
 *                      16-bit window times 0x3A2F mod 2^16, byte sum minus 255. Every mode.
 *   TQ_CODEBOOK_MUL1   exlr8's mul1 (FORMAT F20, a reading: 16-bit window times 0x83DCD12D
 *                      mod 2^32, byte sum minus 510). With TQ_FP8 only: operand E4M3(q/2)
 *                      with block scale 2.
 *   TQ_CODEBOOK_PMCGX  exlr8's pmcgx V2 L20 (FORMAT F21, a reading: 20-bit pair windows,
 *                      multipliers 0xCBAC1FED / 0xBCA14C51, masked fp16 halves summed and
 *                      rounded to E4M3). With TQ_FP8 only: the E4M3 weights are the operand.
 * mul1 and pmcgx layers use TQ_LAYOUT_STORE or TQ_LAYOUT_GEMV.
 */
#define TQ_CODEBOOK_T16 0
#define TQ_CODEBOOK_MUL1 1
#define TQ_CODEBOOK_PMCGX 2

/*
 * A trellis expert layer (FORMAT F1-F7, F12). Expert e's unit holds out*in*K/8 bytes at
 * byte offset code_off[e] of `codes`: 16 x 16 tiles in strip-major order (tile (to, ti)
 * at index to*(in/16)+ti), each tile 8*K little-endian uint32 words, bits read most
 * significant first, the state of position p being the 16-bit window at bit p*K read
 * circularly within the tile. Mixed widths may share one buffer (the pages' layers group
 * k2, k3, k4 units with ascending expert ids — DeepSeek-V4.1-Flash-1017 TrellisMX K2 Mix,
 * "What is stored"; any layout works through the per-expert descriptor).
 */
typedef struct tq_trellis_layer {
  int32_t E;                /* experts in the layer, 1 .. 4096                           */
  int32_t out;              /* output channels per expert, multiple of 16                 */
  int32_t in;               /* inputs per expert, multiple of 256                         */
  int32_t layout;           /* TQ_LAYOUT_STORE, TQ_LAYOUT_UNIT128 or (after              */
                            /* trellis_repack) TQ_LAYOUT_GEMV                             */
  const uint8_t* bits;      /* device [E]: K of each expert (2, 3 or 4)                   */
  const int64_t* code_off;  /* device [E]: byte offset of each unit in codes, 16-aligned  */
  const uint32_t* codes;    /* device: the units                                          */
  const uint16_t* scales;   /* device [E][out]: fp16 per-output-channel scales            */
  const int8_t* signs;      /* device [in]: +-1 rotation signs for TQ_ROTATE, or NULL     */
  int64_t codes_bytes;      /* bytes of `codes` (> 0): a unit must lie inside them         */
  const int8_t* out_signs;  /* device [out]: +-1 signs of the output-side rotation, or NULL  */
                            /* for none (FORMAT F17; out a multiple of 128 when given)     */
  int32_t codebook;         /* TQ_CODEBOOK_T16 (0), TQ_CODEBOOK_MUL1 or TQ_CODEBOOK_PMCGX  */
} tq_trellis_layer;

/*
 * An MXFP4 expert layer (FORMAT F9). E units back to back, each out*in/2 code bytes
 * (row = output channel, element 2j in the low nibble of byte j) followed by out*in/32
 * E8M0 scale bytes (row-major [out][in/32]).
 */
typedef struct tq_mxfp4_layer {
  int32_t E;                /* experts, 1 .. 4096                                         */
  int32_t out;              /* output channels, multiple of 16                            */
  int32_t in;               /* inputs, multiple of 512                                    */
  int32_t layout;           /* TQ_LAYOUT_STORE, or TQ_LAYOUT_GEMV after mxfp4_repack      */
  const uint8_t* units;     /* device: E * (out*in/2 + out*in/32) bytes, 16-aligned       */
} tq_mxfp4_layer;

/*
 * An fp8b32 expert layer (FORMAT F16; DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores": the
 * shared expert's store, FP8 E4M3 values with one E8M0 scale per 32 x 32 block, 656,000
 * bytes per 128 x 5120 unit). E units back to back, each out*in code bytes (row = output
 * channel, one E4M3 byte per weight) followed by (out/32)*(in/32) E8M0 scale bytes
 * (row-major [out/32][in/32]). The shared expert is a layer with E = 1 that every token
 * routes to (topk = 1, all ids 0).
 */
typedef struct tq_fp8b32_layer {
  int32_t E;                /* experts, 1 .. 4096                                         */
  int32_t out;              /* output channels, multiple of 32                            */
  int32_t in;               /* inputs, multiple of 512                                    */
  int32_t layout;           /* TQ_LAYOUT_STORE, or TQ_LAYOUT_GEMV after fp8b32_repack     */
  const uint8_t* units;     /* device: E * (out*in + out*in/1024) bytes, 16-aligned       */
} tq_fp8b32_layer;

/*
 * trellis_expert_gemm — routed activations x trellis-coded expert weights.
 *
 *   y[t][k][o] = g[t][k] * f32(scale_e[o]) * sum_i x[t][i] * q_e[i][o],  e = topk_ids[t][k]
 *
 * then, when L->out_signs is given, the output-side rotation of every 128 outputs of a slot
 * (or of a token with TQ_COMBINE), y <- s_out * ((H / sqrt(128)) y) (FORMAT F17;
 * DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores": the 128 x 128 Hadamard on both sides).
 *
 * (DeepSeek-V4.1-Flash-1017 · dsx T16 page, "How T16 works" items 1, 2 and 4; FORMAT
 * F5, F6, F10, F11.) q_e is decoded from the codes inside the kernels; it is never
 * materialised in memory.
 *   L         host: the layer description above.
 *   x         device bf16 [T][L->in], 16-byte aligned rows. Pass the rotated inputs
 *             (hadamard128 output) for layers encoded with rotated inputs, or the
 *             unrotated ones with TQ_ROTATE.
 *   T         tokens (>= 0; T == 0 is a successful no-op).
 *   topk_ids  device int32 [T][topk]; -1 = empty slot (output zero).
 *   topk_w    device fp32 [T][topk] gates, or NULL for gate 1.
 *   topk      slots per token, 1 .. 64.
 *   y         device fp32, 16-byte aligned: [T][topk][out], or [T][out] with TQ_COMBINE.
 *   flags     TQ_AUTO / TQ_GEMV / TQ_GEMM, optionally | TQ_COMBINE and | TQ_ROTATE
 *             (then x is the unrotated input; the rotation of hadamard128 with L->signs,
 *             or without signs when it is NULL, is applied while the activations are
 *             prepared, bit for bit as a separate hadamard128 call would).
 *   ws        device workspace of at least tq_workspace_bytes(T, topk, E, out, in, flags)
 *             bytes, 256-byte aligned, ZERO-FILLED BEFORE ITS FIRST USE. Every call leaves
 *             its counters at zero again, so a workspace is initialised once and reused;
 *             calls that share a workspace must be ordered on one stream.
 * Determinism (FORMAT F14): the same inputs give the same bits, whatever the launch
 * timing, and within one mode a slot gets the same bits whatever the rest of the batch
 * routes: a mixed-width layer equals separate single-width layers bit for bit (the
 * mixed-width kernels of the DeepSeek-V4.1-Flash-1017 TrellisMX K2 Mix page, intro, keep
 * each width's routes bit-identical to the single-rate kernels). The decode-batch mode
 * splits an expert's inputs among waves by the batch's whole routed work, but its piece
 * sums are exact integers, added exactly, so the split never shows in a result.
 * Operands (FORMAT F10): both modes put each token on a power-of-two scale of its own.
 * The prefill mode feeds the matrix cores f16 activations (exact for every element within
 * 2^31 of its token's largest magnitude); the decode-batch mode feeds 16-bit integers in
 * two int8 halves, whose rounding of elements far below the token's largest one is covered
 * by the parity bound. Any finite bf16 input is valid; a token with an infinite or NaN
 * element gets NaN in its slots.
 * With TQ_FP8 (FORMAT F19; DeepSeek-V4.1-Flash-1017 TrellisMX K2 Mix page, "Credits": the
 * trellis decoded straight into FP8 E4M3 tensor-core operands) the call computes
 *   y[t][k][o] = g[t][k] * f32(scale_e[o]) * sum_i xq[t][i] * E4M3(q_e[i][o]),
 * E4M3(q) the nearest E4M3 value to q (ties to even) and xq the MXFP8 values of x (after
 * the rotation with TQ_ROTATE), accumulated in fp32 by v_mfma_scale_f32_16x16x128_f8f6f4.
 * A 32-input block of a token holding an infinity or NaN makes that token's slots NaN.
 */
int trellis_expert_gemm(const tq_trellis_layer* L, const void* x, int64_t T,
                        const int32_t* topk_ids, const float* topk_w, int32_t topk,
                        float* y, uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/*
 * mxfp4_expert_gemm — routed activations x MXFP4 expert weights.
 *
 *   y[t][k][o] = g[t][k] * sum_i x[t][i] * E2M1[c_e[o][i]] * 2^(b_e[o][i/32] - 127)
 *
 * (DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores": FP4 E2M1 values with one E8M0 scale
 * per 32 inputs; FORMAT F9-F11.) Arguments as trellis_expert_gemm; no per-channel scale.
 */
int mxfp4_expert_gemm(const tq_mxfp4_layer* L, const void* x, int64_t T,
                      const int32_t* topk_ids, const float* topk_w, int32_t topk,
                      float* y, uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/*
 * With TQ_FP8 (FORMAT F18; DeepSeek-V4.1-Flash-1017 TrellisMX K2 Mix page, "Credits": FP8
 * E4M3 tensor-core operands), the result is the same contraction over the MXFP8 form of x:
 *   y[t][k][o] = g[t][k] * sum_i xq[t][i] * E2M1[c_e[o][i]] * 2^(b_e[o][i/32] - 127),
 *   xq[t][i] = E4M3[a[t][i]] * 2^(s[t][i/32] - 127)   (a, s: mxfp8_quantize of x)
 * accumulated in fp32 by v_mfma_scale_f32_16x16x128_f8f6f4.
 */

/*
 * mxfp8_quantize — the MXFP8 form of bf16 rows (FORMAT F18; OCP MX block scaling as in the
 * exlr8 page's "Stores"): per block of 32 consecutive inputs of a row, the E8M0 byte b with
 * max|x| / 2^(b - 127) in [128, 256) (127 for an all-zero block, 255 when the block holds an
 * infinity or NaN), and each element's E4M3 code, the nearest (ties to even) to
 * x * 2^(127 - b). The activation conversion of TQ_FP8, exposed on its own.
 *   x       device bf16 [rows][n], 16-byte aligned; n a multiple of 32.
 *   codes   device uint8 [rows][n], 16-byte aligned.   scales  device uint8 [rows][n / 32].
 */
int mxfp8_quantize(const void* x, int64_t rows, int64_t n, uint8_t* codes, uint8_t* scales,
                   void* stream);

/*
 * fp8b32_expert_gemm — routed activations x fp8b32 expert weights.
 *
 *   y[t][k][o] = g[t][k] * sum_i x[t][i] * E4M3[c_e[o][i]] * 2^(b_e[o/32][i/32] - 127)
 *
 * (DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores"; FORMAT F16, F10, F11.) Arguments,
 * workspace, modes and determinism as mxfp4_expert_gemm. The decoded weights are exact in
 * bf16 (the matrix-core operand) for scale bytes 10 .. 246; outside that range a product
 * below the smallest normal bf16 value or above the largest one is rounded by the
 * hardware conversion.
 */
int fp8b32_expert_gemm(const tq_fp8b32_layer* L, const void* x, int64_t T,
                       const int32_t* topk_ids, const float* topk_w, int32_t topk,
                       float* y, uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/*
 * hadamard128 — the 128-wide input rotation (FORMAT F8; DeepSeek-V4.1-Flash-1017 · dsx T16
 * page, "How T16 works", opening paragraph; exlr8 page, "Stores": per-layer signs).
 * Per block of 128 inputs: v = s * x; seven fp32 butterfly stages (strides 1..64,
 * (a, b) -> (a + b, a - b)); times fp32 0x3DB504F3; round to nearest-even bf16.
 *   x      device bf16 [rows][n], 16-byte aligned.
 *   y      device bf16 [rows][n], 16-byte aligned; may equal x (in place).
 *   rows   >= 0.   n  multiple of 128.
 *   signs  device int8 [n] of +1 / -1, or NULL for all +1.
 */
int hadamard128(const void* x, void* y, int64_t rows, int64_t n, const int8_t* signs,
                void* stream);

/*
 * route_bucket — stable counting sort of the (token, slot) pairs by expert id (FORMAT F11,
 * F14). The prefill path runs the same kernels internally; this entry point exposes them.
 *   topk_ids  device int32 [T][topk].
 *   counts    device int32 [E]: pairs per expert.
 *   offsets   device int32 [E+1]: exclusive prefix of counts.
 *   pairs     device int32 [T*topk]: flat slot indices t*topk+k of valid slots ordered by
 *             (expert, flat index); entries past offsets[E] are left unchanged.
 *   ws        workspace as for trellis_expert_gemm with TQ_GEMM.
 */
int route_bucket(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                 int32_t* counts, int32_t* offsets, int32_t* pairs, void* ws,
                 size_t ws_bytes, void* stream);

/*
 * trellis_decode — test hook: decode one trellis unit to its integer values
 *   q[o][i] = lo8(m) + hi8(m) - 255,  m = state * 0x3A2F mod 2^16
 * (DeepSeek-V4.1-Flash-1017 · dsx T16 page, "How T16 works", items 1 and 2: the 16-bit
 * window, the multiply by 0x3A2F, the byte sum, column-major positions in 16 x 16 tiles;
 * FORMAT F1-F5) with the device decoders the kernels run, read back from the operands the
 * matrix cores receive. Path 0: the decode-batch GEMV's column decoder and signed bytes
 * lo8(m) - 128 and hi8(m) - 128 (q = their sum + 1). Path 1: the prefill GEMM's decoders
 * (each half of a tile column on its own for K = 2 and 3, the whole column for K = 4) and
 * its byte sums q + 255 as f16 subnormals. Paths 2, 3, 4: the FP8 prefill's decoders
 * (TQ_FP8) of the T16 (FORMAT F19), mul1 (F20) and pmcgx (F21) codebooks; q[o][i] then
 * holds the E4M3 code byte (0..255) of the operand: E4M3(q) for T16, E4M3(q / 2) for mul1
 * (the exlr8 page, "Stores": mul1 0x83DCD12D, one weight per state; pmcgx V2 L20
 * 0xCBAC1FED / 0xBCA14C51, two weights per 20-bit state), the weight itself for pmcgx.
 *   codes  device, out*in*K/8 bytes, 16-byte aligned.   K in {2, 3, 4}.
 *   out    multiple of 16.   in  multiple of 64.
 *   q      device int16 [out][in] (HF orientation: row = output channel), 4-byte aligned.
 * Errors: TQ_EINVAL for a bad K, shape or path, TQ_EALIGN for misaligned pointers.
 */
int trellis_decode(const uint32_t* codes, int32_t K, int32_t out, int32_t in, int16_t* q,
                   int32_t path, void* stream);

/*
 * mxfp4_decode — test hook: decode one MXFP4 unit to bf16 [out][in],
 *   w[o][i] = E2M1[code] * 2^(b[o][i/32] - 127)
 * (DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores": E2M1 values, one E8M0 scale per 32
 * inputs, codes then scales; FORMAT F9) with the device decoder the MXFP4 kernels use.
 *   unit   device, out*in/2 + out*in/32 bytes, 16-byte aligned.   in multiple of 32.
 *   w      device bf16 [out][in], 16-byte aligned.
 */
int mxfp4_decode(const uint8_t* unit, int32_t out, int32_t in, uint16_t* w, void* stream);

/*
 * trellis_repack — copy a trellis layer's units from TQ_LAYOUT_STORE or TQ_LAYOUT_UNIT128
 * into TQ_LAYOUT_GEMV (see above): once, when a layer is loaded. Every unit with a good descriptor (width 2, 3 or
 * 4, 16-byte aligned, inside codes_bytes) is written at its own offset code_off[e] of dst;
 * other bytes of dst are left as they are.
 *   L      host: the layer, L->layout == TQ_LAYOUT_STORE or TQ_LAYOUT_UNIT128.
 *   dst    device, 16-byte aligned, L->codes_bytes bytes, not overlapping L->codes; use it
 *          as the codes of a layer with layout TQ_LAYOUT_GEMV (same bits, code_off, scales).
 */
int trellis_repack(const tq_trellis_layer* L, uint32_t* dst, void* stream);

/*
 * mxfp4_repack / fp8b32_repack — copy a layer's units from TQ_LAYOUT_STORE into
 * TQ_LAYOUT_GEMV (see above): once, when a layer is loaded.
 *   L      host: the layer, L->layout == TQ_LAYOUT_STORE.
 *   dst    device, 16-byte aligned, as many bytes as L->units holds, not overlapping it;
 *          use it as the units of a layer with layout TQ_LAYOUT_GEMV.
 */
int mxfp4_repack(const tq_mxfp4_layer* L, uint8_t* dst, void* stream);
int fp8b32_repack(const tq_fp8b32_layer* L, uint8_t* dst, void* stream);

/*
 * fp8b32_decode — test hook: decode one fp8b32 unit to bf16 [out][in],
 *   w[o][i] = E4M3[code] * 2^(b[o/32][i/32] - 127)
 * (DeepSeek-V4.1-Flash-1017 · exlr8 page, "Stores": FP8 E4M3 values with one E8M0 scale per
 * 32 x 32 block; FORMAT F16) with the device decoder the fp8b32 kernels use. out multiple
 * of 32, in multiple of 32, out*in < 2^31; unit and w 16-byte aligned.
 */
int fp8b32_decode(const uint8_t* unit, int32_t out, int32_t in, uint16_t* w, void* stream);

/*
 * trellis_expert_ffn — the routed expert FFN over trellis-coded projections (FORMAT F15;
 * DeepSeek-V4.1-Flash-1017 · exlr8 page, "Layout" and "Stores": every expert projection cut
 * into units of 128 intermediate channels, gate and up stored together, trellis units
 * rotated on both sides; dsx T16 page, "October 25 runtime checkpoint": fused gate/up
 * post-processing):
 *
 *   gu = gate_up_e(x~)       fp32, as trellis_expert_gemm (per-channel scales; then the
 *                            layer's output-side rotation when it has out_signs)
 *   g = gu[0 .. I-1], u = gu[I .. 2I-1]
 *   h = silu(g) * u,  silu(a) = a / (1 + e^-a)          fp32, never rounded to bf16
 *   v = (H / sqrt(128)) (down->signs * h) per 128-block  fp32 (no bf16 rounding), then the
 *                            mode's operand conversion (FORMAT F10)
 *   z = down_e(v)            (then down's output-side rotation when it has out_signs)
 *   y[t] = sum over k = 0..topk-1, in order, of g[t][k] * z[t][k]
 *
 *   gate_up   host: trellis layer with out = 2I (the gate's I channels, then the up's),
 *             in = H.
 *   down      host: trellis layer with out = H, in = I, same E; TQ_LAYOUT_UNIT128 stores it
 *             as the page's units of 128 intermediate channels.
 *   x         device bf16 [T][H]; with TQ_ROTATE the unrotated input (gate_up->signs rotate
 *             it), else the rotated one.
 *   topk_ids, topk_w, topk   as trellis_expert_gemm.
 *   y         device fp32 [T][H], 16-byte aligned.
 *   flags     TQ_AUTO / TQ_GEMV / TQ_GEMM (both projections), | TQ_ROTATE.
 *   ws        device workspace of tq_ffn_workspace_bytes(T, topk, E, H, I, flags) bytes,
 *             256-byte aligned, zero-filled before its first use (as for trellis_expert_gemm);
 *             the status word of tq_device_status is its first word.
 * H and I are multiples of 256, I at most 4096. The decode-batch mode runs five launches:
 * both plans with the gate/up activation prep, the gate/up GEMV, the middle step (the
 * gate/up reduction, SwiGLU, the intermediate's rotation and the down operands, one
 * workgroup per slot), the down GEMV, the down reduction with the combine.
 */
int trellis_expert_ffn(const tq_trellis_layer* gate_up, const tq_trellis_layer* down,
                       const void* x, int64_t T, const int32_t* topk_ids, const float* topk_w,
                       int32_t topk, float* y, uint32_t flags, void* ws, size_t ws_bytes,
                       void* stream);

/* Workspace bytes trellis_expert_ffn needs (0 for invalid sizes). */
size_t tq_ffn_workspace_bytes(int64_t T, int32_t topk, int32_t E, int32_t H, int32_t I,
                              uint32_t flags);

/*
 * mxfp4_to_nvfp4 — transcode an MXFP4 layer to NVFP4 (FORMAT F13; DeepSeek-V4.1-Flash-1017
 * NVFP4 page, "Model": 16-element blocks with E4M3 scales under one fp32 scale per tensor).
 * Per unit e (one expert's out x in weights), with bmax its largest E8M0 scale byte:
 *   codes[e]    = the unit's E2M1 nibbles, unchanged (out*in/2 bytes);
 *   scales[e]   = E4M3 [out][in/16]: both 16-blocks of the 32-block with byte b get
 *                 2^(b - bmax + 8), or 0 when bmax - b > 17 (below E4M3's smallest power of
 *                 two: the block's values flush to zero), or 0x7F (NaN) when b = 255;
 *   scale2[e]   = fp32 2^(bmax - 135), so that scale * scale2 = 2^(b - 127);
 *   status[e]   = 1 if the transcode is exact (bmax - b <= 17 for every block), 0 if some
 *                 block flushed, 2 if the unit holds a NaN scale byte.
 *   L        host: the MXFP4 layer (E up to 65535).
 *   codes    device, E * out*in/2 bytes, 16-byte aligned.
 *   scales   device, E * out*in/16 bytes, 16-byte aligned.
 *   scale2   device fp32 [E].   status  device uint8 [E].
 * The outputs must not overlap the layer. Asynchronous on `stream`.
 */
int mxfp4_to_nvfp4(const tq_mxfp4_layer* L, uint8_t* codes, uint8_t* scales, float* scale2,
                   uint8_t* status, void* stream);

/*
 * trellis_expert_gemm_noalloc — trellis_expert_gemm for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Arguments, results and errors as trellis_expert_gemm, without ws / ws_bytes:
 * the workspace is a static device array of TQ_NOALLOC_SCRATCH_BYTES bytes that each GPU
 * the library runs on holds until the process ends (looked up once per device, its status
 * word zeroed by a small kernel on the first call's stream). The call allocates nothing.
 *   - A call whose tq_workspace_bytes(T, topk, E, out, in, flags) exceeds
 *     TQ_NOALLOC_SCRATCH_BYTES returns TQ_EWORKSPACE before any GPU work (32 MiB holds a
 *     decode batch of 1,024 slots of 128 x 5120 units, or a prefill of about 2,500 tokens).
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents:
 *     calls that overlap on one GPU (on different streams, or from different threads
 *     without ordering) race. Order them on one stream.
 *   - Data errors give NaN slots as in trellis_expert_gemm; the status word that records
 *     them is not exposed.
 */
#define TQ_NOALLOC_SCRATCH_BYTES (32u << 20)
int trellis_expert_gemm_noalloc(const tq_trellis_layer* L, const void* x, int64_t T,
                                const int32_t* topk_ids, const float* topk_w, int32_t topk,
                                float* y, uint32_t flags, void* stream);

/* Workspace bytes the expert GEMM calls (and route_bucket with flags TQ_GEMM) need. */
size_t tq_workspace_bytes(int64_t T, int32_t topk, int32_t E, int32_t out, int32_t in,
                          uint32_t flags);

/* Message of the last error on this thread ("" if none). */
const char* tq_last_error(void);

/* Synchronises `stream`, copies the workspace status word to *flags_out and clears it. */
int tq_device_status(void* ws, void* stream, uint32_t* flags_out);

/*
 * Measurement hook, for benchmarks and profilers (not part of the computation). After this
 * call, the calling thread's next trellis_expert_gemm, mxfp4_expert_gemm or
 * trellis_expert_ffn times its main kernel (the grouped GEMV in the decode-batch mode, the
 * down projection's GEMV in the FFN, the grouped GEMM in the prefill mode): the kernel is
 * launched with hipExtLaunchKernel, which sets `start` and `stop` to the dispatch's own
 * start and end; under stream capture they are recorded on the stream right before and
 * after the launch instead (event-record nodes of the graph). The hook is then cleared.
 * start and stop are hipEvent_t passed as void*, created by the caller with timing
 * enabled. NULL, NULL clears the hook.
 */
int tq_time_kernel(void* start, void* stop);

/* Library version, major * 10000 + minor * 100 + patch. */
int tq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */

// C ABI of the library (include/tq.h): argument checks, workspace layout and dispatch.
// Every check runs before the first HIP call of an entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "tq.h"
#include "gemv_plan.h"
#include "tq_internal.h"

namespace {

thread_local std::string g_error;
thread_local hipEvent_t g_time_start = nullptr, g_time_stop = nullptr;
thread_local bool g_time_armed = false;     // the next launch_timed takes the events
thread_local bool g_time_recorded = false;  // stream capture: events recorded around it

// Measurement hook (tq_time_kernel), around the next main kernel launch. Outside stream
// capture the launch itself records the kernel's start and end into the events
// (launch_timed); under capture the events are recorded on the stream before and after it.
hipError_t time_begin(hipStream_t s) {
  if (!g_time_start) return hipSuccess;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  hipError_t err = hipStreamIsCapturing(s, &st);
  if (err != hipSuccess) return err;
  if (st == hipStreamCaptureStatusNone) {
    g_time_armed = true;
    return hipSuccess;
  }
  g_time_recorded = true;
  return hipEventRecord(g_time_start, s);
}
hipError_t time_end(hipStream_t s) {
  hipError_t err = hipSuccess;
  if (g_time_recorded) {
    err = hipEventRecord(g_time_stop, s);
  } else if (g_time_armed) {  // no kernel was launched (an empty launch): zero duration
    err = hipEventRecord(g_time_start, s);
    if (err == hipSuccess) err = hipEventRecord(g_time_stop, s);
  }
  g_time_start = g_time_stop = nullptr;
  g_time_armed = g_time_recorded = false;
  return err;
}

}  // namespace

void tq::take_kernel_events(hipEvent_t* start, hipEvent_t* stop) {
  if (g_time_armed) {
    *start = g_time_start;
    *stop = g_time_stop;
    g_time_armed = false;
    g_time_start = g_time_stop = nullptr;
  } else {
    *start = *stop = nullptr;
  }
}

namespace {

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return TQ_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int hip_fail(hipError_t err, const char* what) {
  return fail(TQ_EHIP, "%s: %s", what, hipGetErrorString(err));
}

// gfx950 check, cached per device.
int check_device() {
  static int cache[64];  // 0 unknown, 1 ok, 2 unsupported
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
  if (dev >= 0 && dev < 64 && cache[dev] == 1) return TQ_OK;
  hipDeviceProp_t prop;
  err = hipGetDeviceProperties(&prop, dev);
  if (err != hipSuccess) return hip_fail(err, "hipGetDeviceProperties");
  const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) cache[dev] = good ? 1 : 2;
  if (!good) return fail(TQ_EUNSUPPORTED, "device %d is %s; this library is built for gfx950",
                         dev, prop.gcnArchName);
  return TQ_OK;
}

bool flags_valid(uint32_t flags) {
  return (flags & ~31u) == 0 && (flags & 3u) != 3u;
}

// The prefill GEMM pays off when experts average more than 16 routed slots and its items
// (128 routed rows of one group) are enough to give every compute unit of the GPU one;
// otherwise the decode batch, whose waves take 8 or 16 slots each, spreads the work wider.
constexpr int64_t GEMM_MIN_ITEMS = 256;

bool use_gemm(int64_t T, int topk, int E, int groups, uint32_t flags) {
  const uint32_t mode = flags & 3u;
  if (mode == TQ_GEMV) return false;
  if (mode == TQ_GEMM || (flags & TQ_FP8)) return true;
  const int64_t N = T * topk;
  return N > 16LL * E && (int64_t)groups * ((N + 127) / 128) >= GEMM_MIN_ITEMS;
}

int check_routes(int64_t T, int topk, const void* ids) {
  if (T < 0) return fail(TQ_EINVAL, "T = %lld is negative", (long long)T);
  if (topk < 1 || topk > 64) return fail(TQ_EINVAL, "topk = %d is outside 1..64", topk);
  if (T * (int64_t)topk >= (int64_t)1 << 31)
    return fail(TQ_EINVAL, "T * topk = %lld does not fit in int32", (long long)(T * topk));
  if (T > 0 && !ids) return fail(TQ_EINVAL, "topk_ids is NULL");
  return TQ_OK;
}

int check_io(int64_t T, const void* x, const float* y) {
  if (T == 0) return TQ_OK;
  if (!x || !y) return fail(TQ_EINVAL, "x or y is NULL");
  if (!aligned(x, 16) || !aligned(y, 16))
    return fail(TQ_EALIGN, "x and y must be 16-byte aligned");
  return TQ_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(TQ_EWORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(TQ_EALIGN, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(TQ_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return TQ_OK;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace

namespace tq {

int set_error(int code, const char* msg) { return fail(code, "%s", msg); }

// Routed slots one decode-batch wave takes: the token rows of its matrix-core operations.
int gemv_rows(bool mxfp4) { return mxfp4 ? 16 : 8; }

// Pieces the reduction loads ahead of each slot's record. When the (group, expert) pairs
// alone can fill the GEMV grid the split is expected to give one piece per slot, and planes
// past the first would be stale reads; else up to 8 are fetched ahead. Only speed depends on
// it: pieces past a slot's count are never added.
static int reduce_prefetch(int64_t N, int E, int groups, int grid, int qmax) {
  if ((int64_t)groups * std::min<int64_t>(E, N) >= grid) return 1;
  return std::max(1, std::min(8, qmax));
}

// Upper bound on the decode-batch plan's (group, chunk) pairs, each of which gets at least
// one wave: every active expert has ceil(cnt / R) <= cnt / R + 1 chunks.
int64_t gemv_chunk_bound(int64_t N, int E, int groups, bool mxfp4) {
  const int R = gemv_rows(mxfp4);
  return (int64_t)groups * ((int64_t)E + (N + R - 1) / R);
}

WsLayout ws_layout(int64_t T, int topk, int E, int out, int in, uint32_t flags, bool mxfp4) {
  WsLayout L;
  const int64_t N = T * topk;
  L.groups = (out + 127) / 128;
  L.gemm = use_gemm(T, topk, E, L.groups, flags);
  // a decode batch gives every active expert group and chunk at least one piece of its own
  if ((flags & 3u) == TQ_AUTO && gemv_chunk_bound(N, E, L.groups, mxfp4) > tq::GEMV_MAX_G)
    L.gemm = true;
  size_t off = 256;  // status word
  if (!L.gemm) {
    // planned decode batch: plan records, prepared activations (trellis), per-piece partial
    // sums (at most in / 256 pieces per slot for trellis steps of 64 inputs, in / 512 for
    // MXFP4 steps of 128)
    const size_t Q = (size_t)in / (mxfp4 ? 512 : 256);
    L.info = off;
    off += 256;
    L.rec = off;
    off += round_up((size_t)E * sizeof(tq::PlanRec), 256);
    L.desc = off;
    off += round_up((size_t)tq::GEMV_MAX_G * 16, 256);
    L.list = off;
    off += round_up((size_t)N * 4, 256);
    L.slot_info = off;
    off += round_up((size_t)N * 16, 256);
    L.prank = off;
    off += round_up((size_t)N * 4, 256);
    if (!mxfp4) {
      L.xq = off;
      off += round_up((size_t)T * in * 4, 256);
      L.xscale = off;
      off += round_up((size_t)T * 4, 256);
      L.xsum = off;
      off += round_up((size_t)T * 4, 256);
    }
    L.partial = off;
    L.partial_bytes = round_up(Q * N * out * (mxfp4 ? 4 : 8), 256);  // int64 trellis sums
    off += L.partial_bytes;
  } else {
    L.route_blocks = (int)((N + ROUTE_CHUNK - 1) / ROUTE_CHUNK);
    // items placed by token range only where rows are shared between experts' items (a
    // token has several experts), for up to 1024 experts
    L.split_rows = (topk > 1 && E <= 1024) ? GEMM_SPLIT : 0;
    L.max_items = (int)((N + GEMM_MT - 1) / GEMM_MT) + E;
    const size_t start = off;
    L.counts = off;
    off += round_up((size_t)E * 4, 256);
    L.offsets = off;
    off += round_up((size_t)(E + 1) * 4, 256);
    L.hist = off;
    off += round_up((size_t)L.route_blocks * E * 4, 256);
    L.rank = off;
    off += round_up((size_t)N * 4, 256);
    L.pairs = off;
    off += round_up((size_t)N * 4, 256);
    L.items = off;
    off += round_up((size_t)L.max_items * 16, 256);
    L.n_items = off;
    off += 256;
    L.route_bytes = off - start;
    if (!mxfp4 && !(flags & TQ_FP8)) {  // the trellis GEMM reads prepared f16 activations
      L.xprep = off;
      off += round_up((size_t)T * in * 2, 256);
      L.rowsum = off;
      off += round_up((size_t)T * 8, 256);
    } else if (flags & TQ_FP8) {  // MXFP8 activations
      L.xa = off;
      off += round_up((size_t)T * in, 256);
      L.xs = off;
      off += round_up((size_t)T * in / 32, 256);
    }
  }
  if ((flags & TQ_COMBINE) && L.gemm) {
    L.slots = off;
    L.slots_bytes = round_up((size_t)N * out * 4, 256);
    off += L.slots_bytes;
  }
  L.total = off;
  return L;
}

}  // namespace tq

extern "C" {

size_t tq_workspace_bytes(int64_t T, int32_t topk, int32_t E, int32_t out, int32_t in,
                          uint32_t flags) {
  if (T < 0 || topk < 1 || E < 1 || out < 16 || in < 256) return 0;
  const tq::WsLayout a = tq::ws_layout(T, topk, E, out, in, flags, false);
  const tq::WsLayout b = tq::ws_layout(T, topk, E, out, in, flags, true);
  return a.total > b.total ? a.total : b.total;
}

const char* tq_last_error(void) { return g_error.c_str(); }

int tq_time_kernel(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr))
    return fail(TQ_EINVAL, "tq_time_kernel needs both events or neither");
  g_time_start = static_cast<hipEvent_t>(start);
  g_time_stop = static_cast<hipEvent_t>(stop);
  return ok();
}

int tq_version(void) { return 100; }

int tq_device_status(void* ws, void* stream, uint32_t* flags_out) {
  if (!ws || !flags_out) return fail(TQ_EINVAL, "ws and flags_out must not be NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipStreamSynchronize(s);
  if (err != hipSuccess) return hip_fail(err, "hipStreamSynchronize");
  uint32_t v = 0;
  err = hipMemcpy(&v, ws, 4, hipMemcpyDeviceToHost);
  if (err != hipSuccess) return hip_fail(err, "hipMemcpy");
  err = hipMemset(ws, 0, 4);
  if (err != hipSuccess) return hip_fail(err, "hipMemset");
  *flags_out = v;
  return ok();
}

int hadamard128(const void* x, void* y, int64_t rows, int64_t n, const int8_t* signs,
                void* stream) {
  if (rows < 0) return fail(TQ_EINVAL, "rows = %lld is negative", (long long)rows);
  if (n <= 0 || n % 128) return fail(TQ_EINVAL, "n = %lld is not a positive multiple of 128",
                                     (long long)n);
  if (rows == 0) return ok();
  if (!x || !y) return fail(TQ_EINVAL, "x or y is NULL");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(TQ_EALIGN, "x and y must be 16-byte aligned");
  if (signs && !aligned(signs, 8)) return fail(TQ_EALIGN, "signs must be 8-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  hipError_t err = tq::launch_hadamard(static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y),
                                       rows, n, signs, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "hadamard128 launch");
  return ok();
}

int mxfp8_quantize(const void* x, int64_t rows, int64_t n, uint8_t* codes, uint8_t* scales,
                   void* stream) {
  if (rows < 0) return fail(TQ_EINVAL, "rows = %lld is negative", (long long)rows);
  if (n <= 0 || n % 32) return fail(TQ_EINVAL, "n = %lld is not a positive multiple of 32",
                                    (long long)n);
  if (n >= ((int64_t)1 << 30)) return fail(TQ_EINVAL, "n = %lld is too large", (long long)n);
  if (rows == 0) return ok();
  if (!x || !codes || !scales) return fail(TQ_EINVAL, "x, codes or scales is NULL");
  if (!aligned(x, 16) || !aligned(codes, 16))
    return fail(TQ_EALIGN, "x and codes must be 16-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  hipError_t err = tq::launch_mxfp8_prep(static_cast<const uint16_t*>(x), rows, (int)n, codes,
                                         scales, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "mxfp8_quantize launch");
  return ok();
}

int trellis_decode(const uint32_t* codes, int32_t K, int32_t out, int32_t in, int16_t* q,
                   int32_t path, void* stream) {
  if (K < 2 || K > 4) return fail(TQ_EINVAL, "K = %d is not 2, 3 or 4", K);
  if (out <= 0 || out % 16) return fail(TQ_EINVAL, "out = %d is not a positive multiple of 16", out);
  if (in <= 0 || in % 64) return fail(TQ_EINVAL, "in = %d is not a positive multiple of 64", in);
  if (path < 0 || path > 4) return fail(TQ_EINVAL, "path = %d is not 0 .. 4", path);
  if (!codes || !q) return fail(TQ_EINVAL, "codes or q is NULL");
  if (!aligned(codes, 16)) return fail(TQ_EALIGN, "codes must be 16-byte aligned");
  if (!aligned(q, 4)) return fail(TQ_EALIGN, "q must be 4-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  hipError_t err =
      path >= 2 ? tq::launch_tf8_decode(codes, K, out, in, q, path - 2,
                                        static_cast<hipStream_t>(stream))
                : tq::launch_trellis_decode(codes, K, out, in, q, path,
                                            static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "trellis_decode launch");
  return ok();
}

int mxfp4_decode(const uint8_t* unit, int32_t out, int32_t in, uint16_t* w, void* stream) {
  if (out <= 0) return fail(TQ_EINVAL, "out = %d is not positive", out);
  if (in <= 0 || in % 32) return fail(TQ_EINVAL, "in = %d is not a positive multiple of 32", in);
  if (!unit || !w) return fail(TQ_EINVAL, "unit or w is NULL");
  if (!aligned(unit, 16) || !aligned(w, 16)) return fail(TQ_EALIGN, "unit and w must be 16-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  hipError_t err = tq::launch_mxfp4_decode(unit, out, in, w, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "mxfp4_decode launch");
  return ok();
}

int fp8b32_decode(const uint8_t* unit, int32_t out, int32_t in, uint16_t* w, void* stream) {
  if (out <= 0 || out % 32) return fail(TQ_EINVAL, "out = %d is not a positive multiple of 32", out);
  if (in <= 0 || in % 32) return fail(TQ_EINVAL, "in = %d is not a positive multiple of 32", in);
  if ((int64_t)out * in >= ((int64_t)1 << 31)) return fail(TQ_EINVAL, "out * in must stay below 2^31");
  if (!unit || !w) return fail(TQ_EINVAL, "unit or w is NULL");
  if (!aligned(unit, 16) || !aligned(w, 16)) return fail(TQ_EALIGN, "unit and w must be 16-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  hipError_t err = tq::launch_fp8b32_decode(unit, out, in, w, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "fp8b32_decode launch");
  return ok();
}

int mxfp4_to_nvfp4(const tq_mxfp4_layer* L, uint8_t* codes, uint8_t* scales, float* scale2,
                   uint8_t* status, void* stream) {
  if (!L) return fail(TQ_EINVAL, "layer is NULL");
  if (L->E < 1 || L->E > 65535) return fail(TQ_EINVAL, "E = %d is outside 1..65535", L->E);
  if (L->out <= 0 || L->out % 16) return fail(TQ_EINVAL, "out = %d is not a positive multiple of 16", L->out);
  if (L->in <= 0 || L->in % 512) return fail(TQ_EINVAL, "in = %d is not a positive multiple of 512", L->in);
  if (L->layout != TQ_LAYOUT_STORE)
    return fail(TQ_EINVAL, "the transcode reads units in TQ_LAYOUT_STORE (layout = %d)", L->layout);
  if ((int64_t)L->out * L->in / 2 >= ((int64_t)1 << 31))
    return fail(TQ_EINVAL, "out * in is too large");
  if (!L->units || !codes || !scales || !scale2 || !status)
    return fail(TQ_EINVAL, "a pointer is NULL");
  if (!aligned(L->units, 16) || !aligned(codes, 16) || !aligned(scales, 16))
    return fail(TQ_EALIGN, "units, codes and scales must be 16-byte aligned");
  if (!aligned(scale2, 4)) return fail(TQ_EALIGN, "scale2 must be 4-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  hipError_t err = tq::launch_nvfp4_transcode(L->units, L->E, L->out, L->in, codes, scales,
                                              scale2, status, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "mxfp4_to_nvfp4 launch");
  return ok();
}

int route_bucket(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E, int32_t* counts,
                 int32_t* offsets, int32_t* pairs, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_routes(T, topk, topk_ids);
  if (rc) return rc;
  if (E < 1 || E > 4096) return fail(TQ_EINVAL, "E = %d is outside 1..4096", E);
  if (!counts || !offsets || (T > 0 && !pairs)) return fail(TQ_EINVAL, "an output is NULL");
  const tq::WsLayout L = tq::ws_layout(T, topk, E, 16, 256, TQ_GEMM, false);
  rc = check_ws(ws, ws_bytes, L.total);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  tq::RouteArgs r{};
  r.ids = topk_ids;
  r.N = T * topk;
  r.E = E;
  r.out = 16;
  r.counts = counts;
  r.offsets = offsets;
  r.hist = at<int32_t>(ws, L.hist);
  r.rank = at<int32_t>(ws, L.rank);
  r.pairs = pairs;
  r.items = nullptr;
  r.n_items = nullptr;
  r.y_special = nullptr;
  r.status = at<uint32_t>(ws, L.status);
  r.blocks = L.route_blocks;
  r.item_rows = tq::GEMM_MT;
  r.max_items = 0;
  r.split_rows = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (r.N == 0) {
    // no slots: counts and offsets are all zero (a fill kernel, so graphs may capture it)
    err = tq::launch_fill_i32(counts, E, 0, s);
    if (err == hipSuccess) err = tq::launch_fill_i32(offsets, E + 1, 0, s);
  } else {
    err = tq::launch_route(r, s);
  }
  if (err != hipSuccess) return hip_fail(err, "route_bucket launch");
  return ok();
}

namespace {

static int check_trellis_layer(const tq_trellis_layer* L) {
  if (!L) return fail(TQ_EINVAL, "layer is NULL");
  if (L->E < 1 || L->E > 4096) return fail(TQ_EINVAL, "E = %d is outside 1..4096", L->E);
  if (L->out <= 0 || L->out % 16) return fail(TQ_EINVAL, "out = %d is not a positive multiple of 16", L->out);
  if (L->in <= 0 || L->in % 256) return fail(TQ_EINVAL, "in = %d is not a positive multiple of 256", L->in);
  if (L->layout != TQ_LAYOUT_STORE && L->layout != TQ_LAYOUT_GEMV && L->layout != TQ_LAYOUT_UNIT128)
    return fail(TQ_EINVAL, "layout = %d is not TQ_LAYOUT_STORE, TQ_LAYOUT_GEMV or TQ_LAYOUT_UNIT128",
                L->layout);
  if (L->layout == TQ_LAYOUT_UNIT128 && L->in % 128)
    return fail(TQ_EINVAL, "TQ_LAYOUT_UNIT128 needs in to be a multiple of 128 (in = %d)", L->in);
  if (!L->bits || !L->code_off || !L->codes || !L->scales)
    return fail(TQ_EINVAL, "a layer pointer is NULL");
  if (!aligned(L->codes, 16)) return fail(TQ_EALIGN, "codes must be 16-byte aligned");
  if (!aligned(L->code_off, 8)) return fail(TQ_EALIGN, "code_off must be 8-byte aligned");
  if (!aligned(L->scales, 2)) return fail(TQ_EALIGN, "scales must be 2-byte aligned");
  if (L->codes_bytes <= 0) return fail(TQ_EINVAL, "codes_bytes = %lld is not positive",
                                       (long long)L->codes_bytes);
  if (L->out_signs && L->out % 128)
    return fail(TQ_EINVAL, "an output-side rotation needs out to be a multiple of 128 (out = %d)",
                L->out);
  if (L->out_signs && !aligned(L->out_signs, 4))
    return fail(TQ_EALIGN, "out_signs must be 4-byte aligned");
  if (L->codebook < TQ_CODEBOOK_T16 || L->codebook > TQ_CODEBOOK_PMCGX)
    return fail(TQ_EINVAL, "codebook = %d is not TQ_CODEBOOK_T16, _MUL1 or _PMCGX", L->codebook);
  if (L->codebook != TQ_CODEBOOK_T16 && L->layout == TQ_LAYOUT_UNIT128)
    return fail(TQ_EINVAL, "TQ_LAYOUT_UNIT128 is read for T16 layers only");
  return TQ_OK;
}

static int check_mxfp4_layer(const tq_mxfp4_layer* L) {
  if (!L) return fail(TQ_EINVAL, "layer is NULL");
  if (L->E < 1 || L->E > 4096) return fail(TQ_EINVAL, "E = %d is outside 1..4096", L->E);
  if (L->out <= 0 || L->out % 16) return fail(TQ_EINVAL, "out = %d is not a positive multiple of 16", L->out);
  if (L->in <= 0 || L->in % 512) return fail(TQ_EINVAL, "in = %d is not a positive multiple of 512", L->in);
  if (L->layout != TQ_LAYOUT_STORE && L->layout != TQ_LAYOUT_GEMV)
    return fail(TQ_EINVAL, "layout = %d is not TQ_LAYOUT_STORE or TQ_LAYOUT_GEMV", L->layout);
  if (!L->units) return fail(TQ_EINVAL, "units is NULL");
  if (!aligned(L->units, 16)) return fail(TQ_EALIGN, "units must be 16-byte aligned");
  return TQ_OK;
}

static int check_fp8b32_layer(const tq_fp8b32_layer* L) {
  if (!L) return fail(TQ_EINVAL, "layer is NULL");
  if (L->E < 1 || L->E > 4096) return fail(TQ_EINVAL, "E = %d is outside 1..4096", L->E);
  if (L->out <= 0 || L->out % 32) return fail(TQ_EINVAL, "out = %d is not a positive multiple of 32", L->out);
  if (L->in <= 0 || L->in % 512) return fail(TQ_EINVAL, "in = %d is not a positive multiple of 512", L->in);
  if (L->layout != TQ_LAYOUT_STORE && L->layout != TQ_LAYOUT_GEMV)
    return fail(TQ_EINVAL, "layout = %d is not TQ_LAYOUT_STORE or TQ_LAYOUT_GEMV", L->layout);
  if (!L->units) return fail(TQ_EINVAL, "units is NULL");
  if (!aligned(L->units, 16)) return fail(TQ_EALIGN, "units must be 16-byte aligned");
  return TQ_OK;
}

// Bytes of one unit of the E8M0-scaled stores.
static int64_t mx_unit_bytes(int fmt, int out, int in) {
  if (fmt == tq::MX_FP8B32) return (int64_t)out * in + (int64_t)(out / 32) * (in / 32);
  return (int64_t)out * in / 2 + (int64_t)out * in / 32;
}

// Shared front half of the expert GEMM calls. mx_unit: bytes per unit of an E8M0-scaled
// store, 0 for trellis layers.
static int common_checks(int E, int out, int in, const void* x, int64_t T, const int32_t* ids,
                  int32_t topk, float* y, uint32_t flags, void* ws, size_t ws_bytes,
                  int64_t mx_unit, tq::WsLayout* layout) {
  const bool mxfp4 = mx_unit != 0;
  int rc = check_routes(T, topk, ids);
  if (rc) return rc;
  if (!flags_valid(flags)) return fail(TQ_EINVAL, "flags = 0x%x is not valid", flags);
  rc = check_io(T, x, y);
  if (rc) return rc;
  *layout = tq::ws_layout(T, topk, E, out, in, flags, mxfp4);
  if ((layout->gemm || !mxfp4) && E > 4096)
    return fail(TQ_EINVAL, "this path supports E <= 4096 (E = %d)", E);
  if (!layout->gemm && tq::gemv_chunk_bound(T * topk, E, layout->groups, mxfp4) > tq::GEMV_MAX_G)
    return fail(TQ_EINVAL,
                "decode batches take at most %d (group, chunk) pairs: (E + T*topk/%d) * out/128",
                tq::GEMV_MAX_G, tq::gemv_rows(mxfp4));
  if ((layout->gemm || !mxfp4) && T * (int64_t)in * (layout->gemm ? 2 : 4) >= ((int64_t)1 << 31))
    return fail(TQ_EINVAL, "the prepared activations (T * in * %d bytes) must stay below 2^31",
                layout->gemm ? 2 : 4);
  if (mxfp4 && mx_unit >= ((int64_t)1 << 31))
    return fail(TQ_EINVAL, "a unit of out * in weights must stay below 2^31 bytes");
  if (!layout->gemm && !mxfp4 && (int64_t)out * in / 2 >= ((int64_t)1 << 31))
    return fail(TQ_EINVAL, "out * in is too large for the decode-batch path");
  if (T == 0) return TQ_OK;
  return check_ws(ws, ws_bytes, layout->total);
}

// The output-side rotation of a layer that has one (FORMAT F17), on `rows` rows of y.
static int rotate_outputs(const tq_trellis_layer* L, float* y, int64_t rows, hipStream_t s) {
  if (!L->out_signs) return ok();
  hipError_t err = tq::launch_rotate_out(y, rows, L->out, L->out_signs, s);
  if (err != hipSuccess) return hip_fail(err, "output rotation launch");
  return ok();
}

static int run_route(const tq::WsLayout& L, void* ws, const int32_t* ids, int64_t N, int E, int out,
              float* y_slots, hipStream_t s) {
  tq::RouteArgs r{};
  r.ids = ids;
  r.N = N;
  r.E = E;
  r.out = out;
  r.counts = at<int32_t>(ws, L.counts);
  r.offsets = at<int32_t>(ws, L.offsets);
  r.hist = at<int32_t>(ws, L.hist);
  r.rank = at<int32_t>(ws, L.rank);
  r.pairs = at<int32_t>(ws, L.pairs);
  r.items = at<int32_t>(ws, L.items);
  r.n_items = at<int32_t>(ws, L.n_items);
  r.y_special = y_slots;
  r.status = at<uint32_t>(ws, L.status);
  r.blocks = L.route_blocks;
  r.item_rows = tq::GEMM_MT;
  r.max_items = L.max_items;
  r.split_rows = L.split_rows;
  hipError_t err = tq::launch_route(r, s);
  if (err != hipSuccess) return hip_fail(err, "route launch");
  return TQ_OK;
}


}  // namespace

int trellis_expert_gemm(const tq_trellis_layer* L, const void* x, int64_t T,
                        const int32_t* topk_ids, const float* topk_w, int32_t topk, float* y,
                        uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_trellis_layer(L);
  if (rc) return rc;
  if ((flags & TQ_FP8) && (flags & 3u) == TQ_GEMV)
    return fail(TQ_EINVAL, "TQ_FP8 runs in the prefill mode only (not with TQ_GEMV)");
  if ((flags & TQ_FP8) && T * (int64_t)L->in >= ((int64_t)1 << 31))
    return fail(TQ_EINVAL, "the MXFP8 activations (T * in bytes) must stay below 2^31");
  if (L->codebook != TQ_CODEBOOK_T16 && !(flags & TQ_FP8))
    return fail(TQ_EINVAL, "mul1 and pmcgx layers run on the FP8 matrix cores only (TQ_FP8)");
  if ((flags & TQ_ROTATE) && L->signs && !aligned(L->signs, 16))
    return fail(TQ_EALIGN, "signs must be 16-byte aligned");
  tq::WsLayout W;
  rc = common_checks(L->E, L->out, L->in, x, T, topk_ids, topk, y, flags, ws, ws_bytes, 0, &W);
  if (rc) return rc;
  if (T == 0) return ok();
  rc = check_device();
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t N = T * topk;
  float* y_slots = (flags & TQ_COMBINE) ? at<float>(ws, W.slots) : y;
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  hipError_t err;
  if (!W.gemm) {
    const int G = tq::trellis_gemv_grid();
    if (G <= 0) return fail(TQ_EHIP, "could not size the GEMV grid");
    // launched waves: the plan's target, or one per expert group when that is more
    const int Gl = (int)std::max<int64_t>(G, tq::gemv_chunk_bound(N, L->E, W.groups, false));
    tq::PlanArgs p{};
    p.ids = topk_ids;
    p.N = (int)N;
    p.E = L->E;
    p.topk = topk;
    p.bits = L->bits;
    p.code_off = L->code_off;
    p.codes_bytes = L->codes_bytes;
    p.unit_bytes = (int64_t)L->out * L->in / 8;
    p.groups = W.groups;
    p.S = L->in / 64;
    p.R = tq::gemv_rows(false);
    p.G = G;
    p.Gl = Gl;
    p.info = at<int32_t>(ws, W.info);
    p.rec = at<tq::PlanRec>(ws, W.rec);
    p.desc = at<int4>(ws, W.desc);
    p.list = at<int32_t>(ws, W.list);
    p.slot_info = at<int4>(ws, W.slot_info);
    p.rank = at<int32_t>(ws, W.prank);
    p.status = at<uint32_t>(ws, W.status);
    p.x = xb;
    p.rotate = (flags & TQ_ROTATE) != 0;
    p.signs = L->signs;
    p.T = (int)T;
    p.in = L->in;
    p.xq = at<uint32_t>(ws, W.xq);
    p.xscale = at<float>(ws, W.xscale);
    p.xsum = at<int32_t>(ws, W.xsum);
    err = tq::launch_gemv_plan(p, s);
    if (err != hipSuccess) return hip_fail(err, "decode plan launch");
    tq::TrellisGemvArgs a{};
    a.layout = L->layout;
    a.codes = L->codes;
    a.xq = p.xq;
    a.rec = p.rec;
    a.desc = p.desc;
    a.list = p.list;
    a.partial = at<int64_t>(ws, W.partial);
    a.x_bytes = (uint32_t)(T * L->in * 4);
    a.N = (int)N;
    a.out = L->out;
    a.in = L->in;
    a.topk = topk;
    a.G = Gl;
    err = time_begin(s);
    if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
    err = tq::launch_trellis_gemv(a, s);
    if (err == hipSuccess) err = time_end(s);
    if (err != hipSuccess) return hip_fail(err, "trellis GEMV launch");
    tq::PieceReduceArgs r{};
    r.slot_info = p.slot_info;
    r.partial = a.partial;
    r.exact = 1;
    r.scales = L->scales;
    r.gates = topk_w;
    r.xsum = p.xsum;
    r.xscale = p.xscale;
    r.y = y;
    r.N = (int)N;
    r.out = L->out;
    r.topk = topk;
    r.combine = (flags & TQ_COMBINE) ? 1 : 0;
    r.xdiv = topk;
    r.qmax = L->in / 256;
    r.pre = tq::reduce_prefetch(N, L->E, W.groups, G, r.qmax);
    err = tq::launch_piece_reduce(r, s);
    if (err != hipSuccess) return hip_fail(err, "GEMV piece reduction launch");
    return rotate_outputs(L, y, (flags & TQ_COMBINE) ? T : N, s);
  } else if (flags & TQ_FP8) {
    err = tq::launch_tf8_prep(xb, T, L->in, (flags & TQ_ROTATE) != 0, L->signs,
                              at<uint8_t>(ws, W.xa), at<uint8_t>(ws, W.xs), s);
    if (err != hipSuccess) return hip_fail(err, "MXFP8 activation prep launch");
    rc = run_route(W, ws, topk_ids, N, L->E, L->out, y_slots, s);
    if (rc) return rc;
    tq::TrellisFp8GemmArgs a{};
    a.codebook = L->codebook;
    a.layout = L->layout;
    a.bits = L->bits;
    a.code_off = L->code_off;
    a.codes = L->codes;
    a.codes_bytes = L->codes_bytes;
    a.scales = L->scales;
    a.xa = at<uint8_t>(ws, W.xa);
    a.xa_bytes = (uint32_t)(T * L->in);
    a.xs = at<uint8_t>(ws, W.xs);
    a.xs_bytes = (uint32_t)(T * L->in / 32);
    a.gates = topk_w;
    a.pairs = at<int32_t>(ws, W.pairs);
    a.items = at<int32_t>(ws, W.items);
    a.n_items = at<int32_t>(ws, W.n_items);
    a.y = y_slots;
    a.status = at<uint32_t>(ws, W.status);
    a.E = L->E;
    a.out = L->out;
    a.in = L->in;
    a.topk = topk;
    a.groups = W.groups;
    a.max_items = W.max_items;
    err = time_begin(s);
    if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
    err = tq::launch_tf8_gemm(a, s);
    if (err == hipSuccess) err = time_end(s);
    if (err != hipSuccess) return hip_fail(err, "FP8 trellis GEMM launch");
  } else {
    err = tq::launch_activation_prep(xb, T, L->in, at<uint32_t>(ws, W.xprep),
                                     at<float2>(ws, W.rowsum), (flags & TQ_ROTATE) != 0,
                                     L->signs, s);
    if (err != hipSuccess) return hip_fail(err, "activation prep launch");
    rc = run_route(W, ws, topk_ids, N, L->E, L->out, y_slots, s);
    if (rc) return rc;
    tq::TrellisGemmArgs a{};
    a.layout = L->layout;
    a.bits = L->bits;
    a.code_off = L->code_off;
    a.codes = L->codes;
    a.codes_bytes = L->codes_bytes;
    a.scales = L->scales;
    a.xp = at<uint32_t>(ws, W.xprep);
    a.rowsum = at<float2>(ws, W.rowsum);
    a.x_bytes = (uint32_t)(T * L->in * 2);
    a.gates = topk_w;
    a.pairs = at<int32_t>(ws, W.pairs);
    a.items = at<int32_t>(ws, W.items);
    a.n_items = at<int32_t>(ws, W.n_items);
    a.y = y_slots;
    a.status = at<uint32_t>(ws, W.status);
    a.E = L->E;
    a.out = L->out;
    a.in = L->in;
    a.topk = topk;
    a.groups = W.groups;
    a.max_items = W.max_items;
    err = time_begin(s);
    if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
    err = tq::launch_trellis_gemm(a, s);
    if (err == hipSuccess) err = time_end(s);
    if (err != hipSuccess) return hip_fail(err, "trellis GEMM launch");
  }
  if (flags & TQ_COMBINE) {
    err = tq::launch_combine(y_slots, y, T, topk, L->out, s);
    if (err != hipSuccess) return hip_fail(err, "combine launch");
  }
  return rotate_outputs(L, y, (flags & TQ_COMBINE) ? T : N, s);
}

}  // extern "C"

namespace {

// The expert GEMM of the E8M0-scaled stores (MXFP4, fp8b32): E units of `unit` bytes back
// to back at `units`.
struct MxLayer {
  int fmt, E, out, in, layout;
  const uint8_t* units;
};

int mx_expert_gemm(const MxLayer* L, const void* x, int64_t T, const int32_t* topk_ids,
                   const float* topk_w, int32_t topk, float* y, uint32_t flags, void* ws,
                   size_t ws_bytes, void* stream) {
  if (flags & TQ_ROTATE) return fail(TQ_EINVAL, "TQ_ROTATE applies to trellis layers only");
  if ((flags & TQ_FP8) && L->fmt != tq::MX_FP4)
    return fail(TQ_EINVAL, "TQ_FP8 applies to trellis and MXFP4 layers only");
  if ((flags & TQ_FP8) && (flags & 3u) == TQ_GEMV)
    return fail(TQ_EINVAL, "TQ_FP8 runs in the prefill mode only (not with TQ_GEMV)");
  if ((flags & TQ_FP8) && T * (int64_t)L->in >= ((int64_t)1 << 31))
    return fail(TQ_EINVAL, "the MXFP8 activations (T * in bytes) must stay below 2^31");
  const int64_t unit = mx_unit_bytes(L->fmt, L->out, L->in);
  tq::WsLayout W;
  int rc = common_checks(L->E, L->out, L->in, x, T, topk_ids, topk, y, flags, ws, ws_bytes, unit, &W);
  if (rc) return rc;
  if (T == 0) return ok();
  rc = check_device();
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t N = T * topk;
  float* y_slots = (flags & TQ_COMBINE) ? at<float>(ws, W.slots) : y;
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  hipError_t err;
  if (!W.gemm) {
    const int G = tq::mxfp4_gemv_grid(L->fmt);
    if (G <= 0) return fail(TQ_EHIP, "could not size the GEMV grid");
    const int Gl = (int)std::max<int64_t>(G, tq::gemv_chunk_bound(N, L->E, W.groups, true));
    tq::PlanArgs p{};
    p.ids = topk_ids;
    p.N = (int)N;
    p.E = L->E;
    p.topk = topk;
    p.bits = nullptr;  // every step costs 1
    p.unit_bytes = unit;
    p.groups = W.groups;
    p.S = L->in / 128;
    p.R = tq::gemv_rows(true);
    p.G = G;
    p.Gl = Gl;
    p.info = at<int32_t>(ws, W.info);
    p.rec = at<tq::PlanRec>(ws, W.rec);
    p.desc = at<int4>(ws, W.desc);
    p.list = at<int32_t>(ws, W.list);
    p.slot_info = at<int4>(ws, W.slot_info);
    p.rank = at<int32_t>(ws, W.prank);
    p.status = at<uint32_t>(ws, W.status);
    p.x = nullptr;  // no activation prep: the GEMV reads bf16 x
    err = tq::launch_gemv_plan(p, s);
    if (err != hipSuccess) return hip_fail(err, "decode plan launch");
    tq::Mxfp4GemvArgs a{};
    a.fmt = L->fmt;
    a.layout = L->layout;
    a.units = L->units;
    a.x = xb;
    a.x_bytes = (uint32_t)(T * L->in * 2);
    a.rec = p.rec;
    a.desc = p.desc;
    a.list = p.list;
    a.partial = at<float>(ws, W.partial);
    a.N = (int)N;
    a.out = L->out;
    a.in = L->in;
    a.topk = topk;
    a.G = Gl;
    err = time_begin(s);
    if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
    err = tq::launch_mxfp4_gemv(a, s);
    if (err == hipSuccess) err = time_end(s);
    if (err != hipSuccess) return hip_fail(err, "GEMV launch");
    tq::PieceReduceArgs r{};
    r.slot_info = p.slot_info;
    r.partial = a.partial;
    r.exact = 0;
    r.scales = nullptr;
    r.gates = topk_w;
    r.xsum = nullptr;
    r.xscale = nullptr;
    r.y = y;
    r.N = (int)N;
    r.out = L->out;
    r.topk = topk;
    r.combine = (flags & TQ_COMBINE) ? 1 : 0;
    r.xdiv = topk;
    r.qmax = L->in / 512;
    r.pre = tq::reduce_prefetch(N, L->E, W.groups, G, r.qmax);
    err = tq::launch_piece_reduce(r, s);
    if (err != hipSuccess) return hip_fail(err, "GEMV piece reduction launch");
    return ok();
  } else if (flags & TQ_FP8) {
    err = tq::launch_mxfp8_prep(xb, T, L->in, at<uint8_t>(ws, W.xa), at<uint8_t>(ws, W.xs), s);
    if (err != hipSuccess) return hip_fail(err, "MXFP8 activation launch");
    rc = run_route(W, ws, topk_ids, N, L->E, L->out, y_slots, s);
    if (rc) return rc;
    tq::Mx8GemmArgs a{};
    a.layout = L->layout;
    a.units = L->units;
    a.xa = at<uint8_t>(ws, W.xa);
    a.xa_bytes = (uint32_t)(T * L->in);
    a.xs = at<uint8_t>(ws, W.xs);
    a.xs_bytes = (uint32_t)(T * L->in / 32);
    a.gates = topk_w;
    a.pairs = at<int32_t>(ws, W.pairs);
    a.items = at<int32_t>(ws, W.items);
    a.n_items = at<int32_t>(ws, W.n_items);
    a.y = y_slots;
    a.E = L->E;
    a.out = L->out;
    a.in = L->in;
    a.topk = topk;
    a.groups = W.groups;
    a.max_items = W.max_items;
    err = time_begin(s);
    if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
    err = tq::launch_mx8_gemm(a, s);
    if (err == hipSuccess) err = time_end(s);
    if (err != hipSuccess) return hip_fail(err, "FP8 GEMM launch");
  } else {
    rc = run_route(W, ws, topk_ids, N, L->E, L->out, y_slots, s);
    if (rc) return rc;
    tq::Mxfp4GemmArgs a{};
    a.fmt = L->fmt;
    a.layout = L->layout;
    a.units = L->units;
    a.x = xb;
    a.x_bytes = (uint32_t)(T * L->in * 2);
    a.gates = topk_w;
    a.pairs = at<int32_t>(ws, W.pairs);
    a.items = at<int32_t>(ws, W.items);
    a.n_items = at<int32_t>(ws, W.n_items);
    a.y = y_slots;
    a.E = L->E;
    a.out = L->out;
    a.in = L->in;
    a.topk = topk;
    a.groups = W.groups;
    a.max_items = W.max_items;
    err = time_begin(s);
    if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
    err = tq::launch_mxfp4_gemm(a, s);
    if (err == hipSuccess) err = time_end(s);
    if (err != hipSuccess) return hip_fail(err, "GEMM launch");
  }
  if (flags & TQ_COMBINE) {
    err = tq::launch_combine(y_slots, y, T, topk, L->out, s);
    if (err != hipSuccess) return hip_fail(err, "combine launch");
  }
  return ok();
}

}  // namespace

extern "C" {

int mxfp4_expert_gemm(const tq_mxfp4_layer* L, const void* x, int64_t T,
                      const int32_t* topk_ids, const float* topk_w, int32_t topk, float* y,
                      uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_mxfp4_layer(L);
  if (rc) return rc;
  const MxLayer m{tq::MX_FP4, L->E, L->out, L->in, L->layout, L->units};
  return mx_expert_gemm(&m, x, T, topk_ids, topk_w, topk, y, flags, ws, ws_bytes, stream);
}

static int mx_repack(int fmt, int E, int out, int in, int layout, const uint8_t* units,
                     uint8_t* dst, void* stream) {
  if (layout != TQ_LAYOUT_STORE)
    return fail(TQ_EINVAL, "the layer to repack must be in TQ_LAYOUT_STORE (layout = %d)", layout);
  if (!dst) return fail(TQ_EINVAL, "dst is NULL");
  if (!aligned(dst, 16)) return fail(TQ_EALIGN, "dst must be 16-byte aligned");
  const int64_t total = mx_unit_bytes(fmt, out, in) * E;
  const char* a = reinterpret_cast<const char*>(units);
  const char* b = reinterpret_cast<const char*>(dst);
  if (a < b + total && b < a + total) return fail(TQ_EINVAL, "dst overlaps the layer's units");
  if (mx_unit_bytes(fmt, out, in) >= ((int64_t)1 << 31))
    return fail(TQ_EINVAL, "a unit of out * in weights must stay below 2^31 bytes");
  int rc = check_device();
  if (rc) return rc;
  hipError_t err = tq::launch_mx_repack(fmt, units, dst, E, out, in, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "repack launch");
  return ok();
}

int trellis_repack(const tq_trellis_layer* L, uint32_t* dst, void* stream) {
  int rc = check_trellis_layer(L);
  if (rc) return rc;
  if (L->layout != TQ_LAYOUT_STORE && L->layout != TQ_LAYOUT_UNIT128)
    return fail(TQ_EINVAL, "the layer to repack must be in TQ_LAYOUT_STORE or TQ_LAYOUT_UNIT128 "
                "(layout = %d)", L->layout);
  if (!dst) return fail(TQ_EINVAL, "dst is NULL");
  if (!aligned(dst, 16)) return fail(TQ_EALIGN, "dst must be 16-byte aligned");
  const char* a = reinterpret_cast<const char*>(L->codes);
  const char* b = reinterpret_cast<const char*>(dst);
  if (a < b + L->codes_bytes && b < a + L->codes_bytes)
    return fail(TQ_EINVAL, "dst overlaps the layer's codes");
  if ((int64_t)L->out * L->in / 2 >= ((int64_t)1 << 31))
    return fail(TQ_EINVAL, "out * in is too large");
  rc = check_device();
  if (rc) return rc;
  hipError_t err = tq::launch_trellis_repack(L->bits, L->code_off, L->codes, L->codes_bytes, L->E,
                                             L->out, L->in, L->layout, dst,
                                             static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "trellis_repack launch");
  return ok();
}

int mxfp4_repack(const tq_mxfp4_layer* L, uint8_t* dst, void* stream) {
  int rc = check_mxfp4_layer(L);
  if (rc) return rc;
  return mx_repack(tq::MX_FP4, L->E, L->out, L->in, L->layout, L->units, dst, stream);
}

int fp8b32_repack(const tq_fp8b32_layer* L, uint8_t* dst, void* stream) {
  int rc = check_fp8b32_layer(L);
  if (rc) return rc;
  return mx_repack(tq::MX_FP8B32, L->E, L->out, L->in, L->layout, L->units, dst, stream);
}

int fp8b32_expert_gemm(const tq_fp8b32_layer* L, const void* x, int64_t T,
                       const int32_t* topk_ids, const float* topk_w, int32_t topk, float* y,
                       uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_fp8b32_layer(L);
  if (rc) return rc;
  const MxLayer m{tq::MX_FP8B32, L->E, L->out, L->in, L->layout, L->units};
  return mx_expert_gemm(&m, x, T, topk_ids, topk_w, topk, y, flags, ws, ws_bytes, stream);
}

}  // extern "C"

// ---- the routed expert FFN -------------------------------------------------------------

namespace {

// The FFN workspace: the gate/up call's region (its status word first), the down
// projection's region, then (prefill) the gate/up fp32 rows and the down slots' rows.
struct FfnWs {
  tq::WsLayout gu, dn;
  size_t gu_off, dn_off, rows_off, slots_off, total;
  bool gemm;
};

FfnWs ffn_ws(int64_t T, int32_t topk, int32_t E, int32_t H, int32_t I, uint32_t flags) {
  FfnWs w{};
  const int64_t N = T * topk;
  w.gemm = use_gemm(T, topk, E, (2 * I + 127) / 128, flags);
  // the decode batch needs both projections' (group, chunk) pairs within the GEMV's bound
  if ((flags & 3u) == TQ_AUTO &&
      (tq::gemv_chunk_bound(N, E, (2 * I + 127) / 128, false) > tq::GEMV_MAX_G ||
       tq::gemv_chunk_bound(N, E, (H + 127) / 128, false) > tq::GEMV_MAX_G))
    w.gemm = true;
  const uint32_t mode = w.gemm ? TQ_GEMM : TQ_GEMV;
  w.gu = tq::ws_layout(T, topk, E, 2 * I, H, mode, false);
  w.dn = tq::ws_layout(N, 1, E, H, I, mode, false);
  w.gu_off = 0;
  w.dn_off = round_up(w.gu.total, 256);
  size_t off = w.dn_off + round_up(w.dn.total, 256);
  if (w.gemm) {
    w.rows_off = off;
    off += round_up((size_t)N * 2 * I * 4, 256);
    w.slots_off = off;
    off += round_up((size_t)N * H * 4, 256);
  }
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

size_t tq_ffn_workspace_bytes(int64_t T, int32_t topk, int32_t E, int32_t H, int32_t I,
                              uint32_t flags) {
  if (T < 0 || topk < 1 || E < 1 || H < 256 || I < 256 || H % 256 || I % 256) return 0;
  return ffn_ws(T, topk, E, H, I, flags).total;
}

int trellis_expert_ffn(const tq_trellis_layer* gate_up, const tq_trellis_layer* down,
                       const void* x, int64_t T, const int32_t* topk_ids, const float* topk_w,
                       int32_t topk, float* y, uint32_t flags, void* ws, size_t ws_bytes,
                       void* stream) {
  int rc = check_trellis_layer(gate_up);
  if (rc) return rc;
  rc = check_trellis_layer(down);
  if (rc) return rc;
  if ((flags & ~(3u | TQ_ROTATE)) != 0 || (flags & 3u) == 3u)
    return fail(TQ_EINVAL, "flags = 0x%x is not valid for the FFN", flags);
  if (gate_up->codebook != TQ_CODEBOOK_T16 || down->codebook != TQ_CODEBOOK_T16)
    return fail(TQ_EINVAL, "the FFN runs T16 layers only");
  const int E = gate_up->E, H = gate_up->in, I = gate_up->out / 2;
  if (gate_up->out % 2) return fail(TQ_EINVAL, "gate_up must have an even number of outputs");
  if (down->E != E) return fail(TQ_EINVAL, "the two layers must have the same E");
  if (down->out != H || down->in != I)
    return fail(TQ_EINVAL, "down must be in = gate_up.out / 2 (%d), out = gate_up.in (%d)", I, H);
  if (H % 256 || I % 256) return fail(TQ_EINVAL, "H and I must be multiples of 256");
  if (I > 4096) return fail(TQ_EINVAL, "I = %d is above 4096", I);
  if ((flags & TQ_ROTATE) && gate_up->signs && !aligned(gate_up->signs, 16))
    return fail(TQ_EALIGN, "signs must be 16-byte aligned");
  if (down->signs && !aligned(down->signs, 4)) return fail(TQ_EALIGN, "down signs must be 4-byte aligned");
  rc = check_routes(T, topk, topk_ids);
  if (rc) return rc;
  rc = check_io(T, x, y);
  if (rc) return rc;
  const int64_t N = T * topk;
  const FfnWs W = ffn_ws(T, topk, E, H, I, flags);
  const uint32_t mode = W.gemm ? TQ_GEMM : TQ_GEMV;
  // the gate/up and down calls' own limits
  tq::WsLayout tmp;
  rc = common_checks(E, 2 * I, H, x, T, topk_ids, topk, y, mode, nullptr, 0, 0, &tmp);
  if (rc && rc != TQ_EWORKSPACE) return rc;
  rc = common_checks(E, H, I, x, N, topk_ids, 1, y, mode, nullptr, 0, 0, &tmp);
  if (rc && rc != TQ_EWORKSPACE) return rc;
  if (T == 0) return ok();
  rc = check_ws(ws, ws_bytes, W.total);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  void* wg = base + W.gu_off;
  void* wd = base + W.dn_off;
  uint32_t* status = at<uint32_t>(wg, W.gu.status);
  hipError_t err;
  if (!W.gemm) {
    // 1. both plans and the gate/up activation prep
    const int Gg = tq::trellis_gemv_grid(), Gd = Gg;
    if (Gg <= 0) return fail(TQ_EHIP, "could not size the GEMV grid");
    const int Glg = (int)std::max<int64_t>(Gg, tq::gemv_chunk_bound(N, E, W.gu.groups, false));
    const int Gld = (int)std::max<int64_t>(Gd, tq::gemv_chunk_bound(N, E, W.dn.groups, false));
    tq::PlanArgs pg{}, pd{};
    pg.ids = topk_ids;
    pg.N = (int)N;
    pg.E = E;
    pg.topk = topk;
    pg.bits = gate_up->bits;
    pg.code_off = gate_up->code_off;
    pg.codes_bytes = gate_up->codes_bytes;
    pg.unit_bytes = (int64_t)2 * I * H / 8;
    pg.groups = W.gu.groups;
    pg.S = H / 64;
    pg.R = tq::gemv_rows(false);
    pg.G = Gg;
    pg.Gl = Glg;
    pg.info = at<int32_t>(wg, W.gu.info);
    pg.rec = at<tq::PlanRec>(wg, W.gu.rec);
    pg.desc = at<int4>(wg, W.gu.desc);
    pg.list = at<int32_t>(wg, W.gu.list);
    pg.slot_info = at<int4>(wg, W.gu.slot_info);
    pg.rank = at<int32_t>(wg, W.gu.prank);
    pg.status = status;
    pg.x = static_cast<const uint16_t*>(x);
    pg.rotate = (flags & TQ_ROTATE) != 0;
    pg.signs = gate_up->signs;
    pg.T = (int)T;
    pg.in = H;
    pg.xq = at<uint32_t>(wg, W.gu.xq);
    pg.xscale = at<float>(wg, W.gu.xscale);
    pg.xsum = at<int32_t>(wg, W.gu.xsum);
    pd = pg;
    pd.N = (int)N;
    pd.topk = 1;
    pd.bits = down->bits;
    pd.code_off = down->code_off;
    pd.codes_bytes = down->codes_bytes;
    pd.unit_bytes = (int64_t)H * I / 8;
    pd.groups = W.dn.groups;
    pd.S = I / 64;
    pd.G = Gd;
    pd.Gl = Gld;
    pd.info = at<int32_t>(wd, W.dn.info);
    pd.rec = at<tq::PlanRec>(wd, W.dn.rec);
    pd.desc = at<int4>(wd, W.dn.desc);
    pd.list = at<int32_t>(wd, W.dn.list);
    pd.slot_info = at<int4>(wd, W.dn.slot_info);
    pd.rank = at<int32_t>(wd, W.dn.prank);
    pd.x = nullptr;
    err = tq::launch_ffn_plan(pg, pd, s);
    if (err != hipSuccess) return hip_fail(err, "FFN plan launch");
    // 2. the gate/up GEMV
    tq::TrellisGemvArgs a{};
    a.layout = gate_up->layout;
    a.codes = gate_up->codes;
    a.xq = pg.xq;
    a.rec = pg.rec;
    a.desc = pg.desc;
    a.list = pg.list;
    a.partial = at<int64_t>(wg, W.gu.partial);
    a.x_bytes = (uint32_t)(T * H * 4);
    a.N = (int)N;
    a.out = 2 * I;
    a.in = H;
    a.topk = topk;
    a.G = Glg;
    err = tq::launch_trellis_gemv(a, s);
    if (err != hipSuccess) return hip_fail(err, "gate/up GEMV launch");
    // 3. SwiGLU, the intermediate's rotation, the down projection's operands
    tq::FfnMidArgs m{};
    m.gu.slot_info = pg.slot_info;
    m.gu.partial = a.partial;
    m.gu.exact = 1;
    m.gu.scales = gate_up->scales;
    m.gu.gates = nullptr;
    m.gu.xsum = pg.xsum;
    m.gu.xscale = pg.xscale;
    m.gu.N = (int)N;
    m.gu.out = 2 * I;
    m.gu.topk = topk;
    m.gu.xdiv = topk;
    m.gu.qmax = H / 256;
    m.gu.pre = tq::reduce_prefetch(N, E, W.gu.groups, Gg, m.gu.qmax);
    m.gu_out_signs = gate_up->out_signs;
    m.down_signs = down->signs;
    m.N = (int)N;
    m.I = I;
    m.xq = at<uint32_t>(wd, W.dn.xq);
    m.xscale = at<float>(wd, W.dn.xscale);
    m.xsum = at<int32_t>(wd, W.dn.xsum);
    err = tq::launch_ffn_mid(m, true, s);
    if (err != hipSuccess) return hip_fail(err, "FFN middle step launch");
    // 4. the down GEMV, every slot a row of its own
    tq::TrellisGemvArgs b = a;
    b.layout = down->layout;
    b.codes = down->codes;
    b.xq = m.xq;
    b.rec = pd.rec;
    b.desc = pd.desc;
    b.list = pd.list;
    b.partial = at<int64_t>(wd, W.dn.partial);
    b.x_bytes = (uint32_t)(N * I * 4);
    b.out = H;
    b.in = I;
    b.topk = 1;
    b.G = Gld;
    err = time_begin(s);
    if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
    err = tq::launch_trellis_gemv(b, s);
    if (err == hipSuccess) err = time_end(s);
    if (err != hipSuccess) return hip_fail(err, "down GEMV launch");
    // 5. the down reduction with the gates and the combine over k
    tq::PieceReduceArgs r{};
    r.slot_info = pd.slot_info;
    r.partial = b.partial;
    r.exact = 1;
    r.scales = down->scales;
    r.gates = topk_w;
    r.xsum = m.xsum;
    r.xscale = m.xscale;
    r.y = y;
    r.N = (int)N;
    r.out = H;
    r.topk = topk;
    r.combine = 1;
    r.xdiv = 1;
    r.qmax = I / 256;
    r.pre = tq::reduce_prefetch(N, E, W.dn.groups, Gd, r.qmax);
    err = tq::launch_piece_reduce(r, s);
    if (err != hipSuccess) return hip_fail(err, "down reduction launch");
    return rotate_outputs(down, y, T, s);
  }
  // prefill: the gate/up GEMM (its output-side rotation included), the middle step, route
  // bucketing of the slots as rows, the down GEMM, the combine
  float* gu_rows = reinterpret_cast<float*>(base + W.rows_off);
  float* y_slots = reinterpret_cast<float*>(base + W.slots_off);
  rc = trellis_expert_gemm(gate_up, x, T, topk_ids, nullptr, topk, gu_rows,
                           TQ_GEMM | (flags & TQ_ROTATE), wg, W.gu.total, stream);
  if (rc) return rc;
  tq::FfnMidArgs m{};
  m.gu_rows = gu_rows;
  m.gu_out_signs = nullptr;  // applied by the gate/up call
  m.down_signs = down->signs;
  m.N = (int)N;
  m.I = I;
  m.xp = at<uint32_t>(wd, W.dn.xprep);
  m.rowsum = at<float2>(wd, W.dn.rowsum);
  err = tq::launch_ffn_mid(m, false, s);
  if (err != hipSuccess) return hip_fail(err, "FFN middle step launch");
  rc = run_route(W.dn, wd, topk_ids, N, E, H, y_slots, s);
  if (rc) return rc;
  tq::TrellisGemmArgs a{};
  a.layout = down->layout;
  a.bits = down->bits;
  a.code_off = down->code_off;
  a.codes = down->codes;
  a.codes_bytes = down->codes_bytes;
  a.scales = down->scales;
  a.xp = m.xp;
  a.rowsum = m.rowsum;
  a.x_bytes = (uint32_t)(N * I * 2);
  a.gates = topk_w;
  a.pairs = at<int32_t>(wd, W.dn.pairs);
  a.items = at<int32_t>(wd, W.dn.items);
  a.n_items = at<int32_t>(wd, W.dn.n_items);
  a.y = y_slots;
  a.status = status;
  a.E = E;
  a.out = H;
  a.in = I;
  a.topk = 1;
  a.groups = W.dn.groups;
  a.max_items = W.dn.max_items;
  err = time_begin(s);
  if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
  err = tq::launch_trellis_gemm(a, s);
  if (err == hipSuccess) err = time_end(s);
  if (err != hipSuccess) return hip_fail(err, "down GEMM launch");
  err = tq::launch_combine(y_slots, y, T, topk, H, s);
  if (err != hipSuccess) return hip_fail(err, "combine launch");
  return rotate_outputs(down, y, T, s);
}

}  // extern "C"

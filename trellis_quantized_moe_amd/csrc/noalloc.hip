// trellis_expert_gemm_noalloc: trellis_expert_gemm with its workspace in a static device
// array instead of a caller-provided buffer, for callers that cannot allocate device memory.
//
// `scratch` is one file-scope device array per GPU, held until the process ends. Host code
// never passes its name to a kernel or a copy: the name is a host-side stand-in, not a
// device address. Each device's address is looked up once with hipGetSymbolAddress, with
// that device current, and that pointer is what the kernels receive (as the workspace of
// trellis_expert_gemm, whose kernels all take it as an argument).
#include <hip/hip_runtime.h>

#include <mutex>

#include "tq.h"
#include "tq_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[TQ_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES];       // device address of `scratch` on each device
bool g_cleared[MAX_DEVICES];    // its status word has been zeroed (once, on first use)

// The device address of this device's scratch (looked up once per device), and on the first
// use a fill kernel on `s` that zeroes its status word (the workspace contract: zero before
// first use; every call leaves the rest as it needs it).
int scratch_for_current_device(hipStream_t s, void** out, char* msg, size_t msg_len) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) {
    snprintf(msg, msg_len, "hipGetDevice: %s", hipGetErrorString(err));
    return TQ_EHIP;
  }
  if (dev < 0 || dev >= MAX_DEVICES) {
    snprintf(msg, msg_len, "device %d is beyond the %d devices this entry point serves", dev,
             MAX_DEVICES);
    return TQ_EINVAL;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p) {
      snprintf(msg, msg_len, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(err));
      return TQ_EHIP;
    }
    g_ptr[dev] = p;
  }
  if (!g_cleared[dev]) {
    err = tq::launch_fill_i32(static_cast<int32_t*>(g_ptr[dev]), 64, 0, s);
    if (err != hipSuccess) {
      snprintf(msg, msg_len, "scratch clear: %s", hipGetErrorString(err));
      return TQ_EHIP;
    }
    g_cleared[dev] = true;
  }
  *out = g_ptr[dev];
  return TQ_OK;
}

}  // namespace

extern "C" int trellis_expert_gemm_noalloc(const tq_trellis_layer* L, const void* x, int64_t T,
                                           const int32_t* topk_ids, const float* topk_w,
                                           int32_t topk, float* y, uint32_t flags,
                                           void* stream) {
  if (!L) return tq::set_error(TQ_EINVAL, "layer is NULL");
  if (T == 0) return trellis_expert_gemm(L, x, T, topk_ids, topk_w, topk, y, flags, nullptr, 0,
                                         stream);
  const size_t need = tq_workspace_bytes(T, topk, L->E, L->out, L->in, flags);
  char msg[256];
  if (need == 0) {
    snprintf(msg, sizeof(msg), "invalid sizes (T = %lld, topk = %d, E = %d, out = %d, in = %d)",
             (long long)T, topk, L->E, L->out, L->in);
    return tq::set_error(TQ_EINVAL, msg);
  }
  if (need > TQ_NOALLOC_SCRATCH_BYTES) {
    snprintf(msg, sizeof(msg),
             "this call needs %zu bytes of scratch; the static scratch holds %zu (use "
             "trellis_expert_gemm with a workspace)",
             need, (size_t)TQ_NOALLOC_SCRATCH_BYTES);
    return tq::set_error(TQ_EWORKSPACE, msg);
  }
  void* ws = nullptr;
  const int rc = scratch_for_current_device(static_cast<hipStream_t>(stream), &ws, msg, sizeof(msg));
  if (rc) return tq::set_error(rc, msg);
  return trellis_expert_gemm(L, x, T, topk_ids, topk_w, topk, y, flags, ws,
                             TQ_NOALLOC_SCRATCH_BYTES, stream);
}

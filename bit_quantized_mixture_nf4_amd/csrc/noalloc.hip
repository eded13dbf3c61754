// noalloc.hip -- e4b_moe_forward_noalloc: the forward with its workspace in a
// fixed device array of the library instead of a caller buffer, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// `scratch` is one static device array per GPU (the code object's copy on
// that device). Host code never passes the array's name to a kernel or copy:
// its device address comes from hipGetSymbolAddress, taken once per device
// with that device current and kept in g_scratch. Every call on one GPU
// shares that GPU's array; calls that overlap on one GPU (two streams, two
// threads) race on it. No kernel of the forward reads a workspace byte it
// did not write in the same call, so nothing is cleared between calls.
#include <mutex>

#include "device.h"
#include "kernels.h"

namespace e4b {

constexpr size_t kScratchBytes = E4B_NOALLOC_SCRATCH_BYTES;  // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

struct ScratchSlot {
  std::once_flag once;
  void *ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch array (null on failure).
void *scratch_ptr(hipError_t *err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  ScratchSlot &s = g_scratch[dev];
  std::call_once(s.once, [&s]() {
    s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch));
    if (s.err != hipSuccess) s.ptr = nullptr;
  });
  *err = s.err;
  return s.ptr;
}

}  // namespace
}  // namespace e4b

using namespace e4b;

extern "C" e4b_status e4b_moe_forward_noalloc(const e4b_moe_layer *L, int64_t T, int32_t top_k,
                                              const void *x_bf16, const float *router_logits,
                                              int32_t *topk_idx, float *topk_w, void *y_bf16,
                                              void *saved, int32_t path, hipStream_t stream) {
  const size_t need = e4b_moe_workspace_bytes(L, T, top_k);
  if (need == 0) {
    // invalid arguments: the regular entry point reports which
    return e4b_moe_forward(L, T, top_k, x_bf16, router_logits, topk_idx, topk_w, y_bf16, saved,
                           nullptr, 0, path, stream);
  }
  if (need > kScratchBytes) return E4B_ERR_WORKSPACE;
  hipError_t err = hipSuccess;
  void *ws = scratch_ptr(&err);
  if (!ws) return E4B_ERR_HIP;
  return e4b_moe_forward(L, T, top_k, x_bf16, router_logits, topk_idx, topk_w, y_bf16, saved, ws,
                         kScratchBytes, path, stream);
}

// attn_noalloc.hip -- attn_bwd_noalloc: attn_bwd with its delta rows in a fixed,
// library-owned device array instead of a caller workspace, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// The array `scratch` below has one copy per GPU, held until the process ends.
// On the host its name is only a stand-in, not a device address, so host code
// never passes it to a kernel or a copy: the first call on each device (with
// that device current) resolves the device address with hipGetSymbolAddress and
// keeps it per device, and every use goes through that pointer.  Calls on one
// GPU share the array, so calls that overlap in time on one GPU (two streams,
// two threads) race on it; calls queued on one stream do not.
#include <mutex>

#include "../../include/attn.h"
#include "launch.hpp"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

static_assert(ATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch is a whole number of 256-byte blocks");

// delta of attn_bwd_noalloc: B * Hq * T float32, at most ATTN_NOALLOC_SCRATCH_BYTES bytes.
// Every element a call reads is written by that call's preprocess first, so it
// needs no clearing.
__device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device, once resolved

// Device address of `scratch` on the current device.
attn_status_t scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();  // leave no error pending for the caller's next call
      return ATTN_ERR_HIP;
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return ATTN_OK;
}

}  // namespace

ATTN_EXPORT attn_status_t attn_bwd_noalloc(const void* q, const void* k, const void* v,
                                           const void* o, const float* lse, const void* dO,
                                           void* dq, void* dk, void* dv, int B, int T, int Hq,
                                           int Hkv, int D, float scale, int causal,
                                           attn_dtype_t dtype, void* stream) {
  // The argument checks of attn_bwd (all on the host, before any HIP call), then
  // the size limit of the scratch array.
  const attn_status_t st = rca::check_bwd_args(q, k, v, o, lse, dO, dq, dk, dv, B, T, Hq, Hkv, D,
                                               scale, causal, dtype, nullptr, 0);
  if (st != ATTN_OK) return st;
  const size_t need = attn_bwd_workspace_bytes(B, T, Hq, Hkv, D, dtype);
  if (need == 0 || need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_INVALID_ARG;
  void* ws = nullptr;
  const attn_status_t sst = scratch_on_current_device(&ws);
  if (sst != ATTN_OK) return sst;
  return rca::enqueue_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, T, Hq, Hkv, D, scale, causal, dtype,
                          static_cast<float*>(ws), stream);
}

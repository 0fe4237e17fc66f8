// xattn_bwd_noalloc: the attention backward with its scratch in a static device array, for
// callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The scratch is a file-scope device array of a fixed size; every GPU the library runs on
// holds its own copy until the process ends.  In host code the array's name is only a
// host-side stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (on the first call made with that device current) and kept; kernels
// receive that address, never the name.  Every call on one GPU shares that GPU's array:
// calls that overlap on one GPU (concurrent streams, several threads) race on it.  Nothing
// in it has to start at zero: the backward writes every scratch element it later reads
// (row statistics D and lse*log2(e), per-workgroup dgamma partials), so the contents left by
// the previous call are never used.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/xattn.h"
#include "xattn_internal.h"

namespace {

static_assert(XATTN_BWD_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep alignment");

static __device__ __align__(256) unsigned char scratch[XATTN_BWD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on first use).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" xattn_status xattn_bwd_noalloc(const xattn_dims* dims, const void* q, const void* k,
                                          const void* v, const void* out, const float* lse,
                                          const void* dout, void* dq, void* dk, void* dv,
                                          const xattn_prologue* pro, void* stream) {
  const size_t need = xattn_bwd_workspace_bytes(dims, pro != nullptr);
  // need == 0: invalid dims; xattn_bwd reports them (it checks dims before the workspace)
  if (need == 0) return xattn_bwd(dims, q, k, v, out, lse, dout, dq, dk, dv, pro, nullptr, 0, stream);
  if (need > (size_t)XATTN_BWD_NOALLOC_SCRATCH_BYTES) {
    char msg[200];
    std::snprintf(msg, sizeof msg,
                  "xattn_bwd_noalloc: this shape needs %zu bytes of scratch, the static "
                  "scratch holds %zu (use xattn_bwd with a workspace)",
                  need, (size_t)XATTN_BWD_NOALLOC_SCRATCH_BYTES);
    xattn::set_last_error(msg);
    return XATTN_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) {
    char msg[200];
    std::snprintf(msg, sizeof msg, "xattn_bwd_noalloc: scratch address lookup: %s",
                  hipGetErrorString(e));
    xattn::set_last_error(msg);
    return XATTN_ERR_HIP;
  }
  return xattn_bwd(dims, q, k, v, out, lse, dout, dq, dk, dv, pro, ws,
                   (size_t)XATTN_BWD_NOALLOC_SCRATCH_BYTES, stream);
}

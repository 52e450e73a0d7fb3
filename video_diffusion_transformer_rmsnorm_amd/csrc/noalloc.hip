// noalloc.hip -- vdit_attn_fwd_noalloc: vdit_attn_fwd with the library's own
// device scratch in place of a caller's workspace, for callers that cannot
// allocate device memory (code under graph capture, serving loops, harnesses
// that forbid allocation).  Declared in include/vdit.h.
//
// The scratch is a file-scope device array of kScratchBytes, one copy per
// device, held until the process ends.  In host code its name stands for a
// host-side shadow, not a device address: the device address is looked up
// once per device (hipGetSymbolAddress, with that device current, on the
// entry point's first call there) and only that address is ever handed to
// kernels.  Every call on a device shares the array: calls that overlap in
// time on one device (two streams, two threads) race on it.  None of the
// kernels needs any part of the workspace to start at zero, so the array is
// never cleared.
#include "vdit.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "validate.hpp"
#include "vdit_internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

// Device address of this device's scratch array (looked up on first use).
hipError_t scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

vdit_status err(vdit_status s, const char* msg) {
  return static_cast<vdit_status>(vdit::report_error(int(s), msg));
}

}  // namespace

extern "C" vdit_status vdit_attn_fwd_noalloc(const vdit_attn_args* args, hipStream_t stream) {
  if (!args) return err(VDIT_ERR_INVALID_ARG, "args is NULL");
  if (args->workspace || args->workspace_bytes)
    return err(VDIT_ERR_INVALID_ARG, "vdit_attn_fwd_noalloc: workspace must be NULL and workspace_bytes 0 "
                                     "(the library's scratch takes its place)");
  const size_t need = vdit_attn_workspace_bytes(args);  // validates the shape
  if (need == size_t(-1)) return VDIT_ERR_INVALID_ARG;   // message already set
  vdit_attn_args a = *args;
  const size_t required = vdit::attn_required_bytes(*reinterpret_cast<const vdit::AttnArgs*>(&a));
  if (required > kScratchBytes) {
    char msg[200];
    std::snprintf(msg, sizeof msg,
                  "vdit_attn_fwd_noalloc: this call needs %zu bytes of workspace, the scratch holds %zu "
                  "(use vdit_attn_fwd with a workspace)",
                  required, kScratchBytes);
    return err(VDIT_ERR_UNSUPPORTED, msg);
  }
  if (need > 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
    void* p = nullptr;
    if (e == hipSuccess) e = scratch_address(dev, &p);
    if (e != hipSuccess) {
      char msg[160];
      std::snprintf(msg, sizeof msg, "vdit_attn_fwd_noalloc: scratch address: %s", hipGetErrorString(e));
      return err(VDIT_ERR_HIP, msg);
    }
    // the optional parts (key-norm partials, key-split partials) are used
    // when they fit, as with a caller's workspace of this size
    a.workspace = p;
    a.workspace_bytes = need < kScratchBytes ? need : kScratchBytes;
  }
  return vdit_attn_fwd(&a, stream);
}

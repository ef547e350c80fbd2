// scratch.hip -- moe_expert_forward_static: moe_expert_forward with its workspace in a
// library-owned device array instead of caller memory, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Nothing here allocates: the array is part of the library's code object, and
// each GPU that runs the library holds its own copy until the process ends.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "launch.h"
#include "qmoe.h"

namespace {

// The workspace of every call on one GPU: the intermediate activation (or its two e4m3
// planes), the MXFP4 activation planes and the per-pair partial rows (moe_workspace_bytes).
// In host code `scratch` names a host-side stand-in, not device memory: only the address
// hipGetSymbolAddress returns for the current device may be passed to kernels or copies.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices];  // per device: the array's device address, once looked up

// The current device's address of `scratch`, looked up on the first call on that device.
int scratch_address(void **ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return qmoe::set_last_error(MOE_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return qmoe::set_last_error(MOE_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[256];
      snprintf(msg, sizeof msg, "moe_expert_forward_static: hipGetSymbolAddress of the scratch array failed: %s",
               hipGetErrorString(e));
      return qmoe::set_last_error(MOE_ERR_HIP, msg);
    }
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_expert_forward_static(const moe_bank *routed, const moe_bank *shared, const void *x_bf16, int T,
                                         int k, const float *topk_w, const moe_align_out *al, int slice_lo,
                                         int slice_hi, void *out, int out_dtype, void *stream) {
  size_t need = 0;
  int rc = qmoe::forward_workspace_need(routed, shared, x_bf16, T, k, topk_w, al, slice_lo, slice_hi, out, out_dtype,
                                        &need);
  if (rc) return rc;
  if (need > (size_t)MOE_STATIC_SCRATCH_BYTES) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "moe_expert_forward_static: this call needs %zu bytes of workspace, more than the library's fixed "
             "%zu-byte scratch; use moe_expert_forward with a caller workspace",
             need, (size_t)MOE_STATIC_SCRATCH_BYTES);
    return qmoe::set_last_error(MOE_ERR_WORKSPACE, msg);
  }
  void *ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return moe_expert_forward(routed, shared, x_bf16, T, k, topk_w, al, slice_lo, slice_hi, out, out_dtype, ws,
                            (size_t)MOE_STATIC_SCRATCH_BYTES, stream);
}

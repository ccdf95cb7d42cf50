// moe_layer_forward_noalloc: the layer forward with its workspace in a
// static device array, for callers that cannot allocate device memory.
//
// The array below is one per GPU: the runtime gives every device that loads
// this code object its own copy, at its own address. Host code never passes
// the array's name to a kernel or a copy (on the host it is only a stand-in
// for the symbol); it looks up the device address once per device with
// hipGetSymbolAddress and passes that pointer on, as the caller's workspace
// pointer is passed by moe_layer_forward.

#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on
// that device (with that device current) and kept for the process.
moe_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_layer_forward_noalloc(const moe_config* cfg, const moe_weights* w,
                                                const void* x, void* out, int32_t* ids,
                                                float* gates, int32_t* counts, void* stream) {
  const moe_status st = moe_validate_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  const size_t need = moe_workspace_size(cfg);
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const moe_status sp = scratch_ptr(&ws);
  if (sp != MOE_OK) return sp;
  // every workspace byte the forward reads is written earlier in the same
  // call, so the previous call's contents need no clearing
  return moe_layer_forward(cfg, w, x, out, ids, gates, counts, ws, MOE_NOALLOC_SCRATCH_BYTES,
                           stream);
}

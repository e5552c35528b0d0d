// The fused layer for callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid device allocation): moe_layer_forward with its workspace in a
// fixed device array of this library instead of a caller-provided buffer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"

namespace {

// The layer's scratch (h, routing arrays, dispatch order, staged expert outputs): one copy per
// GPU, created with the library's code object on that GPU and held until the process ends.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device. In host code `scratch` names a host-side
// stand-in, so the address comes from hipGetSymbolAddress, once per device (with that device
// current), and is kept for every later call. NULL on failure.
void* scratch_on_current_device() {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

}  // namespace

extern "C" int moe_layer_forward_noalloc(const moe_layer_args* a, void* stream) {
  if (!a) return MOE_ERR_NULL;
  if (a->struct_size < MOE_LAYER_ARGS_V1_SIZE) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe_workspace_size(a->T, a->d, a->E, a->H, a->k, a->dtype);
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  // T == 0 and invalid sizes (need == 0): moe_layer_forward's own checks decide, before any
  // device memory is involved
  if (need == 0) return moe_layer_forward(a, nullptr, 0, stream);
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_ERR_HIP;
  // every region of the workspace is written before it is read within a call, so nothing left by
  // an earlier call needs clearing
  return moe_layer_forward(a, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

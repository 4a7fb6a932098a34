// moe_layer_forward for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the layer's workspace is a library-owned device array instead
// of a caller buffer.
//
// `scratch` is a file-scope __device__ array, so every GPU the library runs
// on holds its own copy from module load until the process ends.  Host code
// never passes the array's name to a kernel or a copy (on the host it is only
// a stand-in symbol): the first call on a device, with that device current,
// asks HIP for the array's device address and keeps it per device; every
// later call on that device passes that address as the workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"
#include "moe_mi355x.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_WORKSPACE_BYTES];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[moe::kMaxCachedDevices] = {};

// Device address of this device's `scratch`, fetched once per device.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return moe::fail_status(MOE_ERR_HIP, "moe_layer_forward_noalloc: hipGetDevice: %s",
                                                hipGetErrorString(e));
  if (dev < 0 || dev >= moe::kMaxCachedDevices)
    return moe::fail_status(MOE_ERR_LIMIT, "moe_layer_forward_noalloc: device %d is past the %d devices served", dev,
                            moe::kMaxCachedDevices);
  std::lock_guard<std::mutex> g(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return moe::fail_status(MOE_ERR_HIP, "moe_layer_forward_noalloc: hipGetSymbolAddress(scratch): %s",
                              hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_layer_forward_noalloc(const moe_layer_desc* d, const void* x_bf16, const void* topk_ids,
                                         const float* topk_weights, void* out_bf16, hipStream_t stream) {
  const char* fn = "moe_layer_forward_noalloc";
  const int path = moe_layer_path(d);  // checks the descriptor (and a forced path)
  if (path < 0) return path;
  if (d->M == 0) return MOE_OK;
  const size_t need = moe_layer_workspace_bytes(d);
  if (need == 0) return MOE_ERR_SHAPE;
  if (need > (size_t)MOE_NOALLOC_WORKSPACE_BYTES)
    return moe::fail_status(MOE_ERR_WORKSPACE,
                            "%s: this layer needs %zu bytes of workspace, more than the %zu bytes of the "
                            "library's own array; use moe_layer_forward with a caller workspace",
                            fn, need, (size_t)MOE_NOALLOC_WORKSPACE_BYTES);
  void* ws = nullptr;
  const int rc = scratch_of_current_device(&ws);
  if (rc) return rc;
  // nothing in the workspace has to start at zero: every region the layer
  // reads was written earlier in the same call
  return moe_layer_forward(d, x_bf16, topk_ids, topk_weights, out_bf16, ws, MOE_NOALLOC_WORKSPACE_BYTES, stream);
}

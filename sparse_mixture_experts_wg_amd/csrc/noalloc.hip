// noalloc.hip -- moe_forward_noalloc: the whole layer with its workspace in a
// static device array of the library's own, for callers that cannot allocate
// device memory (code under stream capture, tight serving loops).
//
// The array `scratch` is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy, allocated when the code object is loaded
// on that GPU and kept until the process ends. In host code its name is only a
// host-side stand-in, so the device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is ever
// handed to kernels. Nothing in the layer's workspace has to start at zero:
// every step writes what a later step reads. Calls that overlap on one GPU
// share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "abi_internal.h"
#include "moe.h"

namespace {

static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch must be whole 256-byte pieces");

__device__ __attribute__((aligned(256))) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_problem *p, const void *x, const void *w_g,
                                          const void *w1, const void *w3, const void *w2,
                                          void *y, int32_t *topk_idx, float *topk_w,
                                          void *stream) {
  try {
    const int path = moe_resolve_path(p);  // validates p, sets the message on failure
    if (path < 0) return moe_status(-path);
    const size_t need = moe_forward_workspace_bytes(p);
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
      return moe::set_error(MOE_ERR_WORKSPACE,
                            "moe_forward_noalloc: this problem needs %zu bytes of workspace, the "
                            "static scratch array holds %zu (use moe_forward with a workspace)",
                            need, size_t(MOE_NOALLOC_SCRATCH_BYTES));
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
      return moe::set_error(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
      return moe::set_error(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev,
                            kMaxDevices);
    std::call_once(g_once[dev], [dev] {
      g_status[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
    });
    if (g_status[dev] != hipSuccess)
      return moe::set_error(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(g_status[dev]));
    return moe_forward(p, x, w_g, w1, w3, w2, y, topk_idx, topk_w, g_scratch[dev],
                       MOE_NOALLOC_SCRATCH_BYTES, stream);
  } catch (...) {
    return moe::set_error(MOE_ERR_HIP, "moe_forward_noalloc: internal error");
  }
}

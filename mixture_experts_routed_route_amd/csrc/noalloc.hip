// moe_forward_noalloc: the forward pass with its workspace in a file-scope
// device array instead of a caller buffer, for callers that cannot
// allocate. The array's host-side name is only a stand-in for the symbol;
// each device's copy is found once with hipGetSymbolAddress and that
// address is what the kernels get.
#include <mutex>
#include <vector>

#include "moe_internal.h"
#include "moe_noalloc.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
std::vector<void*> g_ptr;   // per device: scratch's device address, or null

// The address of `scratch` on the current device (looked up once per
// device, with that device current), or null with *err set.
void* scratch_on_current(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if ((int)g_ptr.size() <= dev) g_ptr.resize(dev + 1, nullptr);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_plan* plan, const void* x,
                                          int32_t x_dtype, moe_weight w_gate,
                                          moe_weight w_up, moe_weight w_down,
                                          int32_t D, int32_t F, void* y,
                                          int32_t y_dtype,
                                          const moe_options* opt,
                                          void* stream) {
  moe_options o;
  if (opt) o = *opt;
  else moe_options_default(&o);
  o.flags &= ~MOE_OPT_PHASE_EVENTS;   // recording would create events
  o.flags |= MOE_OPT_ONE_STREAM;      // the second stream is created on first use
  // the size query validates the plan, sizes and dtypes and names the cause
  const size_t need = moe_forward_workspace_bytes(plan, D, F, x_dtype,
                                                  w_gate.dtype, &o);
  if (need == 0) return MOE_EINVAL;
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return moe::set_error(MOE_EWORKSPACE,
                          "moe_forward_noalloc: this call needs %zu bytes of "
                          "workspace, the library's scratch holds %zu",
                          need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  hipError_t e = hipSuccess;
  void* ws = scratch_on_current(&e);
  if (!ws)
    return moe::set_error(MOE_EHIP, "moe_forward_noalloc: scratch address: %s (%s)",
                          hipGetErrorName(e), hipGetErrorString(e));
  return moe_forward(plan, x, x_dtype, w_gate, w_up, w_down, D, F, y, y_dtype,
                     ws, MOE_NOALLOC_SCRATCH_BYTES, &o, stream);
}

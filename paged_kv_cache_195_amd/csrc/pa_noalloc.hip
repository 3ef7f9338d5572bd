// pa_decode_noalloc: the decode entry point for callers that cannot allocate.
// The split-KV partials live in `scratch`, a file-scope device array (one copy
// per GPU), instead of a caller-supplied workspace.  In host code the array's
// name is only a host-side stand-in, so the device address of each GPU's copy
// is looked up once per device with hipGetSymbolAddress and only that address
// is ever handed to a kernel.
#include <mutex>

#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of the current device's copy of `scratch`.
int scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_EUNSUPPORTED;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_scratch[dev] == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
      return PA_EHIP;
    g_scratch[dev] = addr;
  }
  *ptr = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(const pa_shape* shape, const pa_options* options,
                                 const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens, float scale,
                                 int causal, int num_splits, void* out, float* lse,
                                 void* stream) {
  // Partials this call needs (0 when the split count resolves to 1 or the
  // shape is invalid; run_attention then reports the invalid shape).
  const size_t need = pa_workspace_bytes(shape, num_splits);
  if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ESCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_of_current_device(&ws);
    if (st != PA_OK) return st;
  }
  return pa::run_attention(shape, options, true, q, k_cache, v_cache, block_table, seq_lens,
                           scale, causal, num_splits, out, lse, ws,
                           need > 0 ? static_cast<size_t>(PA_NOALLOC_SCRATCH_BYTES) : 0, stream);
}

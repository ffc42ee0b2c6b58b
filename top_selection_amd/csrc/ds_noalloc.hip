// ds_topk_noalloc: ds_topk for callers that cannot allocate device memory. Its workspace (the
// split rows' per-slice survivor lists) is one file-scope device array per GPU instead of the
// per-stream cache, so a call never reaches hipMalloc; checks, plan and kernels are ds_topk's.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "ds_internal.h"

namespace {

// The scratch array, DS_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, held until the
// process ends. Host code never passes its name to a kernel or a copy: on the host the name
// is a stand-in, not the device address, which hipGetSymbolAddress gives per device below.
static __device__ __align__(256) uint8_t scratch[DS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch` on each device, once looked up

// The current device's address of `scratch` for a plan that needs `bytes` of it: looked up on
// the first call on that device (with that device current, as each device holds its own copy).
int scratch_workspace(size_t bytes, void* stream, void** out) {
  (void)stream;  // every stream of the device shares the one array
  if (bytes > static_cast<size_t>(DS_NOALLOC_SCRATCH_BYTES)) return DS_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DS_ERR_DEVICE;
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DS_ERR_DEVICE;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return DS_OK;
}

}  // namespace

extern "C" int ds_topk_noalloc(const void* x, int64_t rows, int64_t n, int64_t row_stride, int k, int dtype,
                               uint64_t seed, void* out_vals, int32_t* out_idx, void* stream) {
  return ds::topk_auto(x, rows, n, row_stride, k, dtype, seed, out_vals, out_idx, stream, scratch_workspace);
}

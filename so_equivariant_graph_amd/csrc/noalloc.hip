// so2_attention_fwd_noalloc: so2_attention_fwd with its workspace in a
// library-owned device array instead of a caller buffer, for callers that
// cannot allocate device memory (code under stream capture, tight serving
// loops).  The array is a file-scope __device__ variable, so the code object
// loader reserves it on every device the library runs on, once, for the
// life of the process; its device address is looked up per device with
// hipGetSymbolAddress on the first call on that device and kept.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace so2 {
namespace {

static __device__ __align__(256) unsigned char scratch[SO2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device).  The host-side name `scratch` is only a handle for the lookup and
// is never passed to a kernel or a copy.
so2_status scratch_address(void** out) {
  int dev = 0;
  SO2_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return SO2_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    SO2_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return SO2_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SO2_OK;
}

}  // namespace
}  // namespace so2

using namespace so2;

extern "C" so2_status so2_attention_fwd_noalloc(const so2_attn_desc* desc, const float* pos, const float* box_host,
                                                const int32_t* row_ptr, const int32_t* col, const void* x,
                                                const void* w_q, const void* w_k, const void* w_rad,
                                                const void* w_so2, float* y, so2_stream_t stream) {
  const size_t need = attention_nowait_workspace_bytes(desc);
  if (need == 0) {
    // invalid or unsupported: let the entry point name the error
    return attention_fwd_nowait(desc, pos, box_host, row_ptr, col, x, w_q, w_k, w_rad, w_so2, y, nullptr, 0, stream);
  }
  if (need > (size_t)SO2_NOALLOC_SCRATCH_BYTES) return SO2_ERR_WORKSPACE;
  void* ws = nullptr;
  const so2_status st = scratch_address(&ws);
  if (st != SO2_OK) return st;
  return attention_fwd_nowait(desc, pos, box_host, row_ptr, col, x, w_q, w_k, w_rad, w_so2, y, ws,
                              (size_t)SO2_NOALLOC_SCRATCH_BYTES, stream);
}

// swa_sink_decode for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// the decode's split partials and rotated queries live in one file-scope
// device array instead of a caller workspace.
//
// Each GPU holds its own copy of `scratch` from the moment the library's
// code object is loaded on it until the process ends.  In host code the
// array's name is only a stand-in for the symbol, never a device address:
// the address is taken once per device with hipGetSymbolAddress (with that
// device current) and only that pointer is handed to the kernels.  Every
// call on a GPU shares that GPU's array; the decode kernels write every
// partial they later read, so nothing has to be cleared between calls, and
// calls that may overlap on one GPU (different streams, host threads) race
// on it.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/hswa.h"
#include "launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[HSWA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (taken once).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" hswa_status_t swa_sink_decode_noalloc(
    const void* q, const void* k_cache, const void* v_cache, hswa_kv_layout_t layout,
    const long long* seq_offsets, const long long* pos, const float* sink, void* o, int batch,
    int hq, int hkv, int d_qk, int d_v, int window, long long max_pos, float scale,
    float rope_theta, float rotary_fraction, hswa_dtype_t dtype, void* stream) {
  const size_t need = hswa_decode_workspace_size(layout, batch, hq, d_v, window, max_pos);
  if (need > (size_t)HSWA_NOALLOC_SCRATCH_BYTES) {
    const std::string msg = "swa_sink_decode_noalloc: the call needs " + std::to_string(need) +
                            " bytes of scratch, above the static maximum of " +
                            std::to_string((size_t)HSWA_NOALLOC_SCRATCH_BYTES) +
                            " (use swa_sink_decode with a workspace)";
    return (hswa_status_t)hswa::api_fail(HSWA_ERR_INVALID_ARGUMENT, msg.c_str());
  }
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) {
      const std::string msg = std::string("swa_sink_decode_noalloc: address of the static scratch: ") +
                              hipGetErrorString(e);
      return (hswa_status_t)hswa::api_fail(HSWA_ERR_HIP, msg.c_str());
    }
  }
  return swa_sink_decode(q, k_cache, v_cache, layout, seq_offsets, pos, sink, o, batch, hq, hkv,
                         d_qk, d_v, window, max_pos, scale, rope_theta, rotary_fraction, dtype, ws,
                         need > 0 ? (size_t)HSWA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

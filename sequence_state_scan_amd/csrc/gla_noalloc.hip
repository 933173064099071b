// gla_chunk_fwd_noalloc: gla_chunk_fwd with its workspace in a library-owned device array, for
// callers that cannot allocate device memory (code under graph capture, tight serving loops).
//
// The array `scratch` below is a file-scope __device__ variable: every GPU the library runs on
// holds its own copy, for as long as the process lives.  In host code its name is only a
// host-side stand-in, so the host never passes it to a kernel: on the first call on a device
// (that device current) hipGetSymbolAddress gives that device's address, which is kept per device
// and passed to the kernels as the workspace.  The call itself allocates nothing.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gla.h"
#include "gla_kernels.hpp"

namespace {

constexpr int kMaxDevices = 64;
// One int flag per unit (b, h, segment): room for B * H * P <= kStaticUnits.
static __device__ __align__(256) int scratch[gla::kStaticUnits];

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// The calling thread's current device's copy of `scratch` (looked up once per device).
gla_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return gla::set_error(GLA_ERR_HIP, "gla_chunk_fwd_noalloc: hipGetDevice failed: %s",
                                             hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return gla::set_error(GLA_ERR_UNSUPPORTED, "gla_chunk_fwd_noalloc: device %d is beyond the %d this library serves",
                          dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return gla::set_error(GLA_ERR_HIP, "gla_chunk_fwd_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s",
                            dev, hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return GLA_OK;
}

}  // namespace

extern "C" gla_status gla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g, void* o,
                                            void* chunk_states, float* seg_state, float* seg_logdecay, int B, int H,
                                            int T, int dk, int dv, int chunk, int P, int dtype, void* stream) {
  // the same host checks as gla_chunk_fwd, then the size limit of the static scratch
  const size_t need = gla_workspace_size(GLA_FWD, B, H, T, dk, dv, chunk, P, dtype);
  if (need == 0) return gla::last_status();  // rejected; the message is set
  if ((long long)B * H * P > gla::kStaticUnits)
    return gla::set_error(GLA_ERR_INVALID_ARG,
                          "gla_chunk_fwd_noalloc: B*H*P = %lld units exceed the static scratch (%d units); "
                          "call gla_chunk_fwd with a workspace instead",
                          (long long)B * H * P, gla::kStaticUnits);
  void* ws = nullptr;
  const gla_status st = scratch_ptr(&ws);
  if (st != GLA_OK) return st;
  // the scratch holds the per-unit flags only: offered as a workspace of just that size (one int
  // per unit, rounded up to 256 bytes), the call cuts no sub-segments and re-splits no units
  const size_t flags_bytes = ((size_t)B * H * P * sizeof(int) + 255) / 256 * 256;
  return gla::chunk_fwd_capped(q, k, v, g, nullptr, o, chunk_states, seg_state, seg_logdecay, B, H, T, dk, dv, chunk,
                               P, dtype, ws, flags_bytes, 1, stream);
}

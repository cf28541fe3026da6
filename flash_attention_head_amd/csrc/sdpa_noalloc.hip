// sdpa_forward_noalloc: sdpa_forward for callers that cannot allocate device
// memory.  The split partials that sdpa_forward keeps in the caller's
// workspace live here in one file-scope device array per GPU instead.  The
// contract is in include/sdpa_mi355x.h.
#include <mutex>

#include "sdpa_internal.h"
#include "sdpa_mi355x.h"

#define SDPA_API extern "C" __attribute__((visibility("default")))

namespace sdpa {
namespace {

// Every GPU the library runs on holds its own copy of this array from the
// first call on that GPU until the process ends.
constexpr size_t kScratchBytes = (size_t)SDPA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of each GPU's copy.  In host code `scratch` names a
// host-side stand-in, never the device memory; only these addresses, taken
// once per device with that device current, reach a kernel.
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices] = {};

}  // namespace
}  // namespace sdpa

using namespace sdpa;

SDPA_API int sdpa_forward_noalloc(const void* q, const void* k, const void* v, void* out, int B, int Hq,
                                  int Hkv, int qL, int kL, int D, float scale, int causal, int window,
                                  int q_offset, int dtype, void* stream) {
  clear_error();
  // every argument check before any HIP call
  const size_t need = sdpa_workspace_bytes(B, Hq, Hkv, qL, kL, D);
  if (need != (size_t)-1 && need > kScratchBytes)
    return fail(SDPA_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of scratch; sdpa_forward_noalloc holds %zu (use sdpa_forward with a "
                "workspace)",
                need, kScratchBytes);
  // (the check-only pass is given a non-null stand-in for the workspace; it
  // reads and launches nothing)
  int rc = forward_plain(q, k, v, out, B, Hq, Hkv, qL, kL, D, scale, causal, window, q_offset, dtype,
                         need > 0 ? (void*)&g_scratch : nullptr, kScratchBytes, stream, false);
  if (rc != SDPA_OK) return rc;
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SDPA_HIP_ERROR, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(SDPA_HIP_ERROR, "device %d is beyond the %d supported", dev, kMaxDevices);
    std::call_once(g_scratch_once[dev], [dev] {
      void* ptr = nullptr;
      g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (g_scratch_err[dev] == hipSuccess) g_scratch[dev] = ptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch[dev])
      return fail(SDPA_HIP_ERROR, "hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
                  hipGetErrorString(g_scratch_err[dev]));
    ws = g_scratch[dev];
  }
  return forward_plain(q, k, v, out, B, Hq, Hkv, qL, kL, D, scale, causal, window, q_offset, dtype, ws,
                       kScratchBytes, stream, true);
}

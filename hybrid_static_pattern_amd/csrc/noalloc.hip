// saf_attn_bwd_noalloc: the hybrid backward of saf_attn_bwd with its workspace taken from a
// fixed device array of this library instead of a caller buffer, for callers that cannot
// allocate (code under graph capture, tight serving loops, harnesses that forbid it).
//
// The array lives in device memory once per GPU the library runs on, for the life of the
// process. Its address on the current device is looked up once per device (with that device
// current) and kept; host code never passes the array's own name to a kernel or a copy, only
// that looked-up address. The backward's kernels write every workspace entry they later read
// (delta and lse * log2(e) of the ordinary rows; per-query-head dK, dV with shared key/value
// heads), so nothing needs clearing between calls. Calls that overlap on one GPU (two streams,
// or two threads) share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "saf.h"
#include "saf_internal.h"

constexpr size_t kScratchBytes = SAF_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Address of the current device's copy of `scratch`, looked up on the first call on that device.
saf_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return saf::set_error(SAF_EHIP, "hipGetDevice failed in saf_attn_bwd_noalloc");
  if (dev < 0 || dev >= kMaxDevices) return saf::set_error(SAF_EUNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return saf::set_error(SAF_EHIP, "hipGetSymbolAddress(scratch) failed");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return SAF_OK;
}

}  // namespace

extern "C" saf_status saf_attn_bwd_noalloc(const saf_attn_desc* desc, const void* q, const void* k,
                                           const void* v, const void* o, const void* dO, const float* lse,
                                           const float* alpha, const float* rho, void* dq, void* dk, void* dv,
                                           void* stream) {
  // An invalid descriptor reports 0 bytes here and its error from saf_attn_bwd below.
  const size_t need = saf_attn_workspace_size(desc);
  if (need > kScratchBytes)
    return saf::set_error(SAF_EWORKSPACE, "saf_attn_bwd_noalloc: this layer needs %zu bytes of workspace, the "
                                          "built-in scratch holds %zu; call saf_attn_bwd with a workspace",
                          need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const saf_status st = scratch_ptr(&ws);
    if (st != SAF_OK) return st;
  }
  return saf_attn_bwd(desc, q, k, v, o, dO, lse, alpha, rho, dq, dk, dv, ws, need > 0 ? kScratchBytes : 0, stream);
}

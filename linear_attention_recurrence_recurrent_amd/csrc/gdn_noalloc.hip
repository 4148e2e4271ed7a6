// gdn_scan_noalloc (include/gdn.h): gdn_scan for callers that cannot allocate
// device memory, with the block form's records in a static device array.
//
// `scratch` is a file-scope device array; every GPU the library runs on holds
// its own copy (at its own address) until the process ends.  In host code the
// name `scratch` is only a host-side handle of the symbol, not a device
// address: the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept in g_scratch; only
// that pointer is ever passed to kernels.  Every call on a GPU shares the
// GPU's array, so calls that overlap on one GPU (different streams, or
// threads) race on it; calls ordered on one stream do not.  The kernels write
// every record they read, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first call
// on that device), or nullptr with the reason in the thread's last error.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    set_error("gdn_scan_noalloc: no usable current HIP device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      set_error("gdn_scan_noalloc: hipGetSymbolAddress of the static scratch failed");
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace
}  // namespace gdn

extern "C" int gdn_scan_noalloc(const gdn_desc* d, const void* q, const void* k, const void* v,
                                const void* log_decay, const void* beta, const float* s0,
                                const void* z, const void* w, float* y, float* s_out,
                                void* stream) {
  int rc = gdn::check_desc(d);
  if (rc != GDN_OK) return rc;
  const int64_t need = gdn::scan_workspace_bytes(*d);
  if (need > (int64_t)GDN_NOALLOC_SCRATCH_BYTES) {
    char msg[200];
    std::snprintf(msg, sizeof(msg),
                  "gdn_scan_noalloc: this shape needs %lld bytes of scratch, above the static "
                  "%llu (use gdn_scan with a workspace)",
                  (long long)need, (unsigned long long)GDN_NOALLOC_SCRATCH_BYTES);
    gdn::set_error(msg);
    return GDN_EWORKSPACE;
  }
  void* ws = nullptr;
  if (need > 0 && (ws = gdn::device_scratch()) == nullptr) return GDN_EDEVICE;
  rc = gdn::check(d, q, k, v, log_decay, beta, s0, z, w, y, s_out, ws,
                  need > 0 ? GDN_NOALLOC_SCRATCH_BYTES : 0);
  if (rc != GDN_OK) return rc;
  return gdn::run_scan(*d, q, k, v, log_decay, beta, s0, z, w, y, s_out, ws, stream);
}

// C-ABI entry points (include/gdn.h): validate, then enqueue the kernels.
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "gdn_internal.h"
#include "gdn_launch.h"

namespace gdn {

int run_scan(const gdn_desc& d, const void* q, const void* k, const void* v,
             const void* log_decay, const void* beta, const float* s0, const void* z,
             const void* w, float* y, float* s_out, void* workspace, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d.B == 0) return GDN_OK;
  if (d.T == 0) {
    if (s_out == s0) return GDN_OK;
    const size_t bytes = (size_t)(d.B * d.Hv * d.Dv * d.Dk) * sizeof(float);
    if (hipMemcpyAsync(s_out, s0, bytes, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return device_status("state copy for T == 0");
    return GDN_OK;
  }
  if (d.T == 1)  // one token: the decode kernel is the same computation, streamed once
    return launch_step(d, q, k, v, log_decay, beta, s0, z, w, y, s_out, stream);
  return launch_scan(d, q, k, v, log_decay, beta, s0, z, w, y, s_out, workspace, stream);
}

}  // namespace gdn

extern "C" {

int gdn_recurrent_step(const gdn_desc* d, const void* q, const void* k, const void* v,
                       const void* log_decay, const void* beta, const float* s0, const void* z,
                       const void* w, float* y, float* s_out, void* stream) {
  int rc = gdn::check(d, q, k, v, log_decay, beta, s0, z, w, y, s_out, nullptr, 0);
  if (rc != GDN_OK) return rc;
  if (d->T != 1) {
    gdn::set_error("gdn_recurrent_step needs T == 1 (use gdn_scan for a time axis)");
    return GDN_EUNSUPPORTED;
  }
  if (d->B == 0) return GDN_OK;
  return gdn::launch_step(*d, q, k, v, log_decay, beta, s0, z, w, y, s_out, stream);
}

int gdn_recurrent_step_three_pass(const gdn_desc* d, const void* q, const void* k,
                                  const void* v, const void* log_decay, const void* beta,
                                  const float* s0, const void* z, const void* w, float* y,
                                  float* s_out, void* stream) {
  int rc = gdn::check(d, q, k, v, log_decay, beta, s0, z, w, y, s_out, nullptr, 0);
  if (rc != GDN_OK) return rc;
  if (d->T != 1) {
    gdn::set_error("gdn_recurrent_step_three_pass needs T == 1");
    return GDN_EUNSUPPORTED;
  }
  if (d->B == 0) return GDN_OK;
  return gdn::launch_step_three_pass(*d, q, k, v, log_decay, beta, s0, z, w, y, s_out, stream);
}

int gdn_scan(const gdn_desc* d, const void* q, const void* k, const void* v,
             const void* log_decay, const void* beta, const float* s0, const void* z,
             const void* w, float* y, float* s_out, void* workspace, uint64_t workspace_bytes,
             void* stream) {
  int rc = gdn::check(d, q, k, v, log_decay, beta, s0, z, w, y, s_out, workspace,
                      workspace_bytes);
  if (rc != GDN_OK) return rc;
  return gdn::run_scan(*d, q, k, v, log_decay, beta, s0, z, w, y, s_out, workspace, stream);
}

int gdn_gates(int64_t n, const void* a, const void* b, int32_t in_dtype, float decay_scale,
              void* log_decay, void* beta, int32_t out_dtype, void* stream) {
  int rc = gdn::check_gates(n, a, b, in_dtype, decay_scale, log_decay, beta, out_dtype);
  if (rc != GDN_OK || n == 0) return rc;
  return gdn::launch_gates(n, a, b, in_dtype, decay_scale, log_decay, beta, out_dtype, stream);
}

int gdn_conv_silu(int64_t B, int64_t T, int64_t C, int32_t W, int32_t dtype, int32_t apply_silu,
                  const void* x, const void* w, const void* bias, const void* state_in, void* y,
                  void* state_out, void* stream) {
  int rc = gdn::check_conv(B, T, C, W, dtype, apply_silu, x, w, bias, state_in, y, state_out);
  if (rc != GDN_OK || B == 0 || C == 0) return rc;
  if (T == 0 && (state_out == nullptr || W == 1)) return GDN_OK;
  return gdn::launch_conv(B, T, C, W, dtype, apply_silu, x, w, bias, state_in, y, state_out,
                          stream);
}

}  // extern "C"

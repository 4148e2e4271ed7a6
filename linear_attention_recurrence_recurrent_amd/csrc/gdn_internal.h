// Internal declarations shared by the host-side validator and the HIP launchers.
#pragma once

#include "gdn.h"

namespace gdn {

// Validation behind gdn_check (sets the thread's last error on failure).
int check(const gdn_desc* d, const void* q, const void* k, const void* v, const void* log_decay,
          const void* beta, const float* s0, const void* z, const void* w, const float* y,
          const float* s_out);

// Validation behind gdn_gates.
int check_gates(int64_t n, const void* a, const void* b, int32_t in_dtype, float decay_scale,
                const void* log_decay, const void* beta, int32_t out_dtype);

// Replace the thread's last-error text.
void set_error(const char* msg);

// Launchers (validated arguments; stream is a hipStream_t).  They return GDN_OK,
// GDN_EUNSUPPORTED or GDN_EDEVICE.
int launch_step(const gdn_desc& d, const void* q, const void* k, const void* v, const void* ld,
                const void* beta, const float* s0, const void* z, const void* w, float* y,
                float* s_out, void* stream);
int launch_step_three_pass(const gdn_desc& d, const void* q, const void* k, const void* v,
                           const void* ld, const void* beta, const float* s0, const void* z,
                           const void* w, float* y, float* s_out, void* stream);
int launch_scan(const gdn_desc& d, const void* q, const void* k, const void* v, const void* ld,
                const void* beta, const float* s0, const void* z, const void* w, float* y,
                float* s_out, void* stream);

int launch_gates(int64_t n, const void* a, const void* b, int in_dtype, float decay_scale,
                 void* log_decay, void* beta, int out_dtype, void* stream);

}  // namespace gdn

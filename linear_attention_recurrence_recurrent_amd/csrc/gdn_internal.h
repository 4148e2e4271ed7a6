// Internal declarations shared by the host-side validator and the HIP launchers.
#pragma once

#include "gdn.h"

namespace gdn {

// Layout of the block form's workspace (shared by the validator, which sizes
// it, and the launcher, which lays it out): a record of kBlockRecordBytes per
// (value head, 16-token block), then, when the few-head kernel runs
// (scan_uses_key_products), kKeyCrossBytes per (key head, block).
constexpr int64_t kBlockTokens = 16;
constexpr int64_t kBlockRecordBytes = 2560;
constexpr int64_t kKeyCrossBytes = 3 * 16 * 16 * 4;
constexpr int64_t kManyHeads = 256;
constexpr uintptr_t kWorkspaceAlign = 256;

// Whether the block form covers the head dim (Dk == Dv in {32, 64, 128, 256}).
bool block_head_dims_fit(const gdn_desc& d);
// ... and the shape: Hk*Dk and Hv*Dv below 2^27 and T below 2^29, which keep
// the kernels' 32-bit offsets inside a 16-token block in range.
bool block_form_fits(const gdn_desc& d);
// Whether gdn_scan runs the block form for this (valid) descriptor.
bool scan_uses_block_form(const gdn_desc& d);
// Whether the block form runs its few-head kernel (fewer than kManyHeads value
// heads, or D = 256), which also keeps the cross-block key products.
bool scan_uses_key_products(const gdn_desc& d);
// Bytes of the records (first part of the workspace) and in total.
int64_t scan_record_bytes(const gdn_desc& d);
int64_t scan_workspace_bytes(const gdn_desc& d);

// A launch's work-items (grid x workgroup) travel as a 32-bit count in the
// dispatch packet, and a larger grid is not reliably refused by the runtime
// (it can wrap to a few workgroups), so every launch stays at or below this.
constexpr int64_t kMaxLaunchItems = ((int64_t)1 << 32) - 1;
// The most work-items any one launch of the call that `d` describes takes
// (gdn_recurrent_step, its three-pass form, or gdn_scan), from the shapes the
// launchers pick; 0 when nothing is launched.
int64_t max_launch_items(const gdn_desc& d);

// Descriptor validation (no pointers); sets the thread's last error on failure.
int check_desc(const gdn_desc* d);

// Validation behind gdn_check (sets the thread's last error on failure).  The
// workspace is checked against scan_workspace_bytes(*d).
int check(const gdn_desc* d, const void* q, const void* k, const void* v, const void* log_decay,
          const void* beta, const float* s0, const void* z, const void* w, const float* y,
          const float* s_out, const void* workspace, uint64_t workspace_bytes);

// Validation behind gdn_gates.
int check_gates(int64_t n, const void* a, const void* b, int32_t in_dtype, float decay_scale,
                const void* log_decay, const void* beta, int32_t out_dtype);

// Validation behind gdn_conv_silu.
int check_conv(int64_t B, int64_t T, int64_t C, int32_t W, int32_t dtype, int32_t apply_silu,
               const void* x, const void* w, const void* bias, const void* state_in,
               const void* y, const void* state_out);

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
                float* s_out, void* workspace, void* stream);
// Block form on the matrix cores (block_form_fits), with its records in
// `workspace` (scan_workspace_bytes(d) bytes); *gated reports whether the
// gated norm was applied in the same launch (whole-head workgroups).
int launch_scan_chunked(const gdn_desc& d, const void* q, const void* k, const void* v,
                        const void* ld, const void* beta, const float* s0, const void* z,
                        const void* w, float* y, float* s_out, void* workspace, void* stream,
                        bool* gated);

// gdn_scan after validation: the empty cases, T == 1 on the decode kernel,
// else the scan (the workspace, validated, holds scan_workspace_bytes(d)).
int run_scan(const gdn_desc& d, const void* q, const void* k, const void* v,
             const void* log_decay, const void* beta, const float* s0, const void* z,
             const void* w, float* y, float* s_out, void* workspace, void* stream);

int launch_gates(int64_t n, const void* a, const void* b, int in_dtype, float decay_scale,
                 void* log_decay, void* beta, int out_dtype, void* stream);

int launch_conv(int64_t B, int64_t T, int64_t C, int W, int dtype, int apply_silu,
                const void* x, const void* w, const void* bias, const void* state_in, void* y,
                void* state_out, void* stream);

}  // namespace gdn

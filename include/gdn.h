/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet recurrence library
 * (libgdn_hip.so).
 *
 * What the library computes.  Each value head (b, hv) keeps a D x D float32
 * memory S whose row a is a value lane and whose column c is a key lane
 * (S is stored [B, Hv, Dv, Dk]).  Per token, with q, k read from key head
 * hk = hv / (Hv / Hk):
 *     k^ = k / sqrt(sum k^2 + qk_eps)              (GDN_FOLD_QK_L2NORM)
 *     q^ = q / sqrt(sum q^2 + qk_eps) / sqrt(Dk)   (GDN_FOLD_QK_L2NORM, GDN_FOLD_Q_SCALE)
 *     alpha = exp(log_decay),  beta as given
 *     u = S.k^ ;  S = alpha*S + beta*(v - alpha*u) k^T ;  o = S.q^  (updated S)
 *     y = rmsnorm(o * silu(z)) * w   when z and w are given, else y = o.
 * Sources: the "Module gdn" page (logicaffeine codegen_cuda/gdn), module
 * description, for the recurrence and the gate-first RMSNorm, and its section
 * "The fusion" for the single pass per state row that the kernels use
 * (o = alpha*(S_old.q) + coef*(k.q), coef = beta*(v - alpha*u)); the
 * "gated_delta" page (torch-to-nnef op reference): emit_native_gdn_recurrent
 * for the operand tuple (q, k, v, log_decay, beta, s0), the [B, S, H, W] and
 * head-major [B, H, S, W] layouts and the caller-created (output,
 * final_state); gated_delta_fake for the float32 output whatever the input
 * dtype; native_gdn_reject_reason for the folded q/k L2 norm and
 * 1/sqrt(head_dim) scale and the short reject reason; native_gdn_min_version
 * for the version query.
 *
 * Conventions common to every call.
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, dense and
 *     row-major in the layout given below.  The library keeps no state
 *     between calls and never synchronises: all work is enqueued on `stream`
 *     (a hipStream_t; NULL is the null stream) on the current HIP device, and
 *     the call returns as soon as it is enqueued.  It allocates nothing,
 *     except the block form of gdn_scan (below), which takes a stream-ordered
 *     workspace with hipMallocAsync on `stream` and returns it with
 *     hipFreeAsync on the same stream before the call returns.
 *   - Layouts (head_major == 0 / 1):
 *         q, k        [B, T, Hk, Dk]   /  [B, Hk, T, Dk]      dtype
 *         v, z        [B, T, Hv, Dv]   /  [B, Hv, T, Dv]      dtype
 *         log_decay,
 *         beta        [B, T, Hv]       /  [B, Hv, T]          gate_dtype
 *         y           [B, T, Hv, Dv]   /  [B, Hv, T, Dv]      float32
 *         s0, s_out   [B, Hv, Dv, Dk]                          float32
 *         w           [Dv]                                     dtype
 *   - z and w are optional and go together: both NULL gives the raw output
 *     y = o; both given gives the gated output.
 *   - s_out may be exactly s0 (in-place state update); any other overlap
 *     between an output and any operand is rejected.
 *   - q, k, v, z, y, s0, s_out must be 16-byte aligned; log_decay, beta and w
 *     aligned to their element size.
 *   - Supported by the kernels: Dk == Dv in {16, 32, 64, 128, 256}; dtype and
 *     gate_dtype in {GDN_F32, GDN_F16, GDN_BF16}; Hv a multiple of Hk.
 *   - Size limits (GDN_ESHAPE): B*T*Hv below 2^31, and every kernel launch of
 *     the call at most 2^32 - 1 threads (the 32-bit grid size of a dispatch):
 *     about B*Hv*1024 for the decode at D >= 128, B*Hv*12288 for the scan at
 *     D = 256, 4*B*T*Hk for the block form's per-block prep.  Larger calls
 *     are rejected, not split.
 *   - Error behaviour: every call returns GDN_OK or a gdn_status; the short
 *     reason of the last failure on the calling thread is gdn_last_error().
 *     A rejected call enqueues nothing.  A HIP launch failure returns
 *     GDN_EDEVICE.  NaN/Inf in the operands propagate; they are not checked.
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

typedef enum gdn_dtype { GDN_F32 = 0, GDN_F16 = 1, GDN_BF16 = 2 } gdn_dtype;

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_EINVAL = 1,       /* null descriptor or pointer, bad flag, eps or layout value */
  GDN_ESHAPE = 2,       /* negative or zero extent, or sizes that overflow */
  GDN_EDTYPE = 3,       /* dtype or gate_dtype not one of gdn_dtype */
  GDN_EGROUP = 4,       /* Hv is not a multiple of Hk */
  GDN_EUNSUPPORTED = 5, /* valid, but not covered by the kernels (head dims, T != 1 for a step) */
  GDN_EALIGN = 6,       /* pointer alignment */
  GDN_EALIAS = 7,       /* an output overlaps an operand (other than s_out == s0) */
  GDN_EDEVICE = 8,      /* the HIP runtime reported an error */
  GDN_EWORKSPACE = 9    /* gdn_scan's workspace is missing or smaller than it needs */
} gdn_status;

/* flags */
#define GDN_FOLD_QK_L2NORM 1u /* L2-normalise q and k inside the op */
#define GDN_FOLD_Q_SCALE 2u   /* multiply q^ by 1/sqrt(Dk) inside the op */
/* Form of gdn_scan's time loop.  The token-by-token form runs on the vector
 * units for every head dim; at Dk == Dv in {32, 64, 128, 256} the block form
 * runs 16 tokens at a time as dense products on the matrix cores (the step is affine in S,
 * "Module gdn" page, "The fusion").  Both give the same results up to
 * rounding.  With f16/bf16 q and k the block form multiplies the f32 state
 * (and its per-block correction) on the bf16 matrix cores through bf16 parts:
 * by default two parts rounded to nearest, each term then within 2^-16
 * relative of the f32 product; with GDN_SCAN_EXACT three exact parts, each
 * term an exact f32 product (f32 accuracy; up to 1.2x the time).
 * f32 q and k take f32 products either way (at D == 256 too).  The block form also needs
 * Hk*Dk and Hv*Dv below 2^27 and T below 2^29 (its offsets inside a block are
 * 32-bit).  Without a form flag the block form runs where it fits and the
 * token-by-token form otherwise; with both form flags, or GDN_SCAN_BLOCK
 * where the block form does not fit, the call is rejected (GDN_EINVAL /
 * GDN_EUNSUPPORTED).  The block form keeps per-block
 * records in a caller-supplied workspace (gdn_scan_workspace_size). */
#define GDN_SCAN_PER_TOKEN 4u
#define GDN_SCAN_BLOCK 8u
#define GDN_SCAN_EXACT 16u

typedef struct gdn_desc {
  int64_t B, T, Hk, Hv, Dk, Dv; /* batch, tokens, key heads, value heads, head dims */
  int32_t head_major;           /* 0: [B, T, H, ...] operands; 1: [B, H, T, ...] */
  int32_t dtype;                /* gdn_dtype of q, k, v, z, w */
  int32_t gate_dtype;           /* gdn_dtype of log_decay and beta */
  uint32_t flags;               /* GDN_FOLD_* bits */
  float qk_eps;                 /* eps inside the q/k L2 norm's square root (1e-6) */
  float norm_eps;               /* eps of the gated RMSNorm (1e-6) */
} gdn_desc;

/* One decode step (d->T must be 1): reads s0, writes y [B, 1, Hv, Dv] and the
 * updated state to s_out (s_out == s0 updates the state in place).  The
 * fused decode operator of the "gated_delta" page (native_gdn_reject_reason)
 * with the recurrence and gated norm of the "Module gdn" page.  Each state
 * row is read from memory once and written once. */
int gdn_recurrent_step(const gdn_desc* d, const void* q, const void* k, const void* v,
                       const void* log_decay, const void* beta, const float* s0,
                       const void* z, const void* w, float* y, float* s_out, void* stream);

/* The same step without the fusion ("Module gdn" page, "The fusion": the
 * unfused step visits the state three times, for the product with k, for the
 * rank-1 update and for the product with q), as three launches: u = S.k into
 * the y buffer (reads S), the update (reads S, writes s_out), o = S.q on the
 * updated state plus the output (reads s_out).  Same arguments and results
 * as gdn_recurrent_step; it exists to measure the fusion's saving (three
 * reads and one write of the state instead of one read and one write).
 * The passes are ordered on `stream`, so s_out == s0 (in place) is allowed
 * as for gdn_recurrent_step.  Supported for Dk == Dv == 128 only (else
 * GDN_EUNSUPPORTED). */
int gdn_recurrent_step_three_pass(const gdn_desc* d, const void* q, const void* k,
                                  const void* v, const void* log_decay, const void* beta,
                                  const float* s0, const void* z, const void* w, float* y,
                                  float* s_out, void* stream);

/* Bytes of device workspace gdn_scan needs for the descriptor `d`, written to
 * *bytes.  Zero when the chosen time loop keeps nothing between its kernels
 * (T <= 1, B == 0, the token-by-token form).  The block form (where it runs,
 * see GDN_SCAN_BLOCK, unless GDN_SCAN_PER_TOKEN) needs one 2560-byte record
 * per value head and 16-token block, plus 3072 bytes per key head and block
 * when B * Hv is below 256 or the head dim is 256 (the few-head kernel's
 * cross-block key products):
 *     B*Hv*ceil(T/16)*2560  [+ B*Hk*ceil(T/16)*3072].
 * Validates the descriptor as gdn_check does (pointers aside) and returns
 * GDN_OK or that status.  Host-only, no device work. */
int gdn_scan_workspace_size(const gdn_desc* d, uint64_t* bytes);

/* The recurrence over the whole time axis ("gated_delta" page,
 * gated_delta_reference: the recurrence over the time axis returning
 * (output, final_state)).  Any T >= 0; T == 0 copies s0 to s_out (unless
 * they are the same buffer) and writes no y.  The state stays on chip for
 * the whole time axis; s_out receives the state after the last token.
 * The form of the time loop follows GDN_SCAN_PER_TOKEN / GDN_SCAN_BLOCK.
 * workspace: caller-owned device memory of at least
 * gdn_scan_workspace_size() bytes, 256-byte aligned, overlapping no operand
 * or output, used only by the work this call enqueues (it may be reused or
 * freed once that work has finished on `stream`).  May be NULL when the size
 * is 0.  Too small or NULL when needed: GDN_EWORKSPACE; misaligned:
 * GDN_EALIGN; overlapping: GDN_EALIAS; in each case nothing is enqueued. */
int gdn_scan(const gdn_desc* d, const void* q, const void* k, const void* v,
             const void* log_decay, const void* beta, const float* s0, const void* z,
             const void* w, float* y, float* s_out, void* workspace, uint64_t workspace_bytes,
             void* stream);

/* gdn_scan for callers that cannot allocate device memory at all: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as gdn_scan without the workspace: the block
 * form's records go to a static device array of GDN_NOALLOC_SCRATCH_BYTES
 * that every GPU the library runs on holds until the process ends (its device
 * address is looked up on the first call on each device).  A shape whose
 * workspace (gdn_scan_workspace_size) exceeds it is rejected with
 * GDN_EWORKSPACE before anything is enqueued; the prefill shape B=1 T=4096
 * Hk=16 Hv=32 needs exactly 32 MiB.  All calls on one GPU share its array:
 * calls ordered on one stream are safe, calls that overlap on one GPU (other
 * streams or threads) race on it and give undefined results.  Allocates
 * nothing (no hipMalloc, no allocating library routine). */
#define GDN_NOALLOC_SCRATCH_BYTES (64ull << 20)
int gdn_scan_noalloc(const gdn_desc* d, const void* q, const void* k, const void* v,
                     const void* log_decay, const void* beta, const float* s0, const void* z,
                     const void* w, float* y, float* s_out, void* stream);

/* Gate producer: both gates from their pre-activations in one launch ("Module
 * gdn" page, QWEN38_KERNELS: the gate kernel computes both gates from one
 * launch; the pages do not give the formulas, these are the workloads' own):
 *     log_decay[i] = -decay_scale * softplus(a[i]),   beta[i] = sigmoid(b[i]).
 * a, b: n device elements of in_dtype; log_decay, beta: n device elements of
 * out_dtype (16-bit outputs rounded to nearest even), ready to be passed to
 * gdn_recurrent_step / gdn_scan as their gates.  Pointers aligned to their
 * element size; outputs must not overlap inputs or each other (GDN_EALIAS).
 * n == 0 does nothing; n must be below 2^33 (one launch of n/4 threads).
 * Asynchronous on `stream`, allocates nothing. */
int gdn_gates(int64_t n, const void* a, const void* b, int32_t in_dtype, float decay_scale,
              void* log_decay, void* beta, int32_t out_dtype, void* stream);

/* Producer of q, k and v: causal depthwise convolution over the time axis with
 * the silu fused in ("Module gdn" page, QWEN38_KERNELS: the convolution
 * carries the silu).  The pages give neither the width nor the weight layout;
 * this is the usual causal form, one filter of W taps per channel with the
 * last tap on the current token:
 *     pre[b,t,c] = bias[c] + sum_{i<W} w[c*W + i] * xx(b, t - (W-1) + i, c)
 *     xx(b,t',c) = x[(b*T + t')*C + c] for t' >= 0, else the carried context
 *                  state_in[(b*C + c)*(W-1) + (W-1) + t'] (zero when NULL)
 *     y[(b*T + t)*C + c] = apply_silu ? pre * sigmoid(pre) : pre
 *     state_out[(b*C + c)*(W-1) + j] = xx(b, T - (W-1) + j, c),  j < W-1
 * x, y: [B, T, C]; w: [C, W]; bias: [C] or NULL; state_in, state_out:
 * [B, C, W-1] or NULL (state_out NULL: not written).  Every tensor is dtype
 * (y rounded to nearest even for 16-bit types; the state holds exact copies of
 * inputs).  1 <= W <= 8; C and B*ceil(T/16) below 2^31 (one launch, a thread
 * per one or four channels across).  Device pointers aligned to the element size
 * (16-byte alignment of x and y and C % 4 == 0 take the vector path).
 * state_out may be exactly state_in (updated in place); any other overlap of
 * an output with an operand is GDN_EALIAS.  T == 0 only writes state_out
 * (= state_in, or zeros).  Decode is T == 1 with a state.  Asynchronous on
 * `stream`, allocates nothing; returns GDN_OK or a gdn_status with its reason
 * in gdn_last_error(). */
int gdn_conv_silu(int64_t B, int64_t T, int64_t C, int32_t W, int32_t dtype, int32_t apply_silu,
                  const void* x, const void* w, const void* bias, const void* state_in, void* y,
                  void* state_out, void* stream);

/* Validation only, no device work: GDN_OK when gdn_scan would accept these
 * arguments (workspace included), else the status with its short reason in
 * gdn_last_error() ("gated_delta" page, native_gdn_reject_reason: a rejected
 * operand comes with a short, loggable reason, so the caller can fall back).
 * Host-only; safe to call on a machine with no GPU. */
int gdn_check(const gdn_desc* d, const void* q, const void* k, const void* v,
              const void* log_decay, const void* beta, const float* s0, const void* z,
              const void* w, const float* y, const float* s_out, const void* workspace,
              uint64_t workspace_bytes);

/* Short reason for the last non-OK status returned on this thread ("" if
 * none): the loggable reject reason of the "gated_delta" page,
 * native_gdn_reject_reason.  The text stays valid until the thread's next
 * call into the library. */
const char* gdn_last_error(void);

/* Static name of a gdn_status value ("GDN_UNKNOWN" for other values), for
 * the same logging. */
const char* gdn_status_str(int status);

/* GDN_ABI_VERSION of the loaded library ("gated_delta" page,
 * native_gdn_min_version: the first release carrying the fused operator). */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */

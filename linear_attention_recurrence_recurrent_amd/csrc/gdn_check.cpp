// Host-side argument validation of the C ABI (pure C++, no HIP calls).
//
// The fused operator of the "gated_delta" page (native_gdn_reject_reason) has
// hard constraints checked before anything runs, and a rejected call returns
// a short reason for logging.  gdn_check is that check; gdn_scan and
// gdn_recurrent_step run it before every launch.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int64_t elem_size(int32_t dt) { return dt == GDN_F32 ? 4 : 2; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a == 0 || b == 0) {
    *out = 0;
    return true;
  }
  if (a > INT64_MAX / b) return false;
  *out = a * b;
  return true;
}

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

}  // namespace

namespace gdn {

void set_error(const char* msg) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
}

// Work-items per value head of the decode kernel (launch_step_sp) and of the
// per-token scan kernel (launch_scan_dt / launch_scan_cfg: workgroups of 16,
// 32, 64 or 128 rows at D = 128, by head count).
static int64_t step_threads_per_head(int64_t D) { return D >= 128 ? 1024 : D >= 32 ? 128 : 64; }
static int64_t scan_threads_per_head(int64_t D, int64_t heads) {
  switch (D) {
    case 256: return 16 * 256;
    case 128: return heads >= 512 ? 256 : heads >= 128 ? 4 * 256 : 8 * 256;
    case 64: return heads >= 256 ? 256 : 4 * 128;
    case 32: return 128;
    default: return 64;
  }
}

int64_t max_launch_items(const gdn_desc& d) {
  if (d.B == 0 || d.T == 0) return 0;
  const int64_t heads = d.B * d.Hv, D = d.Dk;
  if (d.T == 1) return heads * step_threads_per_head(D);  // the decode kernel (also three-pass)
  // (the separate gated norm splits itself into launches of bounded size)
  int64_t main = 0;
  if (scan_uses_block_form(d)) {
    const int64_t nblk = (d.T + kBlockTokens - 1) / kBlockTokens;
    const int64_t prep = (d.B * d.Hk * nblk + 3) / 4 * 256;  // a wave per (batch, key head, block)
    main = scan_uses_key_products(d) ? heads * (D / 16) * (D / 32 + 4) * 64  // rows_la_kernel
                                     : heads * 4 * D;                        // state_kernel
    if (prep > main) main = prep;
  } else {
    main = heads * scan_threads_per_head(D, heads);
  }
  return main;
}

int check_desc(const gdn_desc* d) {
  g_last_error[0] = '\0';
  if (!d) return fail(GDN_EINVAL, "null descriptor");
  if (d->B < 0 || d->T < 0) return fail(GDN_ESHAPE, "negative B (%lld) or T (%lld)",
                                        (long long)d->B, (long long)d->T);
  if (d->Hk <= 0 || d->Hv <= 0 || d->Dk <= 0 || d->Dv <= 0)
    return fail(GDN_ESHAPE, "Hk, Hv, Dk, Dv must be positive (got %lld, %lld, %lld, %lld)",
                (long long)d->Hk, (long long)d->Hv, (long long)d->Dk, (long long)d->Dv);
  if (d->Hv % d->Hk)
    return fail(GDN_EGROUP, "Hv (%lld) is not a multiple of Hk (%lld)", (long long)d->Hv,
                (long long)d->Hk);
  if (d->dtype < GDN_F32 || d->dtype > GDN_BF16) return fail(GDN_EDTYPE, "bad dtype %d", d->dtype);
  if (d->gate_dtype < GDN_F32 || d->gate_dtype > GDN_BF16)
    return fail(GDN_EDTYPE, "bad gate_dtype %d", d->gate_dtype);
  if (d->head_major != 0 && d->head_major != 1)
    return fail(GDN_EINVAL, "head_major must be 0 or 1 (got %d)", d->head_major);
  if (d->flags & ~(GDN_FOLD_QK_L2NORM | GDN_FOLD_Q_SCALE | GDN_SCAN_PER_TOKEN | GDN_SCAN_BLOCK |
                   GDN_SCAN_EXACT))
    return fail(GDN_EINVAL, "unknown flag bits 0x%x", d->flags);
  if ((d->flags & GDN_SCAN_PER_TOKEN) && (d->flags & GDN_SCAN_BLOCK))
    return fail(GDN_EINVAL, "GDN_SCAN_PER_TOKEN and GDN_SCAN_BLOCK exclude each other");
  if (!(d->qk_eps >= 0.0f && d->qk_eps < 1e30f) || !(d->norm_eps >= 0.0f && d->norm_eps < 1e30f))
    return fail(GDN_EINVAL, "eps must be finite and >= 0");
  if (d->Dk != d->Dv)
    return fail(GDN_EUNSUPPORTED, "kernels need Dk == Dv (got %lld, %lld)", (long long)d->Dk,
                (long long)d->Dv);
  if (d->Dk != 16 && d->Dk != 32 && d->Dk != 64 && d->Dk != 128 && d->Dk != 256)
    return fail(GDN_EUNSUPPORTED, "head dim %lld not in {16, 32, 64, 128, 256}",
                (long long)d->Dk);
  if ((d->flags & GDN_SCAN_BLOCK) && !block_form_fits(*d))
    return fail(GDN_EUNSUPPORTED,
                block_head_dims_fit(*d)
                    ? "the block form needs Hk*Dk and Hv*Dv below 2^27 and T below 2^29"
                    : "the block form needs Dk == Dv in {32, 64, 128, 256}");

  // sizes (with overflow checks)
  int64_t bt, nqk, nv, ng, ns, tmp;
  if (!mul_ok(d->B, d->T, &bt) || !mul_ok(bt, d->Hk, &tmp) || !mul_ok(tmp, d->Dk, &nqk) ||
      !mul_ok(bt, d->Hv, &ng) || !mul_ok(ng, d->Dv, &nv) || !mul_ok(d->B, d->Hv, &tmp) ||
      !mul_ok(tmp, d->Dv * d->Dk, &ns) || nv > (INT64_MAX / 8) || ns > (INT64_MAX / 8) ||
      nqk > (INT64_MAX / 8))
    return fail(GDN_ESHAPE, "operand sizes overflow");
  if (ng >= (int64_t)1 << 31 || nv >= (int64_t)1 << 40)
    return fail(GDN_ESHAPE, "B*T*Hv (%lld) too large for the launch grid", (long long)ng);
  const int64_t items = max_launch_items(*d);
  if (items > kMaxLaunchItems)
    return fail(GDN_ESHAPE, "the shape needs a launch of %lld work-items (at most 2^32 - 1)",
                (long long)items);
  return GDN_OK;
}

bool block_head_dims_fit(const gdn_desc& d) {
  return d.Dv == d.Dk && (d.Dk == 32 || d.Dk == 64 || d.Dk == 128 || d.Dk == 256);
}

// The block-form kernels address the rows of a 16-token block from the
// block's 64-bit base with 32-bit per-lane offsets: up to 15 token strides of
// Hk*Dk or Hv*Dv elements, or (head-major gates) 3 time strides of T.  Shapes
// past these bounds take the per-token form, whose offsets are all 64-bit.
bool block_form_fits(const gdn_desc& d) {
  const int64_t lim = (int64_t)1 << 27;  // 16 * H * D < 2^31
  return block_head_dims_fit(d) && d.Hk < lim / d.Dk && d.Hv < lim / d.Dv &&
         d.T < ((int64_t)1 << 29);
}

bool scan_uses_block_form(const gdn_desc& d) {
  return block_form_fits(d) && (d.flags & GDN_SCAN_PER_TOKEN) == 0 && d.T >= 2 && d.B > 0;
}

bool scan_uses_key_products(const gdn_desc& d) { return d.B * d.Hv < kManyHeads || d.Dk > 128; }

int64_t scan_record_bytes(const gdn_desc& d) {
  if (!scan_uses_block_form(d)) return 0;
  const int64_t nblk = (d.T + kBlockTokens - 1) / kBlockTokens;
  return d.B * d.Hv * nblk * kBlockRecordBytes;
}

int64_t scan_workspace_bytes(const gdn_desc& d) {
  if (!scan_uses_block_form(d)) return 0;
  const int64_t nblk = (d.T + kBlockTokens - 1) / kBlockTokens;
  int64_t bytes = scan_record_bytes(d);
  if (scan_uses_key_products(d)) bytes += d.B * d.Hk * nblk * kKeyCrossBytes;
  return bytes;
}

int check(const gdn_desc* d, const void* q, const void* k, const void* v, const void* log_decay,
          const void* beta, const float* s0, const void* z, const void* w, const float* y,
          const float* s_out, const void* workspace, uint64_t workspace_bytes) {
  const int rc = check_desc(d);
  if (rc != GDN_OK) return rc;

  // sizes in bytes (check_desc has ruled out overflow)
  const int64_t bt = d->B * d->T, nqk = bt * d->Hk * d->Dk, ng = bt * d->Hv, nv = ng * d->Dv;
  const int64_t ns = d->B * d->Hv * d->Dv * d->Dk;
  const int64_t es = elem_size(d->dtype), ges = elem_size(d->gate_dtype);
  const bool has_tokens = bt > 0;
  const bool has_state = d->B > 0;
  if (has_tokens && (z == nullptr) != (w == nullptr))
    return fail(GDN_EINVAL, "z and w must be given together");
  if (has_tokens && (!q || !k || !v || !log_decay || !beta || !y))
    return fail(GDN_EINVAL, "null operand pointer");
  if (has_state && (!s0 || !s_out)) return fail(GDN_EINVAL, "null state pointer");

  auto al = [](const void* p, uintptr_t a) { return p == nullptr || (uintptr_t)p % a == 0; };
  if (!al(q, 16) || !al(k, 16) || !al(v, 16) || !al(z, 16) || !al(y, 16) || !al(s0, 16) ||
      !al(s_out, 16))
    return fail(GDN_EALIGN, "q, k, v, z, y, s0, s_out must be 16-byte aligned");
  if (!al(log_decay, (uintptr_t)ges) || !al(beta, (uintptr_t)ges) || !al(w, (uintptr_t)es))
    return fail(GDN_EALIGN, "log_decay, beta, w must be aligned to their element size");

  auto rng = [](const char* n, const void* p, int64_t bytes) {
    return Range{n, (uintptr_t)p, p ? (uintptr_t)p + (uintptr_t)bytes : (uintptr_t)p};
  };
  const Range ins[] = {rng("q", q, nqk * es),          rng("k", k, nqk * es),
                       rng("v", v, nv * es),           rng("z", z, z ? nv * es : 0),
                       rng("w", w, w ? d->Dv * es : 0), rng("log_decay", log_decay, ng * ges),
                       rng("beta", beta, ng * ges)};
  const Range ry = rng("y", y, nv * 4);
  const Range rs0 = rng("s0", s0, ns * 4);
  const Range rso = rng("s_out", s_out, ns * 4);
  for (const Range& r : ins) {
    if (overlap(ry, r)) return fail(GDN_EALIAS, "y overlaps %s", r.name);
    if (overlap(rso, r)) return fail(GDN_EALIAS, "s_out overlaps %s", r.name);
  }
  if (overlap(ry, rs0)) return fail(GDN_EALIAS, "y overlaps s0");
  if (overlap(ry, rso)) return fail(GDN_EALIAS, "y overlaps s_out");
  if (overlap(rso, rs0) && rso.lo != rs0.lo)
    return fail(GDN_EALIAS, "s_out partially overlaps s0 (only s_out == s0 is allowed)");

  // the block form's workspace
  const int64_t need = scan_workspace_bytes(*d);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < (uint64_t)need)
      return fail(GDN_EWORKSPACE,
                  "gdn_scan needs %lld bytes of workspace for this shape (got %llu%s)",
                  (long long)need, (unsigned long long)workspace_bytes,
                  workspace ? "" : ", NULL");
    if ((uintptr_t)workspace % kWorkspaceAlign)
      return fail(GDN_EALIGN, "workspace must be %d-byte aligned", (int)kWorkspaceAlign);
    const Range rws = rng("workspace", workspace, need);
    for (const Range& r : ins)
      if (overlap(rws, r)) return fail(GDN_EALIAS, "workspace overlaps %s", r.name);
    for (const Range* r : {&ry, &rs0, &rso})
      if (overlap(rws, *r)) return fail(GDN_EALIAS, "workspace overlaps %s", r->name);
  }
  return GDN_OK;
}

int check_gates(int64_t n, const void* a, const void* b, int32_t in_dtype, float decay_scale,
                const void* log_decay, const void* beta, int32_t out_dtype) {
  g_last_error[0] = '\0';
  if (n < 0) return fail(GDN_ESHAPE, "negative element count %lld", (long long)n);
  // four elements per thread: n / 4 work-items in one launch
  if (n >= (int64_t)1 << 33) return fail(GDN_ESHAPE, "element count too large (at most 2^33 - 1)");
  if (in_dtype < GDN_F32 || in_dtype > GDN_BF16 || out_dtype < GDN_F32 || out_dtype > GDN_BF16)
    return fail(GDN_EDTYPE, "bad dtype (in %d, out %d)", in_dtype, out_dtype);
  if (!(decay_scale >= 0.0f && decay_scale < 1e30f))
    return fail(GDN_EINVAL, "decay_scale must be finite and >= 0");
  if (n == 0) return GDN_OK;
  if (!a || !b || !log_decay || !beta) return fail(GDN_EINVAL, "null pointer");
  const int64_t ies = elem_size(in_dtype), oes = elem_size(out_dtype);
  auto al = [](const void* p, int64_t e) { return (uintptr_t)p % (uintptr_t)e == 0; };
  if (!al(a, ies) || !al(b, ies) || !al(log_decay, oes) || !al(beta, oes))
    return fail(GDN_EALIGN, "pointers must be aligned to their element size");
  auto rng = [](const char* nm, const void* p, int64_t bytes) {
    return Range{nm, (uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes};
  };
  const Range ra = rng("a", a, n * ies), rb = rng("b", b, n * ies);
  const Range rl = rng("log_decay", log_decay, n * oes), rB = rng("beta", beta, n * oes);
  if (overlap(rl, rB)) return fail(GDN_EALIAS, "log_decay overlaps beta");
  for (const Range* in : {&ra, &rb}) {
    if (overlap(rl, *in)) return fail(GDN_EALIAS, "log_decay overlaps %s", in->name);
    if (overlap(rB, *in)) return fail(GDN_EALIAS, "beta overlaps %s", in->name);
  }
  return GDN_OK;
}

int check_conv(int64_t B, int64_t T, int64_t C, int32_t W, int32_t dtype, int32_t apply_silu,
               const void* x, const void* w, const void* bias, const void* state_in,
               const void* y, const void* state_out) {
  g_last_error[0] = '\0';
  if (B < 0 || T < 0 || C < 0) return fail(GDN_ESHAPE, "negative extent");
  if (W < 1 || W > 8) return fail(GDN_EUNSUPPORTED, "conv width %d not in [1, 8]", (int)W);
  if (dtype < GDN_F32 || dtype > GDN_BF16) return fail(GDN_EDTYPE, "bad dtype %d", (int)dtype);
  if (apply_silu != 0 && apply_silu != 1) return fail(GDN_EINVAL, "apply_silu must be 0 or 1");
  const int64_t es = elem_size(dtype), K = W - 1;
  int64_t nx = 0, nst = 0, nw = 0;
  if (!mul_ok(B, T, &nx) || !mul_ok(nx, C, &nx) || !mul_ok(nx, es, &nx) || nx >= ((int64_t)1 << 46))
    return fail(GDN_ESHAPE, "x too large");
  if (!mul_ok(B, C, &nst) || !mul_ok(nst, K, &nst) || !mul_ok(nst, es, &nst) ||
      !mul_ok(C, (int64_t)W * es, &nw))
    return fail(GDN_ESHAPE, "sizes overflow");
  int64_t nblk = 0;  // workgroups along (batch, 16-token tiles)
  // one launch: a thread per channel (or four) across, (batch, tile) pairs down
  if (!mul_ok(B, T > 0 ? (T + 15) / 16 : 1, &nblk) || nblk >= ((int64_t)1 << 31) ||
      C >= ((int64_t)1 << 31))
    return fail(GDN_ESHAPE, "grid too large (B * ceil(T / 16) and C below 2^31)");
  if (B == 0 || C == 0) return GDN_OK;
  if (!w) return fail(GDN_EINVAL, "null weight");
  if (T > 0 && (!x || !y)) return fail(GDN_EINVAL, "null x or y");
  auto al = [es](const void* p) { return (uintptr_t)p % (uintptr_t)es == 0; };
  for (const void* p : {x, w, bias, state_in, y, state_out})
    if (p && !al(p)) return fail(GDN_EALIGN, "pointers must be aligned to their element size");
  auto rng = [](const char* nm, const void* p, int64_t bytes) {
    return Range{nm, (uintptr_t)p, (uintptr_t)p + (uintptr_t)(p ? bytes : 0)};
  };
  const Range rx = rng("x", x, nx), rw = rng("weight", w, nw), rb = rng("bias", bias, C * es);
  const Range rsi = rng("state_in", state_in, nst), ry = rng("y", y, nx);
  const Range rso = rng("state_out", state_out, nst);
  for (const Range* in : {&rx, &rw, &rb, &rsi, &rso})
    if (overlap(ry, *in)) return fail(GDN_EALIAS, "y overlaps %s", in->name);
  for (const Range* in : {&rx, &rw, &rb})
    if (overlap(rso, *in)) return fail(GDN_EALIAS, "state_out overlaps %s", in->name);
  if (state_out != state_in && overlap(rso, rsi))
    return fail(GDN_EALIAS, "state_out partially overlaps state_in");
  return GDN_OK;
}

}  // namespace gdn

extern "C" {

int gdn_check(const gdn_desc* d, const void* q, const void* k, const void* v,
              const void* log_decay, const void* beta, const float* s0, const void* z,
              const void* w, const float* y, const float* s_out, const void* workspace,
              uint64_t workspace_bytes) {
  return gdn::check(d, q, k, v, log_decay, beta, s0, z, w, y, s_out, workspace,
                    workspace_bytes);
}

int gdn_scan_workspace_size(const gdn_desc* d, uint64_t* bytes) {
  const int rc = gdn::check_desc(d);
  if (rc != GDN_OK) return rc;
  if (!bytes) return fail(GDN_EINVAL, "null size pointer");
  *bytes = (uint64_t)gdn::scan_workspace_bytes(*d);
  return GDN_OK;
}

const char* gdn_last_error(void) { return g_last_error; }

const char* gdn_status_str(int status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_EINVAL: return "GDN_EINVAL";
    case GDN_ESHAPE: return "GDN_ESHAPE";
    case GDN_EDTYPE: return "GDN_EDTYPE";
    case GDN_EGROUP: return "GDN_EGROUP";
    case GDN_EUNSUPPORTED: return "GDN_EUNSUPPORTED";
    case GDN_EALIGN: return "GDN_EALIGN";
    case GDN_EALIAS: return "GDN_EALIAS";
    case GDN_EDEVICE: return "GDN_EDEVICE";
    case GDN_EWORKSPACE: return "GDN_EWORKSPACE";
    default: return "GDN_UNKNOWN";
  }
}

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

}  // extern "C"

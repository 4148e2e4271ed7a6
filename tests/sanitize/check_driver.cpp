// Runs the C ABI's host-side validation (csrc/gdn_check.cpp: gdn_check,
// gdn_scan_workspace_size, the gate and conv checks, the status names) over
// accepted and rejected arguments, for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer.  The pointers are fake, well-separated addresses
// that the validation never dereferences.  Test infrastructure only; prints
// "check_driver ok" and exits 0 when every status is the expected one.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

int failures = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, gdn_last_error());
    ++failures;
  }
}

const uintptr_t kBase = (uintptr_t)1 << 32, kGap = (uintptr_t)1 << 28;
const void* at(int i) { return reinterpret_cast<const void*>(kBase + i * kGap); }

gdn_desc good() {
  gdn_desc d;
  std::memset(&d, 0, sizeof(d));
  d.B = 2, d.T = 40, d.Hk = 2, d.Hv = 4, d.Dk = 128, d.Dv = 128;
  d.dtype = GDN_BF16, d.gate_dtype = GDN_BF16, d.flags = 3, d.qk_eps = 1e-6f, d.norm_eps = 1e-6f;
  return d;
}

struct Ptrs {
  const void *q = at(0), *k = at(1), *v = at(2), *g = at(3), *b = at(4), *z = at(6), *w = at(7);
  const float *s0 = (const float*)at(5), *y = (const float*)at(8), *so = (const float*)at(9);
  const void* ws = at(10);
};

int run(const gdn_desc* d, const Ptrs& p, uint64_t ws_bytes) {
  return gdn_check(d, p.q, p.k, p.v, p.g, p.b, p.s0, p.z, p.w, p.y, p.so, p.ws, ws_bytes);
}

}  // namespace

int main() {
  const uint64_t kWs = 1 << 20;
  Ptrs p;
  gdn_desc d = good();
  expect(run(&d, p, kWs), GDN_OK, "valid");
  expect(gdn_check(nullptr, p.q, p.k, p.v, p.g, p.b, p.s0, p.z, p.w, p.y, p.so, p.ws, kWs),
         GDN_EINVAL, "null descriptor");
  uint64_t need = 0;
  expect(gdn_scan_workspace_size(&d, &need), GDN_OK, "size query");
  expect(need == 2 * 4 * 3 * 2560 + 2 * 2 * 3 * 3072 ? GDN_OK : -1, GDN_OK, "size value");
  expect(gdn_scan_workspace_size(&d, nullptr), GDN_EINVAL, "size query without output");
  expect(run(&d, p, need - 1), GDN_EWORKSPACE, "short workspace");
  {
    Ptrs q = p;
    q.ws = nullptr;
    expect(run(&d, q, kWs), GDN_EWORKSPACE, "missing workspace");
    q.ws = (const char*)p.ws + 8;
    expect(run(&d, q, kWs), GDN_EALIGN, "misaligned workspace");
    q.ws = p.v;
    expect(run(&d, q, kWs), GDN_EALIAS, "workspace over v");
  }
  struct Field {
    int64_t gdn_desc::*f;
    int64_t value;
    int want;
    const char* what;
  } fields[] = {{&gdn_desc::Hv, 3, GDN_EGROUP, "Hv not a multiple"},
                {&gdn_desc::Hk, 0, GDN_ESHAPE, "Hk zero"},
                {&gdn_desc::B, -1, GDN_ESHAPE, "B negative"},
                {&gdn_desc::T, -5, GDN_ESHAPE, "T negative"},
                {&gdn_desc::Dk, 48, GDN_EUNSUPPORTED, "Dk != Dv"},
                {&gdn_desc::B, (int64_t)1 << 40, GDN_ESHAPE, "huge B"},
                {&gdn_desc::T, INT64_MAX, GDN_ESHAPE, "T overflows"},
                {&gdn_desc::Hv, INT64_MAX - 1, GDN_ESHAPE, "Hv overflows"}};
  for (const Field& f : fields) {
    gdn_desc e = good();
    e.*(f.f) = f.value;
    if (f.f == &gdn_desc::Hv && f.value > 3) e.Hk = 1;
    expect(run(&e, p, kWs), f.want, f.what);
    uint64_t n = 0;
    expect(gdn_scan_workspace_size(&e, &n), f.want, f.what);
  }
  {
    gdn_desc e = good();
    e.Dk = e.Dv = 512;
    expect(run(&e, p, kWs), GDN_EUNSUPPORTED, "head dim 512");
    e = good();
    e.dtype = 7;
    expect(run(&e, p, kWs), GDN_EDTYPE, "dtype");
    e = good();
    e.flags = 3 | GDN_SCAN_PER_TOKEN | GDN_SCAN_BLOCK;
    expect(run(&e, p, kWs), GDN_EINVAL, "both forms");
    e = good();
    e.qk_eps = -1.0f;
    expect(run(&e, p, kWs), GDN_EINVAL, "eps");
    e = good();
    e.Dk = e.Dv = 16;
    e.dtype = e.gate_dtype = GDN_F32;
    expect(run(&e, p, 0), GDN_OK, "per-token form needs no workspace");
    e.flags = 3 | GDN_SCAN_BLOCK;
    expect(run(&e, p, kWs), GDN_EUNSUPPORTED, "block form at D = 16");
    e = good();
    e.T = 0;
    expect(run(&e, p, 0), GDN_OK, "empty time axis");
  }
  {
    Ptrs q = p;
    q.v = (const char*)p.v + 8;
    expect(run(&d, q, kWs), GDN_EALIGN, "misaligned v");
    q = p;
    q.y = (const float*)p.v;
    expect(run(&d, q, kWs), GDN_EALIAS, "y over v");
    q = p;
    q.so = p.s0 + 64;
    expect(run(&d, q, kWs), GDN_EALIAS, "partial state overlap");
    q = p;
    q.so = p.s0;
    expect(run(&d, q, kWs), GDN_OK, "in-place state");
    q = p;
    q.w = nullptr;
    expect(run(&d, q, kWs), GDN_EINVAL, "z without w");
    q = p;
    q.q = nullptr;
    expect(run(&d, q, kWs), GDN_EINVAL, "null q");
  }
  // gate and conv validation
  expect(gdn::check_gates(16, at(0), at(1), GDN_BF16, 1.0f, at(2), at(3), GDN_F32), GDN_OK,
         "gates");
  expect(gdn::check_gates(-1, at(0), at(1), GDN_BF16, 1.0f, at(2), at(3), GDN_F32), GDN_ESHAPE,
         "gates n");
  expect(gdn::check_gates(16, at(0), at(1), GDN_BF16, 1.0f, (const char*)at(0) + 8, at(3),
                          GDN_F32),
         GDN_EALIAS, "gates overlap");
  expect(gdn::check_conv(2, 4, 8, 4, GDN_BF16, 1, at(0), at(1), at(2), at(3), at(4), at(5)),
         GDN_OK, "conv");
  expect(gdn::check_conv(2, 4, 8, 9, GDN_BF16, 1, at(0), at(1), at(2), at(3), at(4), at(5)),
         GDN_EUNSUPPORTED, "conv width");
  expect(gdn::check_conv((int64_t)1 << 40, (int64_t)1 << 20, 8, 4, GDN_BF16, 1, at(0), at(1),
                         at(2), at(3), at(4), at(5)),
         GDN_ESHAPE, "conv overflow");
  expect(gdn::check_conv(2, 4, 8, 4, GDN_BF16, 1, at(0), at(1), at(2), at(3),
                         (const char*)at(0) + 16, at(5)),
         GDN_EALIAS, "conv y over x");
  for (int s = -1; s <= 10; ++s)
    if (gdn_status_str(s) == nullptr || gdn_status_str(s)[0] == '\0') ++failures;
  if (gdn_abi_version() != GDN_ABI_VERSION) ++failures;
  if (failures) return 1;
  std::printf("check_driver ok\n");
  return 0;
}

// A caller of libgdn_hip.so through its C ABI alone: no Python, no torch.  It
// owns every buffer (hipMalloc), sizes the block form's workspace with
// gdn_scan_workspace_size, runs one gated scan over T tokens on its own
// stream, then one decode step on the next token that updates the scan's
// final state in place, and checks that a bad descriptor is refused with a
// reason.  Operands come from a fixed xorshift generator (bf16, rounded to
// nearest even; gates as the workloads draw them, from uniform variates);
// inputs and outputs go to one file for tests/test_gpu_c_abi.py to compare
// with the float64 oracle.
//
// Built as a shared library with one entry point, gdn_demo_run(out_file),
// returning 0 on success; the test calls it in its own process, so no new
// program is started from a process that already uses the GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gdn.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;

float uniform() {  // xorshift64 -> [-1, 1)
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return (float)((double)(g_state >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0);
}

uint16_t to_bf16(float x) {  // round to nearest even (finite x)
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

std::vector<uint16_t> draw(size_t n, float scale, float shift) {
  std::vector<uint16_t> h(n);
  for (auto& x : h) x = to_bf16(shift + scale * uniform());
  return h;
}

std::vector<uint16_t> draw_log_decay(size_t n) {  // -softplus(u)
  std::vector<uint16_t> h(n);
  for (auto& x : h) x = to_bf16(-std::log1p(std::exp(2.f * uniform())));
  return h;
}

std::vector<uint16_t> draw_beta(size_t n) {  // sigmoid(u)
  std::vector<uint16_t> h(n);
  for (auto& x : h) x = to_bf16(1.f / (1.f + std::exp(-2.f * uniform())));
  return h;
}

bool ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

// Device buffers and the stream, released on every way out of the run.
struct Owned {
  std::vector<void*> bufs;
  hipStream_t stream = nullptr;
  ~Owned() {
    for (void* p : bufs) (void)hipFree(p);
    if (stream) (void)hipStreamDestroy(stream);
  }
  template <typename X>
  X* alloc(size_t n) {
    X* p = nullptr;
    if (!ok(hipMalloc(&p, n * sizeof(X)), "hipMalloc")) return nullptr;
    bufs.push_back(p);
    return p;
  }
  template <typename X>
  X* to_device(const std::vector<X>& h) {
    X* p = alloc<X>(h.size());
    if (p && !ok(hipMemcpy(p, h.data(), h.size() * sizeof(X), hipMemcpyHostToDevice), "hipMemcpy"))
      return nullptr;
    return p;
  }
};

template <typename X>
bool to_host(std::vector<X>& h, const X* p) {
  return ok(hipMemcpy(h.data(), p, h.size() * sizeof(X), hipMemcpyDeviceToHost), "hipMemcpy");
}

template <typename X>
void put(FILE* f, const std::vector<X>& h) {
  std::fwrite(h.data(), sizeof(X), h.size(), f);
}

}  // namespace

extern "C" int gdn_demo_run(const char* out_file) {
  if (!out_file) return 2;
  if (gdn_abi_version() != GDN_ABI_VERSION) {
    std::fprintf(stderr, "ABI version %d, header %d\n", gdn_abi_version(), GDN_ABI_VERSION);
    return 1;
  }
  // few heads at D = 64: the block form's row kernel and its separate norm
  const int64_t B = 2, T = 37, Hk = 2, Hv = 4, D = 64;
  const gdn_desc d = {B, T, Hk, Hv, D, D, 0, GDN_BF16, GDN_BF16,
                      GDN_FOLD_QK_L2NORM | GDN_FOLD_Q_SCALE, 1e-6f, 1e-6f};
  gdn_desc d1 = d;
  d1.T = 1;
  const size_t nqk = B * T * Hk * D, nv = B * T * Hv * D, ng = B * T * Hv, ns = B * Hv * D * D;
  const size_t nqk1 = B * Hk * D, nv1 = B * Hv * D, ng1 = B * Hv;

  // the scan's tokens, then the decode step's token
  const auto q = draw(nqk, 1.f, 0.f), k = draw(nqk, 1.f, 0.f), v = draw(nv, 1.f, 0.f),
             z = draw(nv, 1.f, 0.f), g = draw_log_decay(ng), be = draw_beta(ng);
  const auto q1 = draw(nqk1, 1.f, 0.f), k1 = draw(nqk1, 1.f, 0.f), v1 = draw(nv1, 1.f, 0.f),
             z1 = draw(nv1, 1.f, 0.f), g1 = draw_log_decay(ng1), be1 = draw_beta(ng1);
  const auto w = draw(D, 0.1f, 1.f);
  std::vector<float> s0(ns);
  for (auto& x : s0) x = 0.02f * uniform();

  Owned own;
  const uint16_t *dq = own.to_device(q), *dk = own.to_device(k), *dv = own.to_device(v),
                 *dz = own.to_device(z), *dg = own.to_device(g), *db = own.to_device(be),
                 *dq1 = own.to_device(q1), *dk1 = own.to_device(k1), *dv1 = own.to_device(v1),
                 *dz1 = own.to_device(z1), *dg1 = own.to_device(g1), *db1 = own.to_device(be1),
                 *dw = own.to_device(w);
  const float* ds0 = own.to_device(s0);
  float *dy = own.alloc<float>(nv), *dy1 = own.alloc<float>(nv1), *ds = own.alloc<float>(ns);
  if (!dq || !dk || !dv || !dz || !dg || !db || !dq1 || !dk1 || !dv1 || !dz1 || !dg1 || !db1 ||
      !dw || !ds0 || !dy || !dy1 || !ds)
    return 1;
  uint64_t ws_bytes = 0;
  int rc = gdn_scan_workspace_size(&d, &ws_bytes);
  if (rc != GDN_OK || ws_bytes == 0) {
    std::fprintf(stderr, "workspace size: %s (%llu bytes)\n", gdn_last_error(),
                 (unsigned long long)ws_bytes);
    return 1;
  }
  void* ws = own.alloc<unsigned char>(ws_bytes);
  if (!ws || !ok(hipStreamCreate(&own.stream), "hipStreamCreate")) return 1;
  hipStream_t st = own.stream;

  // a refused call: a value-head count that is not a multiple of the key heads
  gdn_desc bad = d;
  bad.Hv = 3;
  rc = gdn_scan(&bad, dq, dk, dv, dg, db, ds0, dz, dw, dy, ds, ws, ws_bytes, st);
  if (rc != GDN_EGROUP || std::strlen(gdn_last_error()) == 0) {
    std::fprintf(stderr, "bad descriptor: got %s\n", gdn_status_str(rc));
    return 1;
  }

  rc = gdn_scan(&d, dq, dk, dv, dg, db, ds0, dz, dw, dy, ds, ws, ws_bytes, st);
  if (rc != GDN_OK) {
    std::fprintf(stderr, "gdn_scan: %s: %s\n", gdn_status_str(rc), gdn_last_error());
    return 1;
  }
  std::vector<float> y(nv), s_scan(ns), y1(nv1), s_step(ns);
  if (!ok(hipStreamSynchronize(st), "hipStreamSynchronize") || !to_host(y, dy) ||
      !to_host(s_scan, ds))
    return 1;
  rc = gdn_recurrent_step(&d1, dq1, dk1, dv1, dg1, db1, ds, dz1, dw, dy1, ds, st);  // in place
  if (rc != GDN_OK) {
    std::fprintf(stderr, "gdn_recurrent_step: %s: %s\n", gdn_status_str(rc), gdn_last_error());
    return 1;
  }
  if (!ok(hipStreamSynchronize(st), "hipStreamSynchronize") || !to_host(y1, dy1) ||
      !to_host(s_step, ds))
    return 1;

  FILE* f = std::fopen(out_file, "wb");
  if (!f) {
    std::perror(out_file);
    return 1;
  }
  const int64_t dims[5] = {B, T, Hk, Hv, D};
  std::fwrite(dims, sizeof(int64_t), 5, f);
  put(f, q), put(f, k), put(f, v), put(f, z), put(f, g), put(f, be), put(f, w), put(f, s0);
  put(f, q1), put(f, k1), put(f, v1), put(f, z1), put(f, g1), put(f, be1);
  put(f, y), put(f, s_scan), put(f, y1), put(f, s_step);
  std::fclose(f);

  std::printf("gdn_demo: scan (B=%lld T=%lld Hk=%lld Hv=%lld D=%lld, %llu workspace bytes) and "
              "one decode step done\n",
              (long long)B, (long long)T, (long long)Hk, (long long)Hv, (long long)D,
              (unsigned long long)ws_bytes);
  return 0;
}

// Streaming reference kernels (include/gdn_calib.h): in-place read-modify-write
// and copy of a large buffer with the decode step's access shape, to measure
// the HBM rate an in-place state update can reach on this GPU.
#include <cstdio>

#include "gdn_calib.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

// A workgroup owns TPB * U consecutive 16-byte vectors; lane t takes vectors
// t, t + TPB, ... (coalesced), issues all U loads, then all U stores.
template <int TPB, int U, bool NT, bool RMW>
__global__ __launch_bounds__(TPB) void stream_kernel(const float* src, float* dst, int64_t n4) {
  const int64_t base = (int64_t)blockIdx.x * (TPB * U) + threadIdx.x;
  float4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * TPB;
    if (i < n4) {
      if constexpr (NT) v[u] = nt_load4(src + 4 * i);
      else v[u] = *reinterpret_cast<const float4*>(src + 4 * i);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * TPB;
    if (i < n4) {
      float4 s = v[u];
      if constexpr (RMW) {
        s.x = fmaf(s.x, 1.0000001f, 1e-7f);
        s.y = fmaf(s.y, 1.0000001f, 1e-7f);
        s.z = fmaf(s.z, 1.0000001f, 1e-7f);
        s.w = fmaf(s.w, 1.0000001f, 1e-7f);
      }
      if constexpr (NT) nt_store4(s, dst + 4 * i);
      else *reinterpret_cast<float4*>(dst + 4 * i) = s;
    }
  }
}

// The same through buffer loads and stores with the decode's cache policies
// (nt loads, nt | sc1 stores, gdn_device.h); a workgroup's resources span its
// chunk, so the tail of the last chunk reads zeros and writes nothing.
template <int TPB, int U, bool RMW>
__global__ __launch_bounds__(TPB) void stream_buf_kernel(const float* src, float* dst, int64_t n4) {
  const int64_t c0 = (int64_t)blockIdx.x * (TPB * U);
  const int64_t left = n4 - c0;
  const uint32_t bytes = (uint32_t)((left < TPB * U ? left : TPB * U) * 16);
  const __amdgpu_buffer_rsrc_t rs = stream_rsrc(src + 4 * c0, bytes);
  const __amdgpu_buffer_rsrc_t rd = stream_rsrc(dst + 4 * c0, bytes);
  float4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = buf_load4<kStreamLoad>(rs, 16u * (threadIdx.x + u * TPB));
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float4 s = v[u];
    if constexpr (RMW) {
      s.x = fmaf(s.x, 1.0000001f, 1e-7f);
      s.y = fmaf(s.y, 1.0000001f, 1e-7f);
      s.z = fmaf(s.z, 1.0000001f, 1e-7f);
      s.w = fmaf(s.w, 1.0000001f, 1e-7f);
    }
    buf_store4<kStoreThrough>(s, rd, 16u * (threadIdx.x + u * TPB));
  }
}

// Shader-clock reference: every lane runs eight independent chains of
// dependent FMAs (enough to keep a SIMD's vector unit issuing with one wave
// on it) between two reads of the shader-cycle counter and of the constant
// 100 MHz real-time counter.  The chains start from the first readings and an
// empty asm consumes them before the second, so the loop stays between the
// two (and each pair of readings stays together).  Lanes 0 to 3 of each wave store its cycles, its ticks and the chains'
// sum (vector stores; the sum keeps the arithmetic alive).
__global__ __launch_bounds__(256) void clock_kernel(uint64_t* out, int iters) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  float x[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = (float)(((c0 ^ r0) & 7) + threadIdx.x + c) * 1e-3f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = fmaf(x[c], 0.9999999f, 1e-7f);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) asm volatile("" : : "v"(x[c]));
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) acc += x[c];
  const int lane = threadIdx.x % kWave;
  const int64_t wave = (int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  const uint64_t word[4] = {c1 - c0, r1 - r0, (uint64_t)__float_as_uint(acc), 0};
  if (lane < 4) out[4 * wave + lane] = word[lane];
}

// names in the order of the launch switch below
constexpr const char* kVariantNames[GDN_CALIB_VARIANTS] = {
    "512 threads x 8 vectors, nontemporal",  "256 threads x 8 vectors, nontemporal",
    "512 threads x 16 vectors, nontemporal", "256 threads x 16 vectors, nontemporal",
    "1024 threads x 4 vectors, nontemporal", "256 threads x 4 vectors, nontemporal",
    "512 threads x 8 vectors, ordinary",     "256 threads x 8 vectors, ordinary",
    "512 threads x 16 vectors, ordinary",    "256 threads x 16 vectors, ordinary",
    "1024 threads x 4 vectors, ordinary",    "256 threads x 4 vectors, ordinary",
    "256 threads x 4 vectors, buffer, stores through to device scope",
    "1024 threads x 4 vectors, buffer, stores through to device scope",
    "512 threads x 8 vectors, buffer, stores through to device scope",
};

template <int TPB, int U, bool NT>
void launch_v(bool rmw, const float* src, float* dst, int64_t n4, hipStream_t st) {
  const dim3 grid((unsigned)((n4 + TPB * U - 1) / (TPB * U)));
  if (rmw) stream_kernel<TPB, U, NT, true><<<grid, TPB, 0, st>>>(src, dst, n4);
  else stream_kernel<TPB, U, NT, false><<<grid, TPB, 0, st>>>(src, dst, n4);
}

template <int TPB, int U>
void launch_b(bool rmw, const float* src, float* dst, int64_t n4, hipStream_t st) {
  const dim3 grid((unsigned)((n4 + TPB * U - 1) / (TPB * U)));
  if (rmw) stream_buf_kernel<TPB, U, true><<<grid, TPB, 0, st>>>(src, dst, n4);
  else stream_buf_kernel<TPB, U, false><<<grid, TPB, 0, st>>>(src, dst, n4);
}

}  // namespace
}  // namespace gdn

extern "C" {

int gdn_calib_stream(int32_t op, int32_t variant, const void* src, void* dst, uint64_t bytes,
                     void* stream) {
  using namespace gdn;
  if (op != GDN_CALIB_RMW && op != GDN_CALIB_COPY) {
    set_error("op must be GDN_CALIB_RMW or GDN_CALIB_COPY");
    return GDN_EINVAL;
  }
  if (variant < 0 || variant >= GDN_CALIB_VARIANTS) {
    set_error("variant out of range");
    return GDN_EINVAL;
  }
  // at least four 16-byte vectors per thread: below 2^33 vectors keeps a
  // launch's work-items under the 32-bit grid size of the dispatch packet
  if (bytes % 16 || bytes / 16 >= ((uint64_t)1 << 33)) {
    set_error("bytes must be a multiple of 16 (and below 2^37)");
    return GDN_ESHAPE;
  }
  if (bytes == 0) return GDN_OK;
  if (!src || !dst || (uintptr_t)src % 16 || (uintptr_t)dst % 16) {
    set_error("src and dst must be non-null and 16-byte aligned");
    return src && dst ? GDN_EALIGN : GDN_EINVAL;
  }
  const bool rmw = op == GDN_CALIB_RMW;
  if (rmw && src != dst) {
    set_error("the read-modify-write works in place: src must equal dst");
    return GDN_EINVAL;
  }
  if (!rmw && (uintptr_t)src < (uintptr_t)dst + bytes && (uintptr_t)dst < (uintptr_t)src + bytes) {
    set_error("copy source and destination overlap");
    return GDN_EALIAS;
  }
  const float* s = static_cast<const float*>(src);
  float* d = static_cast<float*>(dst);
  const int64_t n4 = (int64_t)(bytes / 16);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (variant) {
    case 0: launch_v<512, 8, true>(rmw, s, d, n4, st); break;
    case 1: launch_v<256, 8, true>(rmw, s, d, n4, st); break;
    case 2: launch_v<512, 16, true>(rmw, s, d, n4, st); break;
    case 3: launch_v<256, 16, true>(rmw, s, d, n4, st); break;
    case 4: launch_v<1024, 4, true>(rmw, s, d, n4, st); break;
    case 5: launch_v<256, 4, true>(rmw, s, d, n4, st); break;
    case 6: launch_v<512, 8, false>(rmw, s, d, n4, st); break;
    case 7: launch_v<256, 8, false>(rmw, s, d, n4, st); break;
    case 8: launch_v<512, 16, false>(rmw, s, d, n4, st); break;
    case 9: launch_v<256, 16, false>(rmw, s, d, n4, st); break;
    case 10: launch_v<1024, 4, false>(rmw, s, d, n4, st); break;
    case 11: launch_v<256, 4, false>(rmw, s, d, n4, st); break;
    case 12: launch_b<256, 4>(rmw, s, d, n4, st); break;
    case 13: launch_b<1024, 4>(rmw, s, d, n4, st); break;
    default: launch_b<512, 8>(rmw, s, d, n4, st); break;
  }
  return device_status("stream_kernel launch");
}

int gdn_calib_clock(int32_t waves, int32_t iters, uint64_t* out, void* stream) {
  using namespace gdn;
  if (waves < 4 || waves > 8192 || waves % 4) {
    set_error("waves must be a multiple of 4 from 4 to 8192");
    return GDN_ESHAPE;
  }
  if (iters < 1 || iters > (1 << 24)) {
    set_error("iters must be from 1 to 2^24");
    return GDN_ESHAPE;
  }
  if (!out || (uintptr_t)out % 8) {
    set_error("out must be a non-null 8-byte aligned device pointer");
    return out ? GDN_EALIGN : GDN_EINVAL;
  }
  clock_kernel<<<dim3((unsigned)(waves / 4)), 256, 0, static_cast<hipStream_t>(stream)>>>(out,
                                                                                          iters);
  return device_status("clock_kernel launch");
}

const char* gdn_calib_variant_name(int32_t variant) {
  if (variant < 0 || variant >= GDN_CALIB_VARIANTS) return "";
  return gdn::kVariantNames[variant];
}

}  // extern "C"

// Gate producer: both gates of a GDN layer from their pre-activations in one
// launch ("Module gdn" page, QWEN38_KERNELS: the gate kernel computes both
// gates from one launch).  The pages do not give the formulas; these are the
// workloads' own:  log_decay = -decay_scale * softplus(a),  beta = sigmoid(b).
// Elementwise and HBM-bound: each thread handles four consecutive elements.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

template <int OT>
__device__ __forceinline__ void store1(void* p, int64_t i, float x) {
  if constexpr (OT == GDN_F32) {
    static_cast<float*>(p)[i] = x;
  } else if constexpr (OT == GDN_F16) {
    static_cast<_Float16*>(p)[i] = (_Float16)x;
  } else {  // round to nearest even
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    if ((__float_as_uint(x) & 0x7f800000u) == 0x7f800000u) u = __float_as_uint(x);  // inf/nan
    static_cast<uint16_t*>(p)[i] = (uint16_t)(u >> 16);
  }
}

__device__ __forceinline__ float softplus(float x) {
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid(float x) {
  const float e = expf(-fabsf(x));
  return x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

template <int IT, int OT>
__global__ __launch_bounds__(256) void gates_kernel(int64_t n, const void* a, const void* b,
                                                    float decay_scale, void* ld, void* be) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t i = i0 + e;
    if (i < n) {
      store1<OT>(ld, i, -decay_scale * softplus(ld1<IT>(a, i)));
      store1<OT>(be, i, sigmoid(ld1<IT>(b, i)));
    }
  }
}

template <int IT>
void launch_gates_it(int64_t n, const void* a, const void* b, float s, void* ld, void* be,
                     int ot, hipStream_t st) {
  const dim3 grid((unsigned)((n + 1023) / 1024));
  switch (ot) {
    case GDN_F32: gates_kernel<IT, GDN_F32><<<grid, 256, 0, st>>>(n, a, b, s, ld, be); break;
    case GDN_F16: gates_kernel<IT, GDN_F16><<<grid, 256, 0, st>>>(n, a, b, s, ld, be); break;
    default: gates_kernel<IT, GDN_BF16><<<grid, 256, 0, st>>>(n, a, b, s, ld, be); break;
  }
}

}  // namespace

int launch_gates(int64_t n, const void* a, const void* b, int in_dtype, float decay_scale,
                 void* log_decay, void* beta, int out_dtype, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!launch_fits((n + 1023) / 1024, 256, "gates_kernel")) return GDN_ESHAPE;
  switch (in_dtype) {
    case GDN_F32: launch_gates_it<GDN_F32>(n, a, b, decay_scale, log_decay, beta, out_dtype, st); break;
    case GDN_F16: launch_gates_it<GDN_F16>(n, a, b, decay_scale, log_decay, beta, out_dtype, st); break;
    default: launch_gates_it<GDN_BF16>(n, a, b, decay_scale, log_decay, beta, out_dtype, st); break;
  }
  return device_status("gates_kernel launch");
}

}  // namespace gdn

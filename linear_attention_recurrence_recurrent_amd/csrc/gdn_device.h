// Device-side helpers shared by the decode and scan kernels: operand loads
// (compile-time dtype), streaming state accesses, and wave64 lane reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "gdn.h"

namespace gdn {
namespace {

constexpr int kWave = 64;

// ------------------------------------------------------------------ loads

// Compile-time dtype versions for the operand loads of the kernels.  ld4 reads
// four consecutive elements starting at i (i is a multiple of 4 and the base
// pointer is 16-byte aligned, so the access is 16 or 8 bytes aligned).
template <int DT>
__device__ __forceinline__ float ld1(const void* p, int64_t i) {
  if constexpr (DT == GDN_F32) return static_cast<const float*>(p)[i];
  const uint16_t h = static_cast<const uint16_t*>(p)[i];
  if constexpr (DT == GDN_F16) return (float)__builtin_bit_cast(_Float16, h);
  return __uint_as_float((uint32_t)h << 16);
}

template <int DT>
__device__ __forceinline__ float4 ld4(const void* p, int64_t i) {
  if constexpr (DT == GDN_F32) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
  } else {
    const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    if constexpr (DT == GDN_F16) {
      typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
      const half4_t h = __builtin_bit_cast(half4_t, r);
      return make_float4((float)h.x, (float)h.y, (float)h.z, (float)h.w);
    } else {
      return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                         __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
    }
  }
}

__device__ __forceinline__ float dot4(const float4 a, const float4 b, float acc) {
  acc = fmaf(a.x, b.x, acc);
  acc = fmaf(a.y, b.y, acc);
  acc = fmaf(a.z, b.z, acc);
  return fmaf(a.w, b.w, acc);
}

__device__ __forceinline__ float4 scale4(const float4 a, float s) {
  return make_float4(a.x * s, a.y * s, a.z * s, a.w * s);
}

// silu(z) = z * sigmoid(z), from the hardware exp2 and reciprocal (a few ulp;
// z -> -inf gives -0, z -> +inf gives z).
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504f));
}

// Streaming (nontemporal) 16-byte state accesses: the state is touched once per
// decode step, so it should not displace other lines from the caches.
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 nt_load4(const float* p) {
  const v4f r = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(r.x, r.y, r.z, r.w);
}
__device__ __forceinline__ void nt_store4(const float4 s, float* p) {
  const v4f r = {s.x, s.y, s.z, s.w};
  __builtin_nontemporal_store(r, reinterpret_cast<v4f*>(p));
}

// The decode's state stream through buffer loads and stores, whose cache
// policy is an operand: gfx950 bits nt (2, streaming) and sc1 (16, device
// scope, so a store is written through to where every XCD sees it rather
// than left dirty in this XCD's L2).  Loads take nt.  Stores take nt | sc1
// (kStoreThrough) when a step's state traffic exceeds the caches anyway
// (about 2% faster than nt alone at 128 MiB of state), nt alone
// (kStoreStream) for smaller states, which the next step then finds in the
// caches (up to 20% faster there), and no hint (kStoreCached) for states that
// fit in half of the L2s, which then keep them.  A resource spans `bytes`
// from `base` (at most 4 GiB); offsets are in bytes, and accesses outside the
// span read zeros and write nothing.
constexpr int kStreamLoad = 2, kStoreCached = 0, kStoreStream = 2, kStoreThrough = 2 | 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const float* base, uint32_t bytes) {
  // dword 3 = 0x00020000: 32-bit data format, the value raw buffers use on gfx9
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, (int)bytes, 0x00020000);
}
template <int POLICY>
__device__ __forceinline__ float4 buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY);
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                     __uint_as_float(v[3]));
}
template <int POLICY>
__device__ __forceinline__ void buf_store4(const float4 s, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4 v = {__float_as_uint(s.x), __float_as_uint(s.y), __float_as_uint(s.z),
                __float_as_uint(s.w)};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, POLICY);
}

// ------------------------------------------------------------------ lane reductions
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of CL consecutive lanes (CL = 1, 2, 4, ..., 32).
// Butterfly order: every lane of a group ends with bit-identical sums.  The
// step across the two DPP rows of a 32-lane group is gfx950's row swap: with
// both operands x, v_permlane16_swap returns the even row's values in one
// result and the odd row's in the other, in every lane of the pair.
template <int CL>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(CL == 1 || CL == 2 || CL == 4 || CL == 8 || CL == 16 || CL == 32,
                "row group size");
  if constexpr (CL >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (CL >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (CL >= 8) x += dpp<0x141>(x);  // row_half_mirror: the other quad of 8
  if constexpr (CL >= 16) x += dpp<0x140>(x); // row_mirror: the other half of 16
  if constexpr (CL >= 32) {
    const int b = __float_as_int(x);
    const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    x = __int_as_float(p[0]) + __int_as_float(p[1]);
  }
  return x;
}

// Sum over the whole wave, returned in every lane.  The four row sums are read
// out lane by lane, so no cross-row exchange through LDS is needed; the exec
// mask must be full.
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  const int b = __float_as_int(x);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// One multiplicative DPP step: x from the lane selected by CTRL, or 1 where
// that lane lies outside the row or the row is masked off by ROW_MASK.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_one(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), CTRL,
                                                    ROW_MASK, 0xF, false));
}

// Inclusive prefix and suffix products inside each row of 16 lanes
// (Hillis-Steele with row_shr / row_shl 1, 2, 4, 8; exec must be full).
__device__ __forceinline__ float row_prefix_prod(float x) {
  x *= dpp_or_one<0x111, 0xF>(x);
  x *= dpp_or_one<0x112, 0xF>(x);
  x *= dpp_or_one<0x114, 0xF>(x);
  x *= dpp_or_one<0x118, 0xF>(x);
  return x;
}
__device__ __forceinline__ float row_suffix_prod(float x) {
  x *= dpp_or_one<0x101, 0xF>(x);
  x *= dpp_or_one<0x102, 0xF>(x);
  x *= dpp_or_one<0x104, 0xF>(x);
  x *= dpp_or_one<0x108, 0xF>(x);
  return x;
}

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so that each
// XCD receives a contiguous range of tiles (the row blocks of one head, and
// the value heads of one key group, then share an L2).
__device__ __forceinline__ int64_t xcd_tile(int64_t i, int64_t n) {
  if (n % 8) return i;
  return (i % 8) * (n / 8) + i / 8;
}

// is N elements wide, so the element index must be a multiple of N.
template <int DT, int N>
struct Raw {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "Raw holds 1, 2, 4 or 8 elements");
  static constexpr bool kF32 = DT == GDN_F32;
  typedef typename std::conditional<kF32, float, uint32_t>::type Word;
  static constexpr int kWords = kF32 ? N : (N + 1) / 2;
  Word w[kWords];
  __device__ __forceinline__ void load(const void* p, int64_t i) {
    if constexpr (kF32) {
      const float* f = static_cast<const float*>(p) + i;
      if constexpr (N == 8) {
        const float4 t = *reinterpret_cast<const float4*>(f);
        const float4 u = *reinterpret_cast<const float4*>(f + 4);
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
        w[4] = u.x; w[5] = u.y; w[6] = u.z; w[7] = u.w;
      } else if constexpr (N == 4) {
        const float4 t = *reinterpret_cast<const float4*>(f);
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
      } else if constexpr (N == 2) {
        const float2 t = *reinterpret_cast<const float2*>(f);
        w[0] = t.x; w[1] = t.y;
      } else {
        w[0] = f[0];
      }
    } else {
      const uint16_t* h = static_cast<const uint16_t*>(p) + i;
      if constexpr (N == 8) {
        const uint4 t = *reinterpret_cast<const uint4*>(h);
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
      } else if constexpr (N == 4) {
        const uint2 t = *reinterpret_cast<const uint2*>(h);
        w[0] = t.x; w[1] = t.y;
      } else if constexpr (N == 2) {
        w[0] = *reinterpret_cast<const uint32_t*>(h);
      } else {
        w[0] = h[0];
      }
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = 0;
  }
  __device__ __forceinline__ float get(int k) const {
    if constexpr (kF32) {
      return w[k];
    } else if constexpr (DT == GDN_BF16) {
      return __uint_as_float((k & 1) ? (w[k >> 1] & 0xffff0000u) : (w[k >> 1] << 16));
    } else {
      const uint16_t bits = (uint16_t)((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xffffu));
      return (float)__builtin_bit_cast(_Float16, bits);
    }
  }
  __device__ __forceinline__ float4 get4(int c) const {  // elements 4c .. 4c+3
    return make_float4(get(4 * c), get(4 * c + 1), get(4 * c + 2), get(4 * c + 3));
  }
};

}  // namespace
}  // namespace gdn

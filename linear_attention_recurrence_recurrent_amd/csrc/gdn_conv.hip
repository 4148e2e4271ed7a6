// Producer of q, k and v: causal depthwise convolution over the time axis with
// the silu fused in ("Module gdn" page, QWEN38_KERNELS: the convolution
// carries the silu).  The pages give neither the width nor the weight layout;
// the kernel computes the usual causal form, one filter of W taps per channel
// with the last tap on the current token:
//   pre[b,t,c] = bias[c] + sum_{i<W} w[c][i] * xx(b, t-(W-1)+i, c)
//   xx(b,t',c) = x[b][t'][c] for t' >= 0, else the carried context
//                state_in[b][c][(W-1)+t'] (zero without one)
//   y = silu(pre) (or pre), in the operand dtype;
//   state_out[b][c][j] = xx(b, T-(W-1)+j, c), the context of the next call.
// HBM-bound: a thread owns VEC adjacent channels (coalesced along C) and a run
// of TT tokens, keeps the last W-1 inputs in registers as a sliding window and
// issues the loads of BATCH tokens together.  Short runs (16 tokens) give many
// workgroups and so many loads in flight; the W-1 inputs before a run are
// re-read by its neighbour (mostly from L2).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kTT = 16;  // tokens per thread (the launch's token tile)

struct ConvArgs {
  const void *x, *w, *bias, *state_in;
  void *y, *state_out;
  int64_t T, C, ntiles;
};

template <int DT>
__device__ __forceinline__ uint32_t pack16(float x) {
  if constexpr (DT == GDN_F16) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
  } else {  // bfloat16, round to nearest even; Inf and NaN keep their class
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  }
}

template <int DT>
__device__ __forceinline__ void store1(void* p, int64_t i, float x) {
  if constexpr (DT == GDN_F32) static_cast<float*>(p)[i] = x;
  else static_cast<uint16_t*>(p)[i] = (uint16_t)pack16<DT>(x);
}

// VEC consecutive elements starting at i (i a multiple of VEC, base aligned).
template <int DT, int VEC>
__device__ __forceinline__ void storev(void* p, int64_t i, const float (&v)[VEC]) {
  if constexpr (VEC == 1) {
    store1<DT>(p, i, v[0]);
  } else if constexpr (DT == GDN_F32) {
#pragma unroll
    for (int k = 0; k < VEC; k += 4)
      *reinterpret_cast<float4*>(static_cast<float*>(p) + i + k) =
          make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
  } else if constexpr (VEC == 4) {
    const uint2 r = make_uint2(pack16<DT>(v[0]) | (pack16<DT>(v[1]) << 16),
                               pack16<DT>(v[2]) | (pack16<DT>(v[3]) << 16));
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = r;
  } else {
    const uint4 r = make_uint4(pack16<DT>(v[0]) | (pack16<DT>(v[1]) << 16),
                               pack16<DT>(v[2]) | (pack16<DT>(v[3]) << 16),
                               pack16<DT>(v[4]) | (pack16<DT>(v[5]) << 16),
                               pack16<DT>(v[6]) | (pack16<DT>(v[7]) << 16));
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + i) = r;
  }
}

template <int DT, int VEC, int W, bool SILU, int TT = kTT, int BATCH = 8>
__global__ __launch_bounds__(256) void conv_kernel(ConvArgs a) {
  static_assert(VEC == 1 || VEC == 4 || VEC == 8, "channel vector");
  constexpr int K = W - 1, KW = K > 0 ? K : 1;
  const int64_t C = a.C, T = a.T;
  const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * VEC;
  if (c0 >= C) return;  // VEC divides C, so a thread's channels are all in range
  const int64_t tile = blockIdx.y % a.ntiles, b = blockIdx.y / a.ntiles;
  const int64_t t0 = tile * TT, t1 = (t0 + TT < T) ? t0 + TT : T;
  const int64_t xb = b * T * C + c0;  // x[b][0][c0]

  float wk[W][VEC], bs[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
#pragma unroll
    for (int i = 0; i < W; ++i) wk[i][v] = ld1<DT>(a.w, (c0 + v) * W + i);
    bs[v] = a.bias ? ld1<DT>(a.bias, c0 + v) : 0.f;
  }
  // window: inputs t0-K .. t0-1 (the carried context for the first tile)
  float win[KW][VEC];
  if (tile == 0) {
    float st[KW][VEC];
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int v = 0; v < VEC; ++v)
        st[j][v] = a.state_in ? ld1<DT>(a.state_in, (b * C + c0 + v) * K + j) : 0.f;
    // The next call's context.  With one tile per sequence (T <= 16: decode)
    // it is the window after the loop, stored at the end, so no store precedes
    // the loads of x (one vmcnt counts both: a wait for those loads would
    // also wait for the stores).  With more tiles this tile writes it here,
    // before any other tile could need state_in; read before written either
    // way, so the in-place update is safe.
    if (a.state_out && a.ntiles > 1) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int64_t tt = T - K + j;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          float val = 0.f;
          if (tt >= 0) val = ld1<DT>(a.x, xb + tt * C + v);
#pragma unroll
          for (int i = 0; i < K; ++i)
            if (tt < 0 && K + tt == i) val = st[i][v];
          store1<DT>(a.state_out, (b * C + c0 + v) * K + j, val);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int v = 0; v < VEC; ++v) win[j][v] = st[j][v];
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      Raw<DT, VEC> r;
      r.load(a.x, xb + (t0 - K + j) * C);
#pragma unroll
      for (int v = 0; v < VEC; ++v) win[j][v] = r.get(v);
    }
  }

  for (int64_t t = t0; t < t1; t += BATCH) {
    Raw<DT, VEC> r[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (t + u < t1) r[u].load(a.x, xb + (t + u) * C);
      else r[u].zero();
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (t + u < t1) {
        float out[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float xv = r[u].get(v);
          float acc = bs[v];
#pragma unroll
          for (int i = 0; i < K; ++i) acc = fmaf(wk[i][v], win[i][v], acc);
          acc = fmaf(wk[K][v], xv, acc);
          out[v] = SILU ? silu(acc) : acc;
#pragma unroll
          for (int i = 0; i + 1 < K; ++i) win[i][v] = win[i + 1][v];
          if constexpr (K > 0) win[K - 1][v] = xv;
        }
        storev<DT, VEC>(a.y, xb + (t + u) * C, out);
      }
    }
  }
  if (a.state_out && a.ntiles == 1) {  // the last K inputs (or the carried context)
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int v = 0; v < VEC; ++v) store1<DT>(a.state_out, (b * C + c0 + v) * K + j, win[j][v]);
  }
}

template <int DT, int VEC, int W>
void launch_w(const ConvArgs& a, dim3 grid, bool silu, hipStream_t st) {
  if (silu) conv_kernel<DT, VEC, W, true><<<grid, 256, 0, st>>>(a);
  else conv_kernel<DT, VEC, W, false><<<grid, 256, 0, st>>>(a);
}

template <int DT, int VEC>
void launch_vec(const ConvArgs& a, dim3 grid, int W, bool silu, hipStream_t st) {
  switch (W) {
    case 1: launch_w<DT, VEC, 1>(a, grid, silu, st); break;
    case 2: launch_w<DT, VEC, 2>(a, grid, silu, st); break;
    case 3: launch_w<DT, VEC, 3>(a, grid, silu, st); break;
    case 4: launch_w<DT, VEC, 4>(a, grid, silu, st); break;
    case 5: launch_w<DT, VEC, 5>(a, grid, silu, st); break;
    case 6: launch_w<DT, VEC, 6>(a, grid, silu, st); break;
    case 7: launch_w<DT, VEC, 7>(a, grid, silu, st); break;
    default: launch_w<DT, VEC, 8>(a, grid, silu, st); break;
  }
}

template <int DT>
void launch_dt(const ConvArgs& a, dim3 grid, bool vec4, int W, bool silu, hipStream_t st) {
  if (vec4) launch_vec<DT, 4>(a, grid, W, silu, st);
  else launch_vec<DT, 1>(a, grid, W, silu, st);
}

}  // namespace

int launch_conv(int64_t B, int64_t T, int64_t C, int W, int dtype, int apply_silu,
                const void* x, const void* w, const void* bias, const void* state_in, void* y,
                void* state_out, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool vec4 = C % 4 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0;
  const int64_t vec = vec4 ? 4 : 1;
  const int64_t ntiles = T > 0 ? (T + kTT - 1) / kTT : 1;
  const ConvArgs a{x, w, bias, state_in, y, state_out, T, C, ntiles};
  if (!launch_fits((C / vec + 255) / 256, 256, "conv_kernel") ||
      !launch_fits(B * ntiles, 1, "conv_kernel"))
    return GDN_ESHAPE;
  const dim3 grid((unsigned)((C / vec + 255) / 256), (unsigned)(B * ntiles));
  switch (dtype) {
    case GDN_F32: launch_dt<GDN_F32>(a, grid, vec4, W, apply_silu != 0, st); break;
    case GDN_F16: launch_dt<GDN_F16>(a, grid, vec4, W, apply_silu != 0, st); break;
    default: launch_dt<GDN_BF16>(a, grid, vec4, W, apply_silu != 0, st); break;
  }
  return device_status("conv_kernel launch");
}

}  // namespace gdn

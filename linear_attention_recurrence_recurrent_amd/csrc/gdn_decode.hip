// Decode step of the Gated DeltaNet recurrence on MI355X (gfx950).
//
// Recurrence ("Module gdn" page, module description), per value head with a
// D x D float32 memory S (row a = value lane, column c = key lane):
//     u = S.k ;  S = alpha*S + beta*(v - alpha*u) k^T ;  o = S.q (updated S)
//     y = rmsnorm(o * silu(z)) * w        (gate first, then normalise)
// Fused row pass ("Module gdn" page, "The fusion"): because the update is
// affine in S, o[a] = alpha*(S_old.q)[a] + coef[a]*(k.q) with
// coef[a] = beta*(v[a] - alpha*u[a]).  One pass over a state row held in
// registers yields both dots; the row is then rewritten from the same
// registers, so each row is read once and written once per token.
//
// Work layout (wave64): a row of D columns is split over CL consecutive lanes
// (a "row group"); lane j of the group owns the float4 column chunks j, j+CL,
// ...; the two dots are reduced inside the group with DPP butterflies, which
// leave bit-identical sums in every lane, so every lane updates its own
// columns with the same coefficient.  A workgroup owns a whole head: it
// streams the head's rows from HBM with nontemporal 16-byte loads and stores,
// issuing every load of a lane before any arithmetic, and applies the gated
// RMSNorm in the same launch.  The state goes through buffer loads and
// stores with streaming cache policies (stores written through at device
// scope from kWriteThroughBytes of state on, with no hint up to
// kCachedStoreBytes: stream_rsrc in gdn_device.h).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

struct StepArgs {
  const void *q, *k, *v, *ld, *beta, *z, *w;
  const float* s0;
  float* y;
  float* s_out;
  int Hk, Hv, G, dt, gdt;
  uint32_t flags;
  float qk_eps, norm_eps, qscale;
};

template <int DT, int D, int CL, int RPL>
struct HeadRegs {
  static constexpr int NV4 = D / CL / 4;
  Raw<DT, 4> k[NV4], q[NV4];
  float4 S[RPL][NV4];
  Raw<DT, RPL> v, z;  // z and the norm weight w only for the gated output
  float w[RPL];
  float ld, be;
};

// Lane layout of the decode: row group g of a wave owns rows
// (wave*RG + g)*RPL ... +RPL-1; lane j of the group owns float4 chunks j, j+CL, ...
template <int CL, int RPL>
__device__ __forceinline__ int decode_row0() {
  constexpr int RG = kWave / CL;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  return (wave * RG + lane / CL) * RPL;
}

// Issue every load of one head.  The small operands go first: loads complete
// in issue order, so the q/k norms can start while the state is in flight.
template <int DT, int GT, int D, int CL, int RPL, int NW>
__device__ __forceinline__ void decode_fetch(const StepArgs& a, int64_t head,
                                             HeadRegs<DT, D, CL, RPL>& R) {
  constexpr int NV4 = D / CL / 4;
  const int j = threadIdx.x % CL;
  const int row0 = decode_row0<CL, RPL>();
  const int64_t b = head / a.Hv;
  const int hv = (int)(head % a.Hv), hk = hv / a.G;
  R.ld = ld1<GT>(a.ld, head);  // T == 1: gates are [B, Hv] in both layouts
  R.be = ld1<GT>(a.beta, head);
  const int64_t qk = (b * a.Hk + hk) * D;  // T == 1: both layouts coincide
#pragma unroll
  for (int m = 0; m < NV4; ++m) {
    R.k[m].load(a.k, qk + 4 * (m * CL + j));
    R.q[m].load(a.q, qk + 4 * (m * CL + j));
  }
  const __amdgpu_buffer_rsrc_t rs = stream_rsrc(a.s0 + head * (int64_t)(D * D), D * D * 4);
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
#pragma unroll
    for (int m = 0; m < NV4; ++m)
      R.S[r][m] = buf_load4<kStreamLoad>(rs, 4 * ((row0 + r) * D + 4 * (m * CL + j)));
  }
  R.v.load(a.v, head * D + row0);
  if (a.z) {
    R.z.load(a.z, head * D + row0);
    // w in flight with the state, not after the norm's barrier; it is aligned
    // to its element size only, so one element per load
#pragma unroll
    for (int r = 0; r < RPL; ++r) R.w[r] = ld1<DT>(a.w, row0 + r);
  }
}

// Fold the norms, run the fused row pass, write the state back and the
// (gated) output, the state stored with cache policy SP.  The L2 norms and
// the q scale are applied to the reduced dots as scalars (u = rk*(S.k),
// w = rq*(S.q), S += (coef*rk) k), so the normalised vectors are never
// materialised.  red[NW] is this head's slot for
// the cross-wave sum of the gated norm.
template <int DT, int GT, int D, int CL, int RPL, int NW, int SP>
__device__ __forceinline__ void decode_finish(const StepArgs& a, int64_t head,
                                              HeadRegs<DT, D, CL, RPL>& R, float* red) {
  constexpr int NV4 = D / CL / 4;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int j = lane % CL;
  const int row0 = decode_row0<CL, RPL>();

  // the row group covers all D columns: its sums are the full norms and k.q
  float skk = 0.f, sqq = 0.f, skq = 0.f;
#pragma unroll
  for (int m = 0; m < NV4; ++m) {
    const float4 kf = R.k[m].get4(0), qf = R.q[m].get4(0);
    skk = dot4(kf, kf, skk);
    sqq = dot4(qf, qf, sqq);
    skq = dot4(kf, qf, skq);
  }
  skk = group_sum<CL>(skk);
  sqq = group_sum<CL>(sqq);
  skq = group_sum<CL>(skq);
  float rk = 1.f, rq = a.qscale;
  if (a.flags & GDN_FOLD_QK_L2NORM) {
    rk = rsqrtf(skk + a.qk_eps);
    rq *= rsqrtf(sqq + a.qk_eps);
  }
  const float kq = skq * rk * rq;
  const float al = expf(R.ld), be = R.be;

  // both dots of every row from the registers
  float u[RPL], w[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) u[r] = w[r] = 0.f;
#pragma unroll
  for (int m = 0; m < NV4; ++m) {
    const float4 kf = R.k[m].get4(0), qf = R.q[m].get4(0);
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      u[r] = dot4(R.S[r][m], kf, u[r]);
      w[r] = dot4(R.S[r][m], qf, w[r]);
    }
  }
  float o[RPL], ck[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const float ur = group_sum<CL>(u[r]) * rk;
    const float wr = group_sum<CL>(w[r]) * rq;
    const float coef = be * (R.v.get(r) - al * ur);
    o[r] = al * wr + coef * kq;
    ck[r] = coef * rk;  // coefficient of the raw k in the update
  }
  // S = alpha*S + coef*k^, written back from the registers
  const __amdgpu_buffer_rsrc_t ro = stream_rsrc(a.s_out + head * (int64_t)(D * D), D * D * 4);
#pragma unroll
  for (int m = 0; m < NV4; ++m) {
    const float4 kf = R.k[m].get4(0);
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      float4 s = R.S[r][m];
      s.x = fmaf(ck[r], kf.x, al * s.x);
      s.y = fmaf(ck[r], kf.y, al * s.y);
      s.z = fmaf(ck[r], kf.z, al * s.z);
      s.w = fmaf(ck[r], kf.w, al * s.w);
      buf_store4<SP>(s, ro, 4 * ((row0 + r) * D + 4 * (m * CL + j)));
    }
  }

  // output: raw o, or the gated RMSNorm over the whole head
  float* y = a.y + head * D + row0;
  if (a.z != nullptr) {
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      o[r] *= silu(R.z.get(r));
      ss = fmaf(o[r], o[r], ss);
    }
    ss = wave_sum(j == 0 ? ss : 0.f);  // every lane of a group holds the same rows
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) tot += red[i];
    const float inv = rsqrtf(tot * (1.0f / D) + a.norm_eps);
#pragma unroll
    for (int r = 0; r < RPL; ++r) o[r] *= inv * R.w[r];
  }
  if (j == 0) {
    if constexpr (RPL == 4) {
      *reinterpret_cast<float4*>(y) = make_float4(o[0], o[1], o[2], o[3]);
    } else if constexpr (RPL == 2) {
      *reinterpret_cast<float2*>(y) = make_float2(o[0], o[1]);
    } else {
#pragma unroll
      for (int r = 0; r < RPL; ++r) y[r] = o[r];
    }
  }
}

// One workgroup per head (b, hv): every state row of the head is read once
// and written once.  Heads are taken in launch order: for this pure stream
// the plain order spreads the concurrent workgroups' addresses over the HBM
// channels better than grouping contiguous head ranges per XCD (measured).
template <int DT, int GT, int D, int CL, int RPL, int NW, int SP>
__global__ __launch_bounds__(NW* kWave) void decode_kernel(StepArgs a) {
  static_assert((D / CL) % 4 == 0, "a lane owns whole float4 chunks");
  static_assert(NW * (kWave / CL) * RPL == D, "a workgroup owns the whole head");
  __shared__ float red[NW];
  const int64_t head = blockIdx.x;
  HeadRegs<DT, D, CL, RPL> R;
  decode_fetch<DT, GT, D, CL, RPL, NW>(a, head, R);
  decode_finish<DT, GT, D, CL, RPL, NW, SP>(a, head, R, red);
}

// ---------------------------------------------------------------- three-pass form
// The step without the fusion ("Module gdn" page, "The fusion": unfused, the
// state is visited three times), kept to measure what the fusion saves:
//   pass 1: u = S.k^            (reads S; u goes to the y buffer)
//   pass 2: S = alpha*S + beta*(v - alpha*u) k^T   (reads S, writes S)
//   pass 3: o = S.q^ on the updated S, then the gated norm (reads S)
// Each pass is its own launch over the whole state, as separate operators
// with materialised outputs would be.
template <int DT, int GT, int D, int CL, int RPL, int NW, int PASS>
__global__ __launch_bounds__(NW* kWave) void threepass_kernel(StepArgs a) {
  constexpr int NV4 = D / CL / 4;
  __shared__ float red[NW];
  const int64_t head = blockIdx.x;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int j = lane % CL;
  const int row0 = decode_row0<CL, RPL>();
  HeadRegs<DT, D, CL, RPL> R;
  decode_fetch<DT, GT, D, CL, RPL, NW>(a, head, R);
  float skk = 0.f, sqq = 0.f;
#pragma unroll
  for (int m = 0; m < NV4; ++m) {
    const float4 kf = R.k[m].get4(0), qf = R.q[m].get4(0);
    skk = dot4(kf, kf, skk);
    sqq = dot4(qf, qf, sqq);
  }
  skk = group_sum<CL>(skk);
  sqq = group_sum<CL>(sqq);
  float rk = 1.f, rq = a.qscale;
  if (a.flags & GDN_FOLD_QK_L2NORM) {
    rk = rsqrtf(skk + a.qk_eps);
    rq *= rsqrtf(sqq + a.qk_eps);
  }
  float* y = a.y + head * D + row0;
  const __amdgpu_buffer_rsrc_t ro = stream_rsrc(a.s_out + head * (int64_t)(D * D), D * D * 4);
  if constexpr (PASS == 1) {  // u = S.k^
    float u[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < NV4; ++m) acc = dot4(R.S[r][m], R.k[m].get4(0), acc);
      u[r] = group_sum<CL>(acc) * rk;
    }
    if (j == 0) {
#pragma unroll
      for (int r = 0; r < RPL; ++r) y[r] = u[r];
    }
  } else if constexpr (PASS == 2) {  // S = alpha*S + beta*(v - alpha*u) k^
    const float al = expf(R.ld), be = R.be;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const float ck = be * (R.v.get(r) - al * y[r]) * rk;
#pragma unroll
      for (int m = 0; m < NV4; ++m) {
        const float4 kf = R.k[m].get4(0);
        float4 s = R.S[r][m];
        s.x = fmaf(ck, kf.x, al * s.x);
        s.y = fmaf(ck, kf.y, al * s.y);
        s.z = fmaf(ck, kf.z, al * s.z);
        s.w = fmaf(ck, kf.w, al * s.w);
        buf_store4<kStoreThrough>(s, ro, 4 * ((row0 + r) * D + 4 * (m * CL + j)));
      }
    }
  } else {  // o = S.q^ on the updated S, then the output
    float o[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < NV4; ++m) acc = dot4(R.S[r][m], R.q[m].get4(0), acc);
      o[r] = group_sum<CL>(acc) * rq;
    }
    if (a.z != nullptr) {
      float ss = 0.f;
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        o[r] *= silu(R.z.get(r));
        ss = fmaf(o[r], o[r], ss);
      }
      ss = wave_sum(j == 0 ? ss : 0.f);
      if (lane == 0) red[wave] = ss;
      __syncthreads();
      float tot = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) tot += red[i];
      const float inv = rsqrtf(tot * (1.0f / D) + a.norm_eps);
#pragma unroll
      for (int r = 0; r < RPL; ++r) o[r] *= inv * R.w[r];  // fetched with the operands
    }
    if (j == 0) {
#pragma unroll
      for (int r = 0; r < RPL; ++r) y[r] = o[r];
    }
  }
}

}  // namespace

// State stores are written through at device scope from this much state on:
// a step then reads and writes at least the 256 MB Infinity Cache's worth, so
// nothing it leaves in the caches survives to the next step.  Up to
// kCachedStoreBytes (half of the eight XCDs' 4 MB L2s) they carry no hint, so
// the state stays in L2 for the next step; nontemporal in between.
constexpr int64_t kWriteThroughBytes = (int64_t)128 << 20, kCachedStoreBytes = (int64_t)16 << 20;
// Up to this many heads (one workgroup per CU at most) the D = 128 step takes
// the latency shape below.
constexpr int64_t kLatencyBoundHeads = 256;

template <int DT, int GT, int SP>
int launch_step_sp(const gdn_desc& d, const StepArgs& a, hipStream_t st) {
  const int64_t threads = d.Dk >= 128 ? 16 * kWave : d.Dk >= 32 ? 2 * kWave : kWave;
  if (!launch_fits(d.B * d.Hv, threads, "decode_kernel")) return GDN_ESHAPE;
  const dim3 grid((unsigned)(d.B * d.Hv));
  switch (d.Dk) {
    case 256: decode_kernel<DT, GT, 256, 16, 4, 16, SP><<<grid, 16 * kWave, 0, st>>>(a); break;
    // 16 lanes per row (256-byte segments per load).  From 512 heads on, 1024
    // threads at 53 VGPRs: 8 waves per SIMD hold two heads per CU and 2048
    // heads run in four even rounds (8 lanes x 512 threads needed 80 VGPRs:
    // three heads per CU and a ragged last round; 46.6 against 45.3 us per
    // step at B = 64).  Up to 256 heads, at most one workgroup per CU, the step
    // is bound by latency: 512 threads of four rows per lane finish sooner
    // (one barrier across 8 waves instead of 16: 3.83 against 4.09 us at B = 1,
    // 5.6 against 5.8 at B = 8; from 512 heads 1024 threads are faster).
    case 128:
      if (d.B * d.Hv <= kLatencyBoundHeads)
        decode_kernel<DT, GT, 128, 16, 4, 8, SP><<<grid, 8 * kWave, 0, st>>>(a);
      else
        decode_kernel<DT, GT, 128, 16, 2, 16, SP><<<grid, 16 * kWave, 0, st>>>(a);
      break;
    case 64: decode_kernel<DT, GT, 64, 4, 2, 2, SP><<<grid, 2 * kWave, 0, st>>>(a); break;
    case 32: decode_kernel<DT, GT, 32, 4, 1, 2, SP><<<grid, 2 * kWave, 0, st>>>(a); break;
    case 16: decode_kernel<DT, GT, 16, 4, 1, 1, SP><<<grid, 1 * kWave, 0, st>>>(a); break;
    default: set_error("unsupported head dim"); return GDN_EUNSUPPORTED;
  }
  return device_status("decode_kernel launch");
}

template <int DT, int GT>
int launch_step_dt(const gdn_desc& d, const StepArgs& a, hipStream_t st) {
  const int64_t state_bytes = d.B * d.Hv * d.Dv * d.Dk * (int64_t)sizeof(float);
  if (state_bytes >= kWriteThroughBytes) return launch_step_sp<DT, GT, kStoreThrough>(d, a, st);
  if (state_bytes <= kCachedStoreBytes) return launch_step_sp<DT, GT, kStoreCached>(d, a, st);
  return launch_step_sp<DT, GT, kStoreStream>(d, a, st);
}

template <int DT>
int launch_step_gt(const gdn_desc& d, const StepArgs& a, hipStream_t st) {
  switch (d.gate_dtype) {
    case GDN_F32: return launch_step_dt<DT, GDN_F32>(d, a, st);
    case GDN_F16: return launch_step_dt<DT, GDN_F16>(d, a, st);
    default: return launch_step_dt<DT, GDN_BF16>(d, a, st);
  }
}

int launch_step(const gdn_desc& d, const void* q, const void* k, const void* v,
                const void* ld, const void* beta, const float* s0, const void* z, const void* w,
                float* y, float* s_out, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const StepArgs a{q, k, v, ld, beta, z, w, s0, y, s_out, (int)d.Hk, (int)d.Hv,
                   (int)(d.Hv / d.Hk), d.dtype, d.gate_dtype, d.flags, d.qk_eps, d.norm_eps,
                   q_scale(d)};
  switch (d.dtype) {
    case GDN_F32: return launch_step_gt<GDN_F32>(d, a, st);
    case GDN_F16: return launch_step_gt<GDN_F16>(d, a, st);
    default: return launch_step_gt<GDN_BF16>(d, a, st);
  }
}

template <int DT, int GT>
int launch_three_pass_dt(const gdn_desc& d, StepArgs a, hipStream_t st) {
  const dim3 grid((unsigned)(d.B * d.Hv));
  if (d.Dk != 128) {
    set_error("the three-pass step is built for D == 128 only");
    return GDN_EUNSUPPORTED;
  }
  if (!launch_fits(d.B * d.Hv, 16 * kWave, "threepass_kernel")) return GDN_ESHAPE;
  // pass 1 reads s0 and pass 2 rewrites it into s_out (the launches are
  // ordered on the stream, so s_out == s0 is fine); pass 3 reads s_out
  threepass_kernel<DT, GT, 128, 16, 2, 16, 1><<<grid, 16 * kWave, 0, st>>>(a);
  int rc = device_status("three-pass kernel 1 launch");
  if (rc != GDN_OK) return rc;
  threepass_kernel<DT, GT, 128, 16, 2, 16, 2><<<grid, 16 * kWave, 0, st>>>(a);
  rc = device_status("three-pass kernel 2 launch");
  if (rc != GDN_OK) return rc;
  a.s0 = a.s_out;
  threepass_kernel<DT, GT, 128, 16, 2, 16, 3><<<grid, 16 * kWave, 0, st>>>(a);
  return device_status("three-pass kernel 3 launch");
}

template <int DT>
int launch_three_pass_gt(const gdn_desc& d, const StepArgs& a, hipStream_t st) {
  switch (d.gate_dtype) {
    case GDN_F32: return launch_three_pass_dt<DT, GDN_F32>(d, a, st);
    case GDN_F16: return launch_three_pass_dt<DT, GDN_F16>(d, a, st);
    default: return launch_three_pass_dt<DT, GDN_BF16>(d, a, st);
  }
}

int launch_step_three_pass(const gdn_desc& d, const void* q, const void* k, const void* v,
                           const void* ld, const void* beta, const float* s0, const void* z,
                           const void* w, float* y, float* s_out, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const StepArgs a{q, k, v, ld, beta, z, w, s0, y, s_out, (int)d.Hk, (int)d.Hv,
                   (int)(d.Hv / d.Hk), d.dtype, d.gate_dtype, d.flags, d.qk_eps, d.norm_eps,
                   q_scale(d)};
  switch (d.dtype) {
    case GDN_F32: return launch_three_pass_gt<GDN_F32>(d, a, st);
    case GDN_F16: return launch_three_pass_gt<GDN_F16>(d, a, st);
    default: return launch_three_pass_gt<GDN_BF16>(d, a, st);
  }
}

}  // namespace gdn

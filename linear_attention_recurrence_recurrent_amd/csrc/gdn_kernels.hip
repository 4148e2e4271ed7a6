// Gated DeltaNet recurrence on MI355X (gfx950): decode step, time-axis scan
// and gated RMSNorm kernels, plus the C-ABI entry points that launch them.
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
// Work layout on CDNA4 (wave64):
//   - a row of D columns is split over CL consecutive lanes ("row group");
//     lane j of the group owns the float4 column chunks j, j+CL, j+2CL, ...,
//     so a wave-wide float4 access of one chunk index touches CL contiguous
//     16-byte pieces per row;
//   - the two dots are reduced inside the row group with DPP butterflies
//     (quad_perm, row_half_mirror, row_mirror), which leave the same sum in
//     every lane of the group, so every lane updates its own columns with an
//     identical coef;
//   - a lane owns RPL rows, a wave 64/CL*RPL rows, a workgroup of NW waves
//     ROWS = NW*(64/CL)*RPL rows of one value head.
// Decode: a workgroup owns a whole head, streams its rows from HBM with
// nontemporal loads/stores (all loads of a lane issued before any math), and
// applies the gated RMSNorm in the same launch.
// Scan: the state stays in VGPRs for the whole time axis; q/k/v/gates are
// staged through LDS in chunks of TC tokens, q/k are normalised once per
// token per workgroup, and the outputs of a chunk are buffered in LDS and
// written back coalesced (gated in the same launch when the workgroup owns
// the whole head, else by the separate gated-norm kernel).
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>
#include <cstdint>
#include <cstdio>

#include "gdn.h"
#include "gdn_internal.h"

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

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

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

// ------------------------------------------------------------------ lane reductions
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of CL consecutive lanes (CL = 1, 2, 4, 8, 16).
// Butterfly order: every lane of a group ends with bit-identical sums.
template <int CL>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(CL == 1 || CL == 2 || CL == 4 || CL == 8 || CL == 16, "row group size");
  if constexpr (CL >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (CL >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (CL >= 8) x += dpp<0x141>(x);  // row_half_mirror: the other quad of 8
  if constexpr (CL >= 16) x += dpp<0x140>(x); // row_mirror: the other half of 16
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so that each
// XCD receives a contiguous range of tiles (the row blocks of one head, and
// the value heads of one key group, then share an L2).
__device__ __forceinline__ int64_t xcd_tile(int64_t i, int64_t n) {
  if (n % 8) return i;
  return (i % 8) * (n / 8) + i / 8;
}

// ------------------------------------------------------------------ decode step
struct StepArgs {
  const void *q, *k, *v, *ld, *beta, *z, *w;
  const float* s0;
  float* y;
  float* s_out;
  int Hk, Hv, G, dt, gdt;
  uint32_t flags;
  float qk_eps, norm_eps, qscale;
};

// N consecutive operand elements kept as their raw bits (16-bit dtypes stay
// packed two per VGPR) and widened to f32 on use.  N = 1, 2 or 4; the access
// is N elements wide, so the element index must be a multiple of N.
template <int DT, int N>
struct Raw {
  static_assert(N == 1 || N == 2 || N == 4, "Raw holds 1, 2 or 4 elements");
  static constexpr bool kF32 = DT == GDN_F32;
  typedef typename std::conditional<kF32, float, uint32_t>::type Word;
  static constexpr int kWords = kF32 ? N : (N + 1) / 2;
  Word w[kWords];
  __device__ __forceinline__ void load(const void* p, int64_t i) {
    if constexpr (kF32) {
      const float* f = static_cast<const float*>(p) + i;
      if constexpr (N == 4) {
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
      if constexpr (N == 4) {
        const uint2 t = *reinterpret_cast<const uint2*>(h);
        w[0] = t.x; w[1] = t.y;
      } else if constexpr (N == 2) {
        w[0] = *reinterpret_cast<const uint32_t*>(h);
      } else {
        w[0] = h[0];
      }
    }
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

// Registers of one head in flight: this lane's columns of q and k (raw), its
// RPL state rows (adjacent rows, float4 chunks), and its rows' v and z (raw).
template <int DT, int D, int CL, int RPL>
struct HeadRegs {
  static constexpr int NV4 = D / CL / 4;
  Raw<DT, 4> k[NV4], q[NV4];
  float4 S[RPL][NV4];
  Raw<DT, RPL> v, z;
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
  const float* s0 = a.s0 + head * (int64_t)(D * D);
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
#pragma unroll
    for (int m = 0; m < NV4; ++m) R.S[r][m] = nt_load4(s0 + (row0 + r) * D + 4 * (m * CL + j));
  }
  R.v.load(a.v, head * D + row0);
  if (a.z) R.z.load(a.z, head * D + row0);
}

// Fold the norms, run the fused row pass, write the state back and the
// (gated) output.  The L2 norms and the q scale are applied to the reduced
// dots as scalars (u = rk*(S.k), w = rq*(S.q), S += (coef*rk) k), so the
// normalised vectors are never materialised.  red[NW] is this head's slot for
// the cross-wave sum of the gated norm.
template <int DT, int GT, int D, int CL, int RPL, int NW>
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
  float* so = a.s_out + head * (int64_t)(D * D);
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
      nt_store4(s, so + (row0 + r) * D + 4 * (m * CL + j));
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
    Raw<DT, RPL> wr;
    wr.load(a.w, row0);
#pragma unroll
    for (int r = 0; r < RPL; ++r) o[r] *= inv * wr.get(r);
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
template <int DT, int GT, int D, int CL, int RPL, int NW>
__global__ __launch_bounds__(NW* kWave) void decode_kernel(StepArgs a) {
  static_assert((D / CL) % 4 == 0, "a lane owns whole float4 chunks");
  static_assert(NW * (kWave / CL) * RPL == D, "a workgroup owns the whole head");
  __shared__ float red[NW];
  const int64_t head = blockIdx.x;
  HeadRegs<DT, D, CL, RPL> R;
  decode_fetch<DT, GT, D, CL, RPL, NW>(a, head, R);
  decode_finish<DT, GT, D, CL, RPL, NW>(a, head, R, red);
}

// Persistent variant: a workgroup walks heads blockIdx.x, +gridDim.x, ... and
// issues the loads of its next head before finishing the current one, so the
// memory system stays busy through the arithmetic and the norm's barrier.
template <int DT, int GT, int D, int CL, int RPL, int NW>
__global__ __launch_bounds__(NW* kWave) void decode_persistent_kernel(StepArgs a, int64_t nheads) {
  static_assert((D / CL) % 4 == 0, "a lane owns whole float4 chunks");
  static_assert(NW * (kWave / CL) * RPL == D, "a workgroup owns the whole head");
  // two slots: a head's slot is rewritten only after the next head's barrier
  __shared__ float red[2][NW];
  HeadRegs<DT, D, CL, RPL> A, B;
  const int64_t stride = gridDim.x;
  int64_t h = blockIdx.x;
  if (h < nheads) decode_fetch<DT, GT, D, CL, RPL, NW>(a, h, A);
  while (h < nheads) {
    const int64_t h1 = h + stride;
    if (h1 < nheads) decode_fetch<DT, GT, D, CL, RPL, NW>(a, h1, B);
    decode_finish<DT, GT, D, CL, RPL, NW>(a, h, A, red[0]);
    if (h1 >= nheads) break;
    const int64_t h2 = h1 + stride;
    if (h2 < nheads) decode_fetch<DT, GT, D, CL, RPL, NW>(a, h2, A);
    decode_finish<DT, GT, D, CL, RPL, NW>(a, h1, B, red[1]);
    h = h2;
  }
}

// ------------------------------------------------------------------ scan
struct ScanArgs {
  const void *q, *k, *v, *ld, *beta, *z, *w;
  const float* s0;
  float* y;
  float* s_out;
  int64_t T;
  int Hk, Hv, G, nrb, dt, gdt, head_major;
  uint32_t flags;
  float qk_eps, norm_eps, qscale;
};

// Raw operands of one chunk of TC tokens, held in registers while the previous
// chunk computes.  Thread tid covers chunk items tid, tid + NT, ...
template <int DT, int GT, int D, int ROWS, int TC, int NT, bool WITH_Z>
struct ChunkRegs {
  static constexpr int D4 = D / 4, R2 = ROWS / 2;
  static constexpr int NQK = (TC * D4 + NT - 1) / NT;  // float4 groups of q and of k
  static constexpr int NV = (TC * R2 + NT - 1) / NT;   // pairs of v (and z) elements
  Raw<DT, 4> k[NQK], q[NQK];
  Raw<DT, 2> v[NV];
  Raw<DT, 2> z[WITH_Z ? NV : 1];
  Raw<GT, 1> ld, be;
};

// Operand bases and per-token strides of one (b, head) in either layout.
struct ScanBases {
  int64_t qk_base, qk_ts, v_base, v_ts, g_base, g_ts;
};

// Smallest and largest decay scale kept folded: outside [2^-30, 2^30] the
// state is brought back to scale 1 (and alpha == 0 always lands here).
constexpr float kFoldMin = 9.3132257e-10f, kFoldMax = 1.0737418e9f;
// Range of a chunk's running decay product for the unchecked chunk loop: the
// state is brought to scale 1 at every chunk start, so the scale inside the
// chunk is exactly this product; [2^-60, 2^60] keeps every folded quantity far
// from f32 overflow and underflow.
constexpr float kFastMin = 8.6736174e-19f, kFastMax = 1.1529215e18f;

// The scan processes the time axis in chunks of TC tokens staged through LDS,
// and each chunk in blocks of L tokens.  Within a block the recurrence is
// unrolled with the affine argument of the "Module gdn" page ("The fusion"),
// carried across tokens: with S the state at the block start,
//   S_i = A_{i+1} S + sum_{j<=i} (prod_{m=j+1..i} alpha_m) c_j k_j^T,
//   A_i = prod_{m<i} alpha_m,   c_i = beta_i (v_i - alpha_i u_i),
//   u_i = S_{i-1}.k_i = A_i (S.k_i) + sum_{j<i} P_ij c_j,
//   o_i = S_i.q_i     = A_{i+1} (S.q_i) + sum_{j<=i} Q_ij c_j,
// with P_ij = (prod_{m=j+1..i-1} alpha_m)(k_j.k_i) and
// Q_ij = (prod_{m=j+1..i} alpha_m)(k_j.q_i) the same for every row of a head.
// So the 2L dots of a row against the block-start state are independent, a
// short L x L substitution per row gives every c_i and o_i, and the state
// takes one rank-L update.  L = 1 is the plain per-token recurrence.
template <int DT, int GT, int D, int CL, int RPL, int NW, int TC, int L, bool FUSE_NORM>
__global__ __launch_bounds__(NW* kWave)
__attribute__((amdgpu_waves_per_eu(FUSE_NORM ? 2 : 1))) void scan_kernel(ScanArgs a) {
  constexpr int NCOL = D / CL, NV4 = NCOL / 4, RG = kWave / CL, ROWS = NW * RG * RPL;
  constexpr int NT = NW * kWave, D4 = D / 4, R2 = ROWS / 2;
  constexpr int LPT = D / 8;  // lanes per token in the norm pass (8 elements of q and k each)
  constexpr int NB = TC / L;  // blocks per chunk
  constexpr int NPB = L * (L - 1);  // off-diagonal Gram entries per block (k.k and k.q)
  constexpr bool KEEP_K = L * NV4 <= 8;  // keep the block's k columns for the update
  // Row-split shapes (one wave per SIMD, latency-bound) get a fully unrolled,
  // unchecked token loop for chunks whose decay products stay in range.
  constexpr bool UNROLL = !FUSE_NORM && L == 1 && NV4 * RPL <= 2;
  static_assert(NCOL % 4 == 0, "a lane owns whole float4 chunks");
  static_assert(D % ROWS == 0 && ROWS % 2 == 0, "row blocks tile the head");
  static_assert(!FUSE_NORM || ROWS == D, "the fused norm needs the whole head");
  static_assert(TC <= NT && NT % LPT == 0 && TC % L == 0, "chunk shape");
  typedef ChunkRegs<DT, GT, D, ROWS, TC, NT, FUSE_NORM> Chunk;
  __shared__ float4 sk[TC][D4];
  __shared__ float4 sq[TC][D4];
  __shared__ float sv[TC][ROWS];
  __shared__ float sz[FUSE_NORM ? 2 : 1][FUSE_NORM ? TC : 1][FUSE_NORM ? D : 1];
  __shared__ float so[TC][ROWS];
  __shared__ float sal[TC], sbe[TC], skq[TC];
  __shared__ float sP[NB][L][L], sQ[NB][L][L], sA[NB][L + 1], sR[NB][L], sAmin[NB], sAmax[NB];
  __shared__ int sfast;  // the chunk's decay products stay inside the folding range

  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int rb = (int)(tile % a.nrb);
  const int64_t bh = tile / a.nrb;
  const int hv = (int)(bh % a.Hv), hk = hv / a.G;
  const int64_t b = bh / a.Hv;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = lane / CL, j = lane % CL;
  const int64_t T = a.T;
  const bool has_z = FUSE_NORM && a.z != nullptr;

  ScanBases sb;
  if (a.head_major) {
    sb = {(b * a.Hk + hk) * T * D, D, (b * a.Hv + hv) * T * D, D, (b * a.Hv + hv) * T, 1};
  } else {
    sb = {(b * T * a.Hk + hk) * D, (int64_t)a.Hk * D, (b * T * a.Hv + hv) * D,
          (int64_t)a.Hv * D, b * T * a.Hv + hv, a.Hv};
  }
  const int row0 = rb * ROWS;
  const int64_t sbase = (b * a.Hv + hv) * (int64_t)(D * D);

  // chunk staging: global -> registers (issued early) -> LDS
  auto chunk_load = [&](Chunk& P, int64_t t0, int tc) {
#pragma unroll
    for (int i = 0; i < Chunk::NQK; ++i) {
      const int e = tid + i * NT, tt = e / D4, c4 = e % D4;
      if (e < TC * D4 && tt < tc) {
        const int64_t off = sb.qk_base + (t0 + tt) * sb.qk_ts + 4 * c4;
        P.k[i].load(a.k, off);
        P.q[i].load(a.q, off);
      }
    }
#pragma unroll
    for (int i = 0; i < Chunk::NV; ++i) {
      const int e = tid + i * NT, tt = e / R2, r2 = e % R2;
      if (e < TC * R2 && tt < tc) {
        const int64_t off = sb.v_base + (t0 + tt) * sb.v_ts + row0 + 2 * r2;
        P.v[i].load(a.v, off);
        if constexpr (FUSE_NORM) {
          if (has_z) P.z[i].load(a.z, off);
        }
      }
    }
    if (tid < tc) {
      const int64_t gi = sb.g_base + (t0 + tid) * sb.g_ts;
      P.ld.load(a.ld, gi);
      P.be.load(a.beta, gi);
    }
  };
  // Tokens tc..TC-1 of a short last chunk become identity steps (alpha = 1,
  // beta = 0, k = q = v = 0), so whole blocks can always be processed.
  auto chunk_store = [&](const Chunk& P, int tc, int zbuf) {
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < Chunk::NQK; ++i) {
      const int e = tid + i * NT, tt = e / D4, c4 = e % D4;
      if (e < TC * D4) {
        sk[tt][c4] = tt < tc ? P.k[i].get4(0) : zero4;
        sq[tt][c4] = tt < tc ? P.q[i].get4(0) : zero4;
      }
    }
#pragma unroll
    for (int i = 0; i < Chunk::NV; ++i) {
      const int e = tid + i * NT, tt = e / R2, r2 = e % R2;
      if (e < TC * R2) {
        sv[tt][2 * r2] = tt < tc ? P.v[i].get(0) : 0.f;
        sv[tt][2 * r2 + 1] = tt < tc ? P.v[i].get(1) : 0.f;
        if constexpr (FUSE_NORM) {
          if (has_z && tt < tc) {
            sz[zbuf][tt][2 * r2] = P.z[i].get(0);
            sz[zbuf][tt][2 * r2 + 1] = P.z[i].get(1);
          }
        }
      }
    }
    if (tid < TC) {
      sal[tid] = tid < tc ? expf(P.ld.get(0)) : 1.f;
      sbe[tid] = tid < tc ? P.be.get(0) : 0.f;
    }
  };

  // State S = gsc * St: St lives in VGPRs for the whole time axis.
  float4 St[RPL][NV4];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int row = row0 + (wave * RPL + r) * RG + g;
#pragma unroll
    for (int m = 0; m < NV4; ++m)
      St[r][m] = *reinterpret_cast<const float4*>(a.s0 + sbase + row * D + 4 * (m * CL + j));
  }
  float gsc = 1.f;
  float wgt[(D + kWave - 1) / kWave];  // norm weight for the fused output
  if constexpr (FUSE_NORM) {
#pragma unroll
    for (int i = 0; i < (D + kWave - 1) / kWave; ++i)
      wgt[i] = (has_z && lane + kWave * i < D) ? ld1<DT>(a.w, lane + kWave * i) : 0.f;
  }

  Chunk P;
  chunk_load(P, 0, (int)(T < TC ? T : TC));
  chunk_store(P, (int)(T < TC ? T : TC), 0);
  // Every load issued so far (state, weights, first chunk) is complete here;
  // saying so explicitly keeps the compiler from re-waiting for them inside
  // the token loop, where the next chunk's loads are in flight.
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  for (int64_t c = 0;; ++c) {
    const int64_t t0 = c * TC;
    const int tc = (int)((T - t0) < TC ? (T - t0) : TC);
    const int nblk = (tc + L - 1) / L;
    __syncthreads();

    // B1. fold the L2 norms and the q scale into the staged q and k, all
    //     tokens of the chunk at once (LPT lanes per token); padding tokens
    //     stay exactly zero
    for (int tt = tid / LPT; tt < tc; tt += NT / LPT) {
      const int p = tid % LPT;
      float4 k0 = sk[tt][2 * p], k1 = sk[tt][2 * p + 1];
      float4 q0 = sq[tt][2 * p], q1 = sq[tt][2 * p + 1];
      float skk = dot4(k1, k1, dot4(k0, k0, 0.f));
      float sqq = dot4(q1, q1, dot4(q0, q0, 0.f));
      float sqk = dot4(k1, q1, dot4(k0, q0, 0.f));
      skk = group_sum<LPT>(skk);
      sqq = group_sum<LPT>(sqq);
      sqk = group_sum<LPT>(sqk);
      float rk = 1.f, rq = a.qscale;
      if (a.flags & GDN_FOLD_QK_L2NORM) {
        rk = rsqrtf(skk + a.qk_eps);
        rq *= rsqrtf(sqq + a.qk_eps);
      }
      sk[tt][2 * p] = scale4(k0, rk);
      sk[tt][2 * p + 1] = scale4(k1, rk);
      sq[tt][2 * p] = scale4(q0, rq);
      sq[tt][2 * p + 1] = scale4(q1, rq);
      if (p == 0) skq[tt] = sqk * rk * rq;
    }
    const bool more = t0 + TC < T;
    if (more) chunk_load(P, t0 + TC, (int)((T - t0 - TC) < TC ? (T - t0 - TC) : TC));
    if (tid == 0) {  // range of the chunk's running decay product (padding has alpha = 1)
      float acc = 1.f;
      bool ok = true;
      for (int tt = 0; tt < TC; ++tt) {
        acc *= sal[tt];
        ok = ok && acc >= kFastMin && acc <= kFastMax;
      }
      sfast = ok ? 1 : 0;
    }
    if constexpr (L > 1) {
      __syncthreads();
      // B2. per-block coefficients shared by every row: the off-diagonal Gram
      //     entries times their decay products, and the decay prefixes.
      for (int x = tid / LPT; x < NB * NPB; x += NT / LPT) {
        const int p = tid % LPT;
        const int bk = x / NPB, y = x % NPB, kind = y / (NPB / 2);
        int pr = y % (NPB / 2), i = 1;
        while (pr >= i) { pr -= i; ++i; }
        const int jj = pr;  // j < i
        const int ti = bk * L + i, tj = bk * L + jj;
        const float4* other = kind ? sq[ti] : sk[ti];
        float dv = dot4(sk[tj][2 * p], other[2 * p], 0.f);
        dv = dot4(sk[tj][2 * p + 1], other[2 * p + 1], dv);
        dv = group_sum<LPT>(dv);
        if (p == 0) {
          float prod = 1.f;
          for (int m = jj + 1; m < i; ++m) prod *= sal[bk * L + m];
          if (kind) sQ[bk][i][jj] = dv * prod * sal[ti];
          else sP[bk][i][jj] = dv * prod;
        }
      }
      if (tid < NB) {
        const int bk = tid;
        float acc = 1.f, amin = 3.0e38f, amax = 0.f;
        sA[bk][0] = 1.f;
        for (int i = 0; i < L; ++i) {
          acc *= sal[bk * L + i];
          sA[bk][i + 1] = acc;
          amin = fminf(amin, acc);
          amax = fmaxf(amax, acc);
          sQ[bk][i][i] = skq[bk * L + i];
        }
        sAmin[bk] = amin;
        sAmax[bk] = amax;
        float rr = 1.f;
        for (int i = L - 1; i >= 0; --i) {
          sR[bk][i] = rr;
          rr *= sal[bk * L + i];
        }
      }
    }
    __syncthreads();

    // C. the recurrence: token by token (L == 1) or one block of L tokens after the other.  With
    //    S = gsc*St the update becomes St += sum_j c_j/(gsc*A_{j+1}) k_j and
    //    gsc *= A_L: one FMA per state element per token.  When the scale
    //    would leave [2^-30, 2^30] (and whenever an alpha is 0) St is brought
    //    to the block's end scale in place and the scale restarts at 1.
    // Bring the state to scale 1 at the chunk start (one multiply per element
    // per chunk); when the chunk's decay products stay in range the whole chunk
    // then runs without per-token range checks.
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int m = 0; m < NV4; ++m) St[r][m] = scale4(St[r][m], gsc);
    gsc = 1.f;
    auto checked_tokens = [&]() {
        // one token at a time with range checks: St += (coef/gsc') k with
        // gsc' = alpha*gsc, or a rescale of St when gsc' leaves the range
        for (int tt = 0; tt < tc; ++tt) {
          const float al = sal[tt], be = sbe[tt], kq = skq[tt];
          const float gn = gsc * al;
          const bool rescale = !(gn >= kFoldMin && gn <= kFoldMax);  // uniform, rare
          const float gnext = rescale ? 1.f : gn;
          const float ig = rescale ? 1.f : __builtin_amdgcn_rcpf(gn);
          float4 kc[NV4];
          float u0[RPL], u1[RPL], w0[RPL], w1[RPL];
#pragma unroll
          for (int r = 0; r < RPL; ++r) u0[r] = u1[r] = w0[r] = w1[r] = 0.f;
#pragma unroll
          for (int m = 0; m < NV4; ++m) {
            kc[m] = sk[tt][m * CL + j];
            const float4 qc = sq[tt][m * CL + j];
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
              if (m & 1) {
                u1[r] = dot4(St[r][m], kc[m], u1[r]);
                w1[r] = dot4(St[r][m], qc, w1[r]);
              } else {
                u0[r] = dot4(St[r][m], kc[m], u0[r]);
                w0[r] = dot4(St[r][m], qc, w0[r]);
              }
            }
          }
          float c2[RPL];
#pragma unroll
          for (int r = 0; r < RPL; ++r) {
            const int lr = (wave * RPL + r) * RG + g;
            const float u = group_sum<CL>(u0[r] + u1[r]) * gsc;
            const float wq = group_sum<CL>(w0[r] + w1[r]) * gsc;
            const float coef = be * (sv[tt][lr] - al * u);
            if (j == 0) so[tt][lr] = al * wq + coef * kq;
            c2[r] = coef * ig;
          }
          if (rescale) {
#pragma unroll
            for (int r = 0; r < RPL; ++r)
#pragma unroll
              for (int m = 0; m < NV4; ++m) St[r][m] = scale4(St[r][m], gn);
          }
#pragma unroll
          for (int r = 0; r < RPL; ++r) {
#pragma unroll
            for (int m = 0; m < NV4; ++m) {
              St[r][m].x = fmaf(c2[r], kc[m].x, St[r][m].x);
              St[r][m].y = fmaf(c2[r], kc[m].y, St[r][m].y);
              St[r][m].z = fmaf(c2[r], kc[m].z, St[r][m].z);
              St[r][m].w = fmaf(c2[r], kc[m].w, St[r][m].w);
            }
          }
          gsc = gnext;
        }
    };
    if constexpr (UNROLL) {
      if (sfast != 0) {
      // one token at a time, unchecked: St += (coef/g_t) k with g_t the running
        // decay product; short chunks are padded with identity tokens
        float obuf[UNROLL ? TC : 1][RPL];
#pragma unroll(UNROLL ? TC : 1)
        for (int tt = 0; tt < (UNROLL ? TC : tc); ++tt) {
          const float al = sal[tt], be = sbe[tt], kq = skq[tt];
          const float gn = gsc * al;
          const float ig = __builtin_amdgcn_rcpf(gn);
          float4 kc[NV4];
          float u0[RPL], u1[RPL], w0[RPL], w1[RPL];
#pragma unroll
          for (int r = 0; r < RPL; ++r) u0[r] = u1[r] = w0[r] = w1[r] = 0.f;
#pragma unroll
          for (int m = 0; m < NV4; ++m) {
            kc[m] = sk[tt][m * CL + j];
            const float4 qc = sq[tt][m * CL + j];
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
              if (m & 1) {
                u1[r] = dot4(St[r][m], kc[m], u1[r]);
                w1[r] = dot4(St[r][m], qc, w1[r]);
              } else {
                u0[r] = dot4(St[r][m], kc[m], u0[r]);
                w0[r] = dot4(St[r][m], qc, w0[r]);
              }
            }
          }
          float c2[RPL];
#pragma unroll
          for (int r = 0; r < RPL; ++r) {
            const int lr = (wave * RPL + r) * RG + g;
            const float u = group_sum<CL>(u0[r] + u1[r]) * gsc;
            const float wq = group_sum<CL>(w0[r] + w1[r]) * gsc;
            const float coef = be * (sv[tt][lr] - al * u);
            const float o = al * wq + coef * kq;
            if constexpr (UNROLL) {
              obuf[tt][r] = o;
            } else {
              if (j == 0) so[tt][lr] = o;
            }
            c2[r] = coef * ig;
          }
#pragma unroll
          for (int r = 0; r < RPL; ++r) {
#pragma unroll
            for (int m = 0; m < NV4; ++m) {
              St[r][m].x = fmaf(c2[r], kc[m].x, St[r][m].x);
              St[r][m].y = fmaf(c2[r], kc[m].y, St[r][m].y);
              St[r][m].z = fmaf(c2[r], kc[m].z, St[r][m].z);
              St[r][m].w = fmaf(c2[r], kc[m].w, St[r][m].w);
            }
          }
          gsc = gn;
        }
        if constexpr (UNROLL) {
          if (j == 0) {
#pragma unroll
            for (int tt = 0; tt < TC; ++tt)
#pragma unroll
              for (int r = 0; r < RPL; ++r) so[tt][(wave * RPL + r) * RG + g] = obuf[tt][r];
          }
        }
      } else {
        checked_tokens();
      }
    } else if constexpr (L == 1) {
      checked_tokens();
    } else {
      for (int bk = 0; bk < nblk; ++bk) {
        const int tb = bk * L;
        float4 kreg[KEEP_K ? L : 1][KEEP_K ? NV4 : 1];
        float d[RPL][L], e[RPL][L];
#pragma unroll
        for (int r = 0; r < RPL; ++r)
#pragma unroll
          for (int i = 0; i < L; ++i) d[r][i] = e[r][i] = 0.f;
#pragma unroll
        for (int m = 0; m < NV4; ++m) {
#pragma unroll
          for (int i = 0; i < L; ++i) {
            const float4 kc = sk[tb + i][m * CL + j];
            const float4 qc = sq[tb + i][m * CL + j];
            if constexpr (KEEP_K) kreg[i][m] = kc;
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
              d[r][i] = dot4(St[r][m], kc, d[r][i]);
              e[r][i] = dot4(St[r][m], qc, e[r][i]);
            }
          }
        }
        float cc[RPL][L];
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
          const int lr = (wave * RPL + r) * RG + g;
#pragma unroll
          for (int i = 0; i < L; ++i) {
            d[r][i] = group_sum<CL>(d[r][i]) * gsc;
            e[r][i] = group_sum<CL>(e[r][i]) * gsc;
          }
#pragma unroll
          for (int i = 0; i < L; ++i) {
            float u = sA[bk][i] * d[r][i];
#pragma unroll
            for (int jj = 0; jj < i; ++jj) u = fmaf(sP[bk][i][jj], cc[r][jj], u);
            cc[r][i] = sbe[tb + i] * (sv[tb + i][lr] - sal[tb + i] * u);
          }
#pragma unroll
          for (int i = 0; i < L; ++i) {
            float o = sA[bk][i + 1] * e[r][i];
#pragma unroll
            for (int jj = 0; jj <= i; ++jj) o = fmaf(sQ[bk][i][jj], cc[r][jj], o);
            if (j == 0) so[tb + i][lr] = o;
          }
        }
        const bool fold = gsc * sAmin[bk] >= kFoldMin && gsc * sAmax[bk] <= kFoldMax;  // uniform
        float f[L];
        if (fold) {
#pragma unroll
          for (int i = 0; i < L; ++i) f[i] = __builtin_amdgcn_rcpf(gsc * sA[bk][i + 1]);
        } else {
          const float gl = gsc * sA[bk][L];
#pragma unroll
          for (int i = 0; i < L; ++i) f[i] = sR[bk][i];
#pragma unroll
          for (int r = 0; r < RPL; ++r)
#pragma unroll
            for (int m = 0; m < NV4; ++m) St[r][m] = scale4(St[r][m], gl);
        }
#pragma unroll
        for (int r = 0; r < RPL; ++r)
#pragma unroll
          for (int i = 0; i < L; ++i) cc[r][i] *= f[i];
#pragma unroll
        for (int m = 0; m < NV4; ++m) {
#pragma unroll
          for (int i = 0; i < L; ++i) {
            float4 kc;
            if constexpr (KEEP_K) kc = kreg[i][m];
            else kc = sk[tb + i][m * CL + j];
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
              St[r][m].x = fmaf(cc[r][i], kc.x, St[r][m].x);
              St[r][m].y = fmaf(cc[r][i], kc.y, St[r][m].y);
              St[r][m].z = fmaf(cc[r][i], kc.z, St[r][m].z);
              St[r][m].w = fmaf(cc[r][i], kc.w, St[r][m].w);
            }
          }
        }
        gsc = fold ? gsc * sA[bk][L] : 1.f;
      }
    }
    __syncthreads();

    // D. write this chunk's outputs (gated here when the workgroup owns the head)
    bool written = false;
    if constexpr (FUSE_NORM) {
      if (has_z) {
        constexpr int EPL = (D + kWave - 1) / kWave;
        const int zb = (int)(c & 1);
        for (int tt = wave; tt < tc; tt += NW) {
          const int64_t vo = sb.v_base + (t0 + tt) * sb.v_ts;
          float x[EPL];
          float ss = 0.f;
#pragma unroll
          for (int i = 0; i < EPL; ++i) {
            const int rr = lane + kWave * i;
            x[i] = 0.f;
            if (rr < D) x[i] = so[tt][rr] * silu(sz[zb][tt][rr]);
            ss = fmaf(x[i], x[i], ss);
          }
          const float inv = rsqrtf(wave_sum(ss) * (1.0f / D) + a.norm_eps);
#pragma unroll
          for (int i = 0; i < EPL; ++i) {
            const int rr = lane + kWave * i;
            if (rr < D) a.y[vo + rr] = x[i] * inv * wgt[i];
          }
        }
        written = true;
      }
    }
    if (!written) {
      for (int e = tid; e < tc * ROWS; e += NT) {
        const int tt = e / ROWS, rr = e % ROWS;
        a.y[sb.v_base + (t0 + tt) * sb.v_ts + row0 + rr] = so[tt][rr];
      }
    }
    if (!more) break;
    // next chunk into LDS: sk/sq/sv/gates/block coefficients were last read in
    // phase C, before the barrier above; z is double-buffered because phase D
    // may still be reading this chunk's slot in other waves.
    chunk_store(P, (int)((T - t0 - TC) < TC ? (T - t0 - TC) : TC), (int)((c + 1) & 1));
  }

#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int row = row0 + (wave * RPL + r) * RG + g;
#pragma unroll
    for (int m = 0; m < NV4; ++m)
      *reinterpret_cast<float4*>(a.s_out + sbase + row * D + 4 * (m * CL + j)) =
          scale4(St[r][m], gsc);
  }
}

// ------------------------------------------------------------------ gated RMSNorm
// In place over y viewed as [nvec, D] (both layouts keep the head dim last and
// dense, and z shares y's layout); one wave per head vector.
template <int DT, int D>
__global__ __launch_bounds__(256) void gated_norm_kernel(float* y, const void* z, const void* w,
                                                         int64_t nvec, float eps) {
  constexpr int EPL = (D + kWave - 1) / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t vec = (int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (vec >= nvec) return;  // uniform per wave
  const int64_t base = vec * D;
  float x[EPL];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int rr = lane + kWave * i;
    x[i] = 0.f;
    if (rr < D) x[i] = y[base + rr] * silu(ld1<DT>(z, base + rr));
    ss = fmaf(x[i], x[i], ss);
  }
  const float inv = rsqrtf(wave_sum(ss) * (1.0f / D) + eps);
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int rr = lane + kWave * i;
    if (rr < D) y[base + rr] = x[i] * inv * ld1<DT>(w, rr);
  }
}

// ------------------------------------------------------------------ launchers
int device_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return GDN_OK;
  char msg[200];
  std::snprintf(msg, sizeof(msg), "%s: %s", what, hipGetErrorString(e));
  set_error(msg);
  return GDN_EDEVICE;
}

float q_scale(const gdn_desc& d) {
  return (d.flags & GDN_FOLD_Q_SCALE) ? 1.0f / std::sqrt((float)d.Dk) : 1.0f;
}

template <int DT, int GT>
int launch_step_dt(const gdn_desc& d, const StepArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(d.B * d.Hv));
  switch (d.Dk) {
    case 128: decode_kernel<DT, GT, 128, 8, 2, 8><<<grid, 8 * kWave, 0, st>>>(a); break;
    case 64: decode_kernel<DT, GT, 64, 4, 2, 2><<<grid, 2 * kWave, 0, st>>>(a); break;
    case 32: decode_kernel<DT, GT, 32, 4, 1, 2><<<grid, 2 * kWave, 0, st>>>(a); break;
    case 16: decode_kernel<DT, GT, 16, 4, 1, 1><<<grid, 1 * kWave, 0, st>>>(a); break;
    default: set_error("unsupported head dim"); return GDN_EUNSUPPORTED;
  }
  return device_status("decode_kernel launch");
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
                float* y, float* s_out, hipStream_t st) {
  const StepArgs a{q, k, v, ld, beta, z, w, s0, y, s_out, (int)d.Hk, (int)d.Hv,
                   (int)(d.Hv / d.Hk), d.dtype, d.gate_dtype, d.flags, d.qk_eps, d.norm_eps,
                   q_scale(d)};
  switch (d.dtype) {
    case GDN_F32: return launch_step_gt<GDN_F32>(d, a, st);
    case GDN_F16: return launch_step_gt<GDN_F16>(d, a, st);
    default: return launch_step_gt<GDN_BF16>(d, a, st);
  }
}

template <int DT, int GT, int D, int CL, int RPL, int NW, int TC, int L>
int launch_scan_cfg(ScanArgs a, int64_t heads, hipStream_t st) {
  constexpr int ROWS = NW * (kWave / CL) * RPL;
  a.nrb = D / ROWS;
  const dim3 grid((unsigned)(heads * a.nrb));
  if constexpr (ROWS == D) {
    scan_kernel<DT, GT, D, CL, RPL, NW, TC, L, true><<<grid, NW * kWave, 0, st>>>(a);
    return device_status("scan_kernel launch");
  } else {
    scan_kernel<DT, GT, D, CL, RPL, NW, TC, L, false><<<grid, NW * kWave, 0, st>>>(a);
    int rc = device_status("scan_kernel launch");
    if (rc != GDN_OK || a.z == nullptr) return rc;
    const int64_t nvec = heads * a.T;
    gated_norm_kernel<DT, D><<<dim3((unsigned)((nvec + 3) / 4)), 256, 0, st>>>(
        a.y, a.z, a.w, nvec, a.norm_eps);
    return device_status("gated_norm_kernel launch");
  }
}

template <int DT, int GT>
int launch_scan_dt(const ScanArgs& a, int D, int64_t heads, hipStream_t st) {
  switch (D) {
    case 128:
      // enough heads to fill the chip with whole-head workgroups: keep the
      // norm fused; otherwise split each head's rows over more workgroups
      if (heads >= 512) return launch_scan_cfg<DT, GT, 128, 4, 2, 4, 16, 1>(a, heads, st);
      if (heads >= 128) return launch_scan_cfg<DT, GT, 128, 8, 1, 4, 16, 1>(a, heads, st);
      return launch_scan_cfg<DT, GT, 128, 16, 1, 4, 16, 1>(a, heads, st);
    case 64:
      if (heads >= 256) return launch_scan_cfg<DT, GT, 64, 4, 1, 4, 32, 1>(a, heads, st);
      return launch_scan_cfg<DT, GT, 64, 8, 1, 2, 32, 1>(a, heads, st);
    case 32: return launch_scan_cfg<DT, GT, 32, 4, 1, 2, 32, 1>(a, heads, st);
    case 16: return launch_scan_cfg<DT, GT, 16, 4, 1, 1, 32, 1>(a, heads, st);
    default: set_error("unsupported head dim"); return GDN_EUNSUPPORTED;
  }
}

template <int DT>
int launch_scan_gt(const ScanArgs& a, int gdt, int D, int64_t heads, hipStream_t st) {
  switch (gdt) {
    case GDN_F32: return launch_scan_dt<DT, GDN_F32>(a, D, heads, st);
    case GDN_F16: return launch_scan_dt<DT, GDN_F16>(a, D, heads, st);
    default: return launch_scan_dt<DT, GDN_BF16>(a, D, heads, st);
  }
}

int launch_scan(const gdn_desc& d, const void* q, const void* k, const void* v, const void* ld,
                const void* beta, const float* s0, const void* z, const void* w, float* y,
                float* s_out, hipStream_t st) {
  const ScanArgs a{q, k, v, ld, beta, z, w, s0, y, s_out, d.T, (int)d.Hk, (int)d.Hv,
                   (int)(d.Hv / d.Hk), 1, d.dtype, d.gate_dtype, d.head_major, d.flags,
                   d.qk_eps, d.norm_eps, q_scale(d)};
  const int64_t heads = d.B * d.Hv;
  switch (d.dtype) {
    case GDN_F32: return launch_scan_gt<GDN_F32>(a, d.gate_dtype, (int)d.Dk, heads, st);
    case GDN_F16: return launch_scan_gt<GDN_F16>(a, d.gate_dtype, (int)d.Dk, heads, st);
    default: return launch_scan_gt<GDN_BF16>(a, d.gate_dtype, (int)d.Dk, heads, st);
  }
}

}  // namespace
}  // namespace gdn

extern "C" {

int gdn_recurrent_step(const gdn_desc* d, const void* q, const void* k, const void* v,
                       const void* log_decay, const void* beta, const float* s0, const void* z,
                       const void* w, float* y, float* s_out, void* stream) {
  int rc = gdn::check(d, q, k, v, log_decay, beta, s0, z, w, y, s_out);
  if (rc != GDN_OK) return rc;
  if (d->T != 1) {
    gdn::set_error("gdn_recurrent_step needs T == 1 (use gdn_scan for a time axis)");
    return GDN_EUNSUPPORTED;
  }
  if (d->B == 0) return GDN_OK;
  return gdn::launch_step(*d, q, k, v, log_decay, beta, s0, z, w, y, s_out,
                          static_cast<hipStream_t>(stream));
}

int gdn_scan(const gdn_desc* d, const void* q, const void* k, const void* v,
             const void* log_decay, const void* beta, const float* s0, const void* z,
             const void* w, float* y, float* s_out, void* stream) {
  int rc = gdn::check(d, q, k, v, log_decay, beta, s0, z, w, y, s_out);
  if (rc != GDN_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d->B == 0) return GDN_OK;
  if (d->T == 0) {
    if (s_out == s0) return GDN_OK;
    const size_t bytes = (size_t)(d->B * d->Hv * d->Dv * d->Dk) * sizeof(float);
    if (hipMemcpyAsync(s_out, s0, bytes, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return gdn::device_status("state copy for T == 0");
    return GDN_OK;
  }
  if (d->T == 1)  // one token: the decode kernel is the same computation, streamed once
    return gdn::launch_step(*d, q, k, v, log_decay, beta, s0, z, w, y, s_out, st);
  return gdn::launch_scan(*d, q, k, v, log_decay, beta, s0, z, w, y, s_out, st);
}

}  // extern "C"

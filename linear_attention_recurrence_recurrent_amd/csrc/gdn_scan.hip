// Time-axis scan of the Gated DeltaNet recurrence on MI355X (gfx950), and the
// standalone gated RMSNorm used when a head's rows are split over workgroups.
//
// The recurrence is the one of the "Module gdn" page (module description),
// fused per row as in its section "The fusion"; the scan covers the time axis
// as the "gated_delta" page's gated_delta_reference does, returning
// (output, final_state).  The state stays in VGPRs for the whole time axis;
// q/k/v/gates are staged through LDS in chunks of TC tokens (the next chunk
// loads into registers while the current one computes, and its q/k norms are
// reduced in registers on the way into LDS); outputs are buffered in LDS and
// written back coalesced, gated in the same launch when the workgroup owns the
// whole head.
// Rows are split over lanes exactly as in the decode kernel.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

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
// chunk computes.  Thread tid covers chunk items tid, tid + NT, ...; an item of
// q and k is 8 consecutive elements, so one token's q (or k) spans D/8
// adjacent lanes.
template <int DT, int GT, int D, int ROWS, int TC, int NT, bool WITH_Z>
struct ChunkRegs {
  static constexpr int D8 = D / 8, R2 = ROWS / 2;
  static constexpr int NQK = (TC * D8 + NT - 1) / NT;  // 8-element groups of q and of k
  static constexpr int NV = (TC * R2 + NT - 1) / NT;   // pairs of v (and z) elements
  Raw<DT, 8> k[NQK], q[NQK];
  Raw<DT, 2> v[NV];
  Raw<DT, 2> z[WITH_Z ? NV : 1];
  Raw<GT, 1> ld, be;
};

// Operand bases and per-token strides of one (b, head) in either layout.
struct ScanBases {
  int64_t qk_base, qk_ts, v_base, v_ts, g_base, g_ts;
};

// Smallest and largest decay scale kept folded in the per-token loop: outside
// [2^-30, 2^30] the state is brought back to scale 1 (and alpha == 0 always
// lands here).
constexpr float kFoldMin = 9.3132257e-10f, kFoldMax = 1.0737418e9f;
// Bound on a chunk's sum of |log_decay| for the chunk-scalar loop: the state is
// brought to scale 1 at every chunk start, so the scale inside the chunk is the
// running decay product, and every such product then lies within
// [e^-41, e^41] (about 2^-59 .. 2^59), far from f32 overflow and underflow.
// NaN or infinite gates fail the test and take the per-token loop.
constexpr float kFastLogSum = 41.0f;

// Inclusive prefix product over the 64 lanes of a wave (exec must be full):
// Hillis-Steele inside each row of 16 (row_shr 1, 2, 4, 8), then the row
// products carried forward (row_bcast 15 into rows 1 and 3, row_bcast 31 into
// rows 2 and 3).
__device__ __forceinline__ float wave_prefix_prod(float x) {
  x = row_prefix_prod(x);
  x *= dpp_or_one<0x142, 0xA>(x);
  x *= dpp_or_one<0x143, 0xC>(x);
  return x;
}

// The scan keeps each value head's state in VGPRs for the whole time axis
// (rows split over lanes as in the decode kernel: CL lanes per row, RPL rows
// per lane, NW waves, ROWS rows per workgroup) and processes the time axis in
// chunks of TC tokens staged through LDS.  q and k are staged raw (f32); their
// L2 norms and the q scale enter as per-token scalars rk, rq, and k^.q^.
//
// The state is kept as S = g * St with one FMA per element per token: with the
// "Module gdn" page's step (module description) and its fused form ("The
// fusion"), du = St.k, dw = St.q (raw vectors) and g_t the running decay
// product inside the chunk (g_t = alpha_t g_{t-1}, 1 at the chunk start),
//   coef' = v - g_t rk du              (= v - alpha u)
//   o     = g_t rq dw + (beta k^.q^) coef'
//   St   += (beta rk / g_t) coef' k    (S_t = alpha S_{t-1} + beta coef' k^)
// When the chunk's |log_decay| sum is small (kFastLogSum) the four per-token
// scalars g rk, g rq, beta rk / g and beta k^.q^ are formed for the whole chunk
// at once (a prefix product of the decays across lanes) and the token loop
// needs four scalar operations per row; otherwise the loop keeps g itself and
// rescales St whenever g leaves [2^-30, 2^30].  St returns to scale 1 at every
// chunk start.
template <int DT, int GT, int D, int CL, int RPL, int NW, int TC, bool FUSE_NORM>
__global__ __launch_bounds__(NW* kWave)
__attribute__((amdgpu_waves_per_eu(FUSE_NORM ? 2 : 1))) void scan_kernel(ScanArgs a) {
  constexpr int NCOL = D / CL, NV4 = NCOL / 4, RG = kWave / CL, ROWS = NW * RG * RPL;
  constexpr int NT = NW * kWave, D4 = D / 4, D8 = D / 8, R2 = ROWS / 2;
  // Row-split shapes (one wave per SIMD, latency-bound) get a fully unrolled
  // chunk-scalar loop with the outputs buffered in registers.
  constexpr bool UNROLL = !FUSE_NORM && NV4 * RPL <= 2;
  // Two accumulators per dot product when the lane's row part is long (a
  // shorter dependent chain); short parts keep one (fewer instructions).
  constexpr bool SPLIT_U = NV4 >= 4, SPLIT_W = NV4 >= 4;
  static_assert(NCOL % 4 == 0, "a lane owns whole float4 chunks");
  static_assert(D % ROWS == 0 && ROWS % 4 == 0, "row blocks tile the head");
  static_assert(!FUSE_NORM || ROWS == D, "the fused norm needs the whole head");
  static_assert(TC <= kWave && TC % NW == 0, "chunk shape");
  static_assert(D8 <= 32, "a token's q/k groups span at most two DPP rows");
  typedef ChunkRegs<DT, GT, D, ROWS, TC, NT, FUSE_NORM> Chunk;
  __shared__ float4 sk[TC][D4];  // raw k and q of the chunk
  __shared__ float4 sq[TC][D4];
  __shared__ float sv[TC][ROWS];
  __shared__ float sz[FUSE_NORM ? 2 : 1][FUSE_NORM ? TC : 1][FUSE_NORM ? D : 1];
  __shared__ __align__(16) float so[TC][ROWS];
  __shared__ float sal[TC], sbe[TC], srk[TC], srq[TC], skq[TC];
  __shared__ float4 spv[NW][TC];  // chunk scalars per token, one copy per wave
  __shared__ int sfast;           // the chunk takes the chunk-scalar loop

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
      const int e = tid + i * NT, tt = e / D8, c8 = e % D8;
      if (e < TC * D8 && tt < tc) {
        const int64_t off = sb.qk_base + (t0 + tt) * sb.qk_ts + 8 * c8;
        P.k[i].load(a.k, off);
        P.q[i].load(a.q, off);
      } else {  // padding: exact zeros, so staging needs no select
        P.k[i].zero();
        P.q[i].zero();
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
  // Registers -> LDS, with the per-token norm scalars: the D8 lanes holding one
  // token's q and k are adjacent and aligned (inside one half wave), so the three
  // dot products reduce across them.  Tokens tc..TC-1 of a short last chunk
  // become identity steps (alpha = 1, beta = 0, k = q = v = 0, rk = rq = 0).
  // FULL (tc == TC, every chunk but a short last one) drops the per-token
  // tests, leaving straight-line code whose chains the compiler interleaves.
  auto chunk_store = [&](const Chunk& P, int tc, int zbuf, auto full) {
    constexpr bool FULL = decltype(full)::value;
    constexpr bool ALL_E = (TC * D8) % NT == 0;  // every item index is in range
    const bool l2 = (a.flags & GDN_FOLD_QK_L2NORM) != 0;
    // The chunk's loads (issued a whole recurrence phase ago) are complete.
    // Waiting for all of them here, on every path, also tells the compiler
    // that none is pending afterwards; otherwise the lanes that load nothing
    // leave a possible pending load into these registers, and the next chunk's
    // load issue would wait for the output stores issued in between.
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
    constexpr int N = Chunk::NQK;
    float skk[N], sqq[N], sqk[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float4 k0 = P.k[i].get4(0), k1 = P.k[i].get4(1);
      const float4 q0 = P.q[i].get4(0), q1 = P.q[i].get4(1);
      skk[i] = dot4(k1, k1, dot4(k0, k0, 0.f));
      sqq[i] = dot4(q1, q1, dot4(q0, q0, 0.f));
      sqk[i] = dot4(k1, q1, dot4(k0, q0, 0.f));
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      skk[i] = group_sum<D8>(skk[i]);
      sqq[i] = group_sum<D8>(sqq[i]);
      sqk[i] = group_sum<D8>(sqk[i]);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int e = tid + i * NT, tt = e / D8, c8 = e % D8;
      if (ALL_E || e < TC * D8) {
        sk[tt][2 * c8] = P.k[i].get4(0);
        sk[tt][2 * c8 + 1] = P.k[i].get4(1);
        sq[tt][2 * c8] = P.q[i].get4(0);
        sq[tt][2 * c8 + 1] = P.q[i].get4(1);
        if (c8 == 0) {
          // without the L2 fold the square roots see 1 and return 1
          float rk = rsqrtf(l2 ? skk[i] + a.qk_eps : 1.f);
          float rq = a.qscale * rsqrtf(l2 ? sqq[i] + a.qk_eps : 1.f);
          if (!FULL && tt >= tc) rk = rq = 0.f;  // exact zeros even with eps == 0
          srk[tt] = rk;
          srq[tt] = rq;
          skq[tt] = sqk[i] * rk * rq;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < Chunk::NV; ++i) {
      const int e = tid + i * NT, tt = e / R2, r2 = e % R2;
      if (e < TC * R2) {
        const bool real = FULL || tt < tc;
        sv[tt][2 * r2] = real ? P.v[i].get(0) : 0.f;
        sv[tt][2 * r2 + 1] = real ? P.v[i].get(1) : 0.f;
        if constexpr (FUSE_NORM) {
          if (has_z && real) {
            sz[zbuf][tt][2 * r2] = P.z[i].get(0);
            sz[zbuf][tt][2 * r2 + 1] = P.z[i].get(1);
          }
        }
      }
    }
    if (tid < TC) {
      const bool real = FULL || tid < tc;
      sal[tid] = real ? expf(P.ld.get(0)) : 1.f;
      sbe[tid] = real ? P.be.get(0) : 0.f;
    }
    if (wave == 0) {  // the chunk's decay products stay in the chunk-scalar range
      const float sum = wave_sum(tid < tc ? fabsf(P.ld.get(0)) : 0.f);
      if (tid == 0) sfast = sum <= kFastLogSum ? 1 : 0;
    }
  };
  auto stage = [&](const Chunk& P, int tc, int zbuf) {
    if (tc == TC) chunk_store(P, tc, zbuf, std::true_type{});
    else chunk_store(P, tc, zbuf, std::false_type{});
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

  // Gated output of a chunk when the workgroup owns the whole head: one wave
  // per token, the wave's TC/NW tokens unrolled so that their reductions
  // overlap.  Every value is computed for every token slot (padding slots read
  // stale but in-range LDS); only the stores are guarded, and only in a short
  // last chunk (FULL false).
  auto write_gated = [&](int64_t t0, int tc, int zb, auto full) {
    constexpr bool FULL = decltype(full)::value;
    constexpr int EPL = (D + kWave - 1) / kWave, TPW = TC / NW;
    float x[TPW][EPL], inv[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = wave + NW * u;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int rr = lane + kWave * i, rc = rr < D ? rr : D - 1;
        x[u][i] = so[tt][rc] * silu(sz[zb][tt][rc]);
        ss = fmaf(x[u][i], (D >= kWave || rr < D) ? x[u][i] : 0.f, ss);
      }
      inv[u] = ss;
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) inv[u] = rsqrtf(wave_sum(inv[u]) * (1.0f / D) + a.norm_eps);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = wave + NW * u;
      if (FULL || tt < tc) {
        const int64_t vo = sb.v_base + (t0 + tt) * sb.v_ts;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          const int rr = lane + kWave * i;
          if (D >= kWave || rr < D) a.y[vo + rr] = x[u][i] * inv[u] * wgt[i];
        }
      }
    }
  };

  // du = St.k and dw = St.q for this lane's columns of its RPL rows (partial
  // sums; the caller reduces them over the CL lanes of each row).
  auto dots = [&](int tt, float4 (&kc)[NV4], float (&du)[RPL], float (&dw)[RPL]) {
    float u1[RPL], w1[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) du[r] = dw[r] = u1[r] = w1[r] = 0.f;
#pragma unroll
    for (int m = 0; m < NV4; ++m) {
      kc[m] = sk[tt][m * CL + j];
      const float4 qc = sq[tt][m * CL + j];
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        if (SPLIT_U && (m & 1)) u1[r] = dot4(St[r][m], kc[m], u1[r]);
        else du[r] = dot4(St[r][m], kc[m], du[r]);
        if (SPLIT_W && (m & 1)) w1[r] = dot4(St[r][m], qc, w1[r]);
        else dw[r] = dot4(St[r][m], qc, dw[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      du[r] = group_sum<CL>(SPLIT_U ? du[r] + u1[r] : du[r]);
      dw[r] = group_sum<CL>(SPLIT_W ? dw[r] + w1[r] : dw[r]);
    }
  };
  auto update = [&](const float4 (&kc)[NV4], const float (&c2)[RPL]) {
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
  };
  // One token given its scalars pv = (g rk, g rq, beta rk / g, beta k^.q^)
  // (g the state's scale after the token); resc first brings St from scale
  // gn to scale 1 (then pv was formed with g = 1 in its third entry).
  auto token = [&](int tt, const float4 pv, bool resc, float gn, float (&o)[RPL]) {
    float4 kc[NV4];
    float du[RPL], dw[RPL], c2[RPL];
    dots(tt, kc, du, dw);
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const float cf = fmaf(-pv.x, du[r], sv[tt][(wave * RPL + r) * RG + g]);
      o[r] = fmaf(pv.y, dw[r], pv.w * cf);
      c2[r] = cf * pv.z;
    }
    if (resc) {  // uniform, rare
#pragma unroll
      for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int m = 0; m < NV4; ++m) St[r][m] = scale4(St[r][m], gn);
    }
    update(kc, c2);
  };
  // The scalars of one token when the loop keeps the scale itself: the new
  // scale gn = alpha gsc is kept folded while it stays in [2^-30, 2^30];
  // otherwise St is brought to scale 1 in the token (alpha == 0 lands here).
  auto checked_scalars = [&](int tt, float4& pv, bool& resc, float& gn) {
    const float al = sal[tt], be = sbe[tt], kq = skq[tt], rk = srk[tt], rq = srq[tt];
    gn = gsc * al;
    resc = !(gn >= kFoldMin && gn <= kFoldMax);
    pv = make_float4(gn * rk, gn * rq, be * rk * (resc ? 1.f : __builtin_amdgcn_rcpf(gn)), be * kq);
    gsc = resc ? 1.f : gn;
  };
  // The chunk scalars for every token at once, one token per lane (padding
  // lanes: alpha = 1, rk = rq = beta = 0); each wave writes and reads its own
  // copy.  Returns the chunk's decay product.
  auto chunk_scalars = [&]() {
    const int tl = lane < TC ? lane : 0;
    const float gt = wave_prefix_prod(lane < TC ? sal[tl] : 1.f);
    if (lane < TC) {
      const float rk = srk[tl], be = sbe[tl];
      spv[wave][lane] = make_float4(gt * rk, gt * srq[tl], be * rk * __builtin_amdgcn_rcpf(gt),
                                    be * skq[tl]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gt), TC - 1));
  };
  auto store_o = [&](int tt, const float (&o)[RPL]) {
    if (j == 0) {
#pragma unroll
      for (int r = 0; r < RPL; ++r) so[tt][(wave * RPL + r) * RG + g] = o[r];
    }
  };

  Chunk P;
  chunk_load(P, 0, (int)(T < TC ? T : TC));
  stage(P, (int)(T < TC ? T : TC), 0);
  // Every load issued so far (state, weights, first chunk) is complete here;
  // saying so explicitly keeps the compiler from re-waiting for them inside
  // the token loop, where the next chunk's loads are in flight.
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  // Per chunk: barrier; issue the next chunk's loads; the recurrence (C);
  // barrier; the next chunk into LDS; this chunk's outputs (D).  The outputs
  // are stored after the next chunk's registers are consumed, so waiting for
  // those loads never waits for the output stores as well.
  for (int64_t c = 0;; ++c) {
    const int64_t t0 = c * TC;
    const int tc = (int)((T - t0) < TC ? (T - t0) : TC);
    const bool more = t0 + TC < T;
    const int tcn = more ? (int)((T - t0 - TC) < TC ? (T - t0 - TC) : TC) : 0;
    __syncthreads();
    if (more) chunk_load(P, t0 + TC, tcn);

    // C. the recurrence.  St to scale 1 at the chunk start (one multiply per
    //    element per chunk).
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int m = 0; m < NV4; ++m) St[r][m] = scale4(St[r][m], gsc);
    gsc = 1.f;
    if constexpr (UNROLL) {
      if (sfast != 0) {
        const float gl = chunk_scalars();
        float obuf[TC][RPL];
#pragma unroll
        for (int tt = 0; tt < TC; ++tt) token(tt, spv[wave][tt], false, 1.f, obuf[tt]);
#pragma unroll
        for (int tt = 0; tt < TC; ++tt) store_o(tt, obuf[tt]);
        gsc = gl;
      } else {
#pragma unroll 1
        for (int tt = 0; tt < tc; ++tt) {
          float4 pv;
          bool resc;
          float gn, o[RPL];
          checked_scalars(tt, pv, resc, gn);
          token(tt, pv, resc, gn, o);
          store_o(tt, o);
        }
      }
    } else {
      // one loop body for both kinds of chunk keeps the register pressure of one
      const bool fast = sfast != 0;
      float gl = 1.f;
      if (fast) gl = chunk_scalars();
#pragma unroll 1
      for (int tt = 0; tt < tc; ++tt) {
        float4 pv;
        bool resc = false;
        float gn = 1.f, o[RPL];
        if (fast) pv = spv[wave][tt];
        else checked_scalars(tt, pv, resc, gn);
        token(tt, pv, resc, gn, o);
        store_o(tt, o);
      }
      if (fast) gsc = gl;
    }
    __syncthreads();

    // next chunk into LDS: every chunk array was last read in phase C, before
    // the barrier above; z is double-buffered because phase D below still
    // reads this chunk's slot.  After the last chunk this stages an empty
    // chunk (tcn == 0): unconditional, so that its wait for the loads lies on
    // every path through the loop.
    stage(P, tcn, (int)((c + 1) & 1));

    // D. write this chunk's outputs (gated here when the workgroup owns the head)
    bool written = false;
    if constexpr (FUSE_NORM) {
      if (has_z) {
        if (tc == TC) write_gated(t0, tc, (int)(c & 1), std::true_type{});
        else write_gated(t0, tc, (int)(c & 1), std::false_type{});
        written = true;
      }
    }
    if (!written) {  // 16-byte stores of 4 rows of one token
      constexpr int R4 = ROWS / 4, NYS = (TC * R4 + NT - 1) / NT;
#pragma unroll
      for (int i = 0; i < NYS; ++i) {
        const int e = tid + i * NT, tt = e / R4, r4 = e % R4;
        if (e < TC * R4 && tt < tc)
          *reinterpret_cast<float4*>(a.y + sb.v_base + (t0 + tt) * sb.v_ts + row0 + 4 * r4) =
              *reinterpret_cast<const float4*>(&so[tt][4 * r4]);
      }
    }
    if (!more) break;
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
// dense, and z shares y's layout).  A lane owns four consecutive elements of a
// vector (16-byte loads and stores of y), D/4 lanes one vector, so a wave
// instruction covers 256/D vectors; a wave takes kNormVectors vectors (at
// least one instruction's worth) with all its loads issued before any use.
constexpr int kNormVectors = 8;
template <int D>
constexpr int norm_vectors_per_wave() {
  return kWave / (D / 4) > kNormVectors ? kWave / (D / 4) : kNormVectors;
}
template <int D>
inline dim3 norm_grid(int64_t nvec) {
  const int64_t per_block = norm_vectors_per_wave<D>() * (256 / kWave);
  return dim3((unsigned)((nvec + per_block - 1) / per_block));
}
template <int DT, int D>
__global__ __launch_bounds__(256) void gated_norm_kernel(float* y, const void* z, const void* w,
                                                         int64_t nvec, float eps) {
  static_assert(D % 4 == 0 && D / 4 <= kWave, "four elements per lane, a vector within a wave");
  constexpr int LPV = D / 4, VPI = kWave / LPV, V = norm_vectors_per_wave<D>() / VPI;
  const int lane = threadIdx.x % kWave;
  const int64_t v0 =
      ((int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave) * (V * VPI) + lane / LPV;
  const int r0 = (lane % LPV) * 4;
  Raw<GDN_F32, 4> yv[V];
  Raw<DT, 4> zv[V];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int64_t vec = v0 + (int64_t)u * VPI;
    if (vec < nvec) {  // uniform within a vector's lanes
      yv[u].load(y, vec * D + r0);
      zv[u].load(z, vec * D + r0);
    } else {
      yv[u].zero();
      zv[u].zero();
    }
  }
  float wl[4];  // w is aligned to its element size only: one element per load
#pragma unroll
  for (int i = 0; i < 4; ++i) wl[i] = ld1<DT>(w, r0 + i);
#pragma unroll
  for (int u = 0; u < V; ++u) {
    float x[4];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = yv[u].get(i) * silu(zv[u].get(i));
      ss = fmaf(x[i], x[i], ss);
    }
    // the sum over the vector's lanes (the exec mask is full here)
    if constexpr (LPV == kWave) ss = wave_sum(ss);
    else ss = group_sum<LPV>(ss);
    const float inv = rsqrtf(ss * (1.0f / D) + eps);
    const int64_t vec = v0 + (int64_t)u * VPI;
    if (vec < nvec)
      *reinterpret_cast<float4*>(y + vec * D + r0) =
          make_float4(x[0] * inv * wl[0], x[1] * inv * wl[1], x[2] * inv * wl[2],
                      x[3] * inv * wl[3]);
  }
}

// The gated norm over nvec vectors in launches of at most kNormChunk vectors
// each (2^31 work-items at most: a dispatch counts them in 32 bits), so its
// size is bounded only by the operands.
constexpr int64_t kNormChunk = (int64_t)1 << 28;
template <int DT, int D>
void launch_norm_d(float* y, const void* z, const void* w, int64_t nvec, float eps,
                   hipStream_t st) {
  constexpr int64_t es = DT == GDN_F32 ? 4 : 2;
  for (int64_t v0 = 0; v0 < nvec; v0 += kNormChunk) {
    const int64_t n = nvec - v0 < kNormChunk ? nvec - v0 : kNormChunk;
    gated_norm_kernel<DT, D><<<norm_grid<D>(n), 256, 0, st>>>(
        y + v0 * D, static_cast<const char*>(z) + v0 * D * es, w, n, eps);
  }
}

}  // namespace

template <int DT, int GT, int D, int CL, int RPL, int NW, int TC>
int launch_scan_cfg(ScanArgs a, int64_t heads, hipStream_t st) {
  constexpr int ROWS = NW * (kWave / CL) * RPL;
  a.nrb = D / ROWS;
  if (!launch_fits(heads * a.nrb, NW * kWave, "scan_kernel")) return GDN_ESHAPE;
  const dim3 grid((unsigned)(heads * a.nrb));
  if constexpr (ROWS == D) {
    scan_kernel<DT, GT, D, CL, RPL, NW, TC, true><<<grid, NW * kWave, 0, st>>>(a);
    return device_status("scan_kernel launch");
  } else {
    scan_kernel<DT, GT, D, CL, RPL, NW, TC, false><<<grid, NW * kWave, 0, st>>>(a);
    int rc = device_status("scan_kernel launch");
    if (rc != GDN_OK || a.z == nullptr) return rc;
    launch_norm_d<DT, D>(a.y, a.z, a.w, heads * a.T, a.norm_eps, st);
    return device_status("gated_norm_kernel launch");
  }
}

template <int DT, int GT>
int launch_scan_dt(const ScanArgs& a, int D, int64_t heads, hipStream_t st) {
  switch (D) {
    case 256:
      // 16 workgroups per head (a whole-head workgroup would need 128 state
      // floats per lane and spill), then the standalone gated norm
      return launch_scan_cfg<DT, GT, 256, 16, 1, 4, 16>(a, heads, st);
    case 128:
      // enough heads to fill the chip with whole-head workgroups: keep the
      // norm fused; otherwise split each head's rows over more workgroups
      if (heads >= 512) return launch_scan_cfg<DT, GT, 128, 4, 2, 4, 16>(a, heads, st);
      if (heads >= 128) return launch_scan_cfg<DT, GT, 128, 8, 1, 4, 16>(a, heads, st);
      return launch_scan_cfg<DT, GT, 128, 16, 1, 4, 32>(a, heads, st);
    case 64:
      if (heads >= 256) return launch_scan_cfg<DT, GT, 64, 4, 1, 4, 32>(a, heads, st);
      return launch_scan_cfg<DT, GT, 64, 8, 1, 2, 32>(a, heads, st);
    case 32: return launch_scan_cfg<DT, GT, 32, 4, 1, 2, 32>(a, heads, st);
    case 16: return launch_scan_cfg<DT, GT, 16, 4, 1, 1, 32>(a, heads, st);
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

// the standalone gated norm over y in place (the few-head block form)
template <int DT>
void launch_norm(int D, float* y, const void* z, const void* w, int64_t nvec, float eps,
                 hipStream_t st) {
  switch (D) {
    case 32: launch_norm_d<DT, 32>(y, z, w, nvec, eps, st); break;
    case 64: launch_norm_d<DT, 64>(y, z, w, nvec, eps, st); break;
    case 256: launch_norm_d<DT, 256>(y, z, w, nvec, eps, st); break;
    default: launch_norm_d<DT, 128>(y, z, w, nvec, eps, st); break;
  }
}

int launch_scan(const gdn_desc& d, const void* q, const void* k, const void* v, const void* ld,
                const void* beta, const float* s0, const void* z, const void* w, float* y,
                float* s_out, void* workspace, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const ScanArgs a{q, k, v, ld, beta, z, w, s0, y, s_out, d.T, (int)d.Hk, (int)d.Hv,
                   (int)(d.Hv / d.Hk), 1, d.dtype, d.gate_dtype, d.head_major, d.flags,
                   d.qk_eps, d.norm_eps, q_scale(d)};
  const int64_t heads = d.B * d.Hv;
  // the block form where it fits (faster there on both the few-head and the
  // many-head shapes) unless the token-by-token form is asked for
  if (scan_uses_block_form(d)) {
    bool gated = false;
    int rc = launch_scan_chunked(d, q, k, v, ld, beta, s0, z, w, y, s_out, workspace, stream,
                                 &gated);
    if (rc != GDN_OK || gated || z == nullptr) return rc;
    const int64_t nvec = heads * d.T;
    switch (d.dtype) {
      case GDN_F32: launch_norm<GDN_F32>((int)d.Dv, y, z, w, nvec, d.norm_eps, st); break;
      case GDN_F16: launch_norm<GDN_F16>((int)d.Dv, y, z, w, nvec, d.norm_eps, st); break;
      default: launch_norm<GDN_BF16>((int)d.Dv, y, z, w, nvec, d.norm_eps, st); break;
    }
    return device_status("gated_norm_kernel launch");
  }
  switch (d.dtype) {
    case GDN_F32: return launch_scan_gt<GDN_F32>(a, d.gate_dtype, (int)d.Dk, heads, st);
    case GDN_F16: return launch_scan_gt<GDN_F16>(a, d.gate_dtype, (int)d.Dk, heads, st);
    default: return launch_scan_gt<GDN_BF16>(a, d.gate_dtype, (int)d.Dk, heads, st);
  }
}

}  // namespace gdn

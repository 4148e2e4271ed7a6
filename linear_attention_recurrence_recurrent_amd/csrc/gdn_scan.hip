// Time-axis scan of the Gated DeltaNet recurrence on MI355X (gfx950), and the
// standalone gated RMSNorm used when a head's rows are split over workgroups.
//
// The recurrence is the one of the "Module gdn" page (module description),
// fused per row as in its section "The fusion"; the scan covers the time axis
// as the "gated_delta" page's gated_delta_reference does, returning
// (output, final_state).  The state stays in VGPRs for the whole time axis;
// q/k/v/gates are staged through LDS in chunks of TC tokens (the next chunk
// loads into registers while the current one computes, and is normalised in
// registers on its way into LDS); outputs are buffered in LDS and written back
// coalesced, gated in the same launch when the workgroup owns the whole head.
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

// Smallest and largest decay scale kept folded: outside [2^-30, 2^30] the
// state is brought back to scale 1 (and alpha == 0 always lands here).
constexpr float kFoldMin = 9.3132257e-10f, kFoldMax = 1.0737418e9f;
// Bound on a chunk's sum of |log_decay| for the unchecked chunk loop: the state
// is brought to scale 1 at every chunk start, so the scale inside the chunk is
// the running decay product, and every such product then lies within
// [e^-41, e^41] (about 2^-59 .. 2^59), far from f32 overflow and underflow.
// NaN or infinite gates fail the test and take the checked loop.
constexpr float kFastLogSum = 41.0f;

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
  constexpr int NT = NW * kWave, D4 = D / 4, D8 = D / 8, R2 = ROWS / 2;
  constexpr int LPT = D / 8;  // lanes per token in the norm pass (8 elements of q and k each)
  constexpr int NB = TC / L;  // blocks per chunk
  constexpr int NPB = L * (L - 1);  // off-diagonal Gram entries per block (k.k and k.q)
  constexpr bool KEEP_K = L * NV4 <= 8;  // keep the block's k columns for the update
  // Row-split shapes (one wave per SIMD, latency-bound) get a fully unrolled,
  // unchecked token loop for chunks whose decay products stay in range.
  constexpr bool UNROLL = !FUSE_NORM && L == 1 && NV4 * RPL <= 2;
  static_assert(NCOL % 4 == 0, "a lane owns whole float4 chunks");
  static_assert(D % ROWS == 0 && ROWS % 4 == 0, "row blocks tile the head");
  static_assert(!FUSE_NORM || ROWS == D, "the fused norm needs the whole head");
  static_assert(TC <= kWave && NT % LPT == 0 && TC % L == 0, "chunk shape");
  static_assert(D / 8 <= 16, "a token's q/k groups span at most one DPP row");
  static_assert(!FUSE_NORM || TC % NW == 0, "whole tokens per wave in the fused output");
  typedef ChunkRegs<DT, GT, D, ROWS, TC, NT, FUSE_NORM> Chunk;
  __shared__ float4 sk[TC][D4];
  __shared__ float4 sq[TC][D4];
  __shared__ float sv[TC][ROWS];
  __shared__ float sz[FUSE_NORM ? 2 : 1][FUSE_NORM ? TC : 1][FUSE_NORM ? D : 1];
  __shared__ __align__(16) float so[TC][ROWS];
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
  // Registers -> LDS, folding in the L2 norms and the q scale on the way: the
  // D8 lanes holding one token's q and k are adjacent and aligned inside one
  // DPP row, so the three dot products reduce across them.  Tokens tc..TC-1 of
  // a short last chunk become identity steps (alpha = 1, beta = 0,
  // k = q = v = 0), so whole blocks can always be processed.  FULL (tc == TC,
  // every chunk but a short last one) drops the per-token tests, leaving
  // straight-line code whose chains the compiler can interleave.
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
      // without the L2 fold the square roots see 1 and return 1
      float rk = rsqrtf(l2 ? skk[i] + a.qk_eps : 1.f);
      float rq = a.qscale * rsqrtf(l2 ? sqq[i] + a.qk_eps : 1.f);
      if constexpr (!FULL) {
        if (tt >= tc) rk = rq = 0.f;  // padding stays exactly zero even with eps == 0
      }
      if (ALL_E || e < TC * D8) {
        sk[tt][2 * c8] = scale4(P.k[i].get4(0), rk);
        sk[tt][2 * c8 + 1] = scale4(P.k[i].get4(1), rk);
        sq[tt][2 * c8] = scale4(P.q[i].get4(0), rq);
        sq[tt][2 * c8 + 1] = scale4(P.q[i].get4(1), rq);
        if (c8 == 0) skq[tt] = sqk[i] * rk * rq;
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
    if constexpr (UNROLL) {
      if (wave == 0) {  // the chunk's decay products stay in the unchecked range
        const float s = wave_sum(tid < tc ? fabsf(P.ld.get(0)) : 0.f);
        if (tid == 0) sfast = s <= kFastLogSum ? 1 : 0;
      }
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
    const int nblk = (tc + L - 1) / L;
    const bool more = t0 + TC < T;
    const int tcn = more ? (int)((T - t0 - TC) < TC ? (T - t0 - TC) : TC) : 0;
    __syncthreads();
    if (more) chunk_load(P, t0 + TC, tcn);

    if constexpr (L > 1) {
      // B. per-block coefficients shared by every row: the off-diagonal Gram
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
      __syncthreads();
    }

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

    // next chunk into LDS: sk/sq/sv/gates/block coefficients were last read in
    // phase C, before the barrier above; z is double-buffered because phase D
    // below still reads this chunk's slot.  After the last chunk this stages
    // an empty chunk (tcn == 0): unconditional, so that its wait for the loads
    // lies on every path through the loop.
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

}  // namespace

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
      return launch_scan_cfg<DT, GT, 128, 16, 1, 4, 32, 1>(a, heads, st);
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
                float* s_out, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
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

}  // namespace gdn

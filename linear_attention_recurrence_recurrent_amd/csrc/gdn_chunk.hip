// Time-axis scan of the Gated DeltaNet recurrence in block form on the matrix
// cores (gfx950 MFMA, FP32 in and out), for D = 128.
//
// The recurrence is the one of the "Module gdn" page (module description).
// Its section "The fusion" observes that the step is affine in the memory S;
// carrying that affine map over a block of L = 16 tokens turns the block into
// dense products.  With S the state at the block start (true scale), k^ and
// q^ the normalised keys and queries, and for tokens i, j of the block
//   Dc[i][j] = alpha_{j+1} ... alpha_i  (j <= i; 1 on the diagonal),
//   gam_i    = alpha_0 ... alpha_i,
// the step S_i = alpha_i S_{i-1} + c_i k^_i^T with c_i = beta_i (v_i - alpha_i
// S_{i-1} k^_i) unrolls to
//   (I + Ls) C = diag(beta) V - diag(beta gam) K^ S^T,
//   Ls[i][j] = beta_i (k^_i . k^_j) Dc[i][j]  (j < i),
//   O  = diag(gam) Q^ S^T + (tril(Q^ K^^T) (.) Dc) C,
//   S' = gam_15 S + ((diag(Dc[15][.]) K^)^T C)^T.
// Everything but the products with S depends on the block's own inputs, so
// the work splits in two launches:
//   prep_kernel  (one workgroup per head and block, all in parallel): the
//                norms, decay products, K K^T and Q K^T on the matrix cores,
//                T = (I + Ls)^-1 by forward substitution and the masked
//                Hd = tril(Q^ K^^T) (.) Dc, written as a small block record;
//   state_kernel (one workgroup per head and 16 * NA value rows, sequential
//                over the blocks): P = K S^T and Q S^T, C = T (diag(beta) V -
//                diag(beta gam rk) P), O = diag(gam rq) Q S^T + Hd C and the
//                rank-16 update of S^T, all as v_mfma_f32_16x16x4f32 on raw
//                q and k with the norms folded into per-token scales.
// The sequential chain then holds only the products with S.  S^T stays in the
// accumulator layout for the whole time axis: lane l, register r of a 16 x 16
// tile holds S^T[4(l/16) + r][l%16] (key row within the tile, value column),
// which is also a valid B operand of the next product when the contraction
// index is taken in the matching order.  Decays are products (never
// quotients), so alpha = 0 needs no special case.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kD = 128;       // head dim handled here
constexpr int kL = 16;        // tokens per block (the MFMA tile)
constexpr int kPad = kD + 4;  // LDS row of q or k: rows 16 banks apart for the operand reads

// Block record, per (value head, block), f32; the records of a head are
// contiguous, kRec floats apart (256-byte aligned).
enum : int {
  kRecT = 0,       // [16][16] T = (I + Ls)^-1, row-major
  kRecH = 256,     // [16][16] Hd = tril(Q^ K^^T) (.) Dc
  kRecSig = 512,   // [16] gam_i rq_i: scale of (Q S^T)_i in O
  kRecWsc = 528,   // [16] beta_i gam_i rk_i: scale of (K S^T)_i in C
  kRecSrs = 544,   // [16] rk_i Dc[15][i]: key scale of the state update
  kRecBe = 560,    // [16] beta_i
  kRecGl = 576,    // gam_15, the decay over the whole block
  kRecUsed = 580,  // floats read back (a multiple of 4)
  kRec = 640       // stride
};

__device__ __forceinline__ int64_t record_at(int64_t bh, int64_t c, int64_t nblk) {
  return (bh * nblk + c) * kRec;
}

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct Bases {
  int64_t qk, qk_ts, v, v_ts, g, g_ts;
};

__device__ __forceinline__ Bases head_bases(int64_t b, int hv, int hk, int Hk, int Hv, int64_t T,
                                            int head_major) {
  Bases r;
  if (head_major) {
    r.qk = (b * Hk + hk) * T * kD; r.qk_ts = kD;
    r.v = (b * Hv + hv) * T * kD; r.v_ts = kD;
    r.g = (b * Hv + hv) * T; r.g_ts = 1;
  } else {
    r.qk = (b * T * Hk + hk) * kD; r.qk_ts = (int64_t)Hk * kD;
    r.v = (b * T * Hv + hv) * kD; r.v_ts = (int64_t)Hv * kD;
    r.g = b * T * Hv + hv; r.g_ts = Hv;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Block pieces that do not depend on the state.

struct PrepArgs {
  const void *q, *k, *ld, *beta;
  float* rec;
  int64_t T, nblk;
  int Hk, Hv, G, head_major;
  uint32_t flags;
  float qk_eps, qscale;
};

template <int DT, int GT>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  __shared__ __align__(16) float sk[kL][kPad];
  __shared__ __align__(16) float sq[kL][kPad];
  __shared__ float sGp[2][kL][kL + 1], sHp[2][kL][kL + 1];
  __shared__ float sLs[kL][kL + 1];
  __shared__ float sal[kL], sbe[kL], srk[kL], srq[kL];

  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t c = tile % a.nblk, bh = tile / a.nblk;
  const int hv = (int)(bh % a.Hv), hk = hv / a.G;
  const int64_t b = bh / a.Hv;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int lg = lane / 16, lc = lane % 16;
  const int64_t t0 = c * kL;
  const int tc = (int)((a.T - t0) < kL ? (a.T - t0) : kL);
  const Bases bs = head_bases(b, hv, hk, a.Hk, a.Hv, a.T, a.head_major);
  float* rec = a.rec + record_at(bh, c, a.nblk);

  {  // raw k and q into LDS (thread: token tid / 16, elements 8 (tid % 16) ..), norms
    const int tt = tid / 16, c8 = tid % 16;
    Raw<DT, 8> rk8, rq8;
    if (tt < tc) {
      rk8.load(a.k, bs.qk + (t0 + tt) * bs.qk_ts + 8 * c8);
      rq8.load(a.q, bs.qk + (t0 + tt) * bs.qk_ts + 8 * c8);
    } else {
      rk8.zero();
      rq8.zero();
    }
    if (tid < kL) {
      float al = 1.f, be = 0.f;
      if (tid < tc) {
        Raw<GT, 1> l1, b1;
        l1.load(a.ld, bs.g + (t0 + tid) * bs.g_ts);
        b1.load(a.beta, bs.g + (t0 + tid) * bs.g_ts);
        al = expf(l1.get(0));
        be = b1.get(0);
      }
      sal[tid] = al;
      sbe[tid] = be;
    }
    const float4 k0 = rk8.get4(0), k1 = rk8.get4(1), q0 = rq8.get4(0), q1 = rq8.get4(1);
    *reinterpret_cast<float4*>(&sk[tt][8 * c8]) = k0;
    *reinterpret_cast<float4*>(&sk[tt][8 * c8 + 4]) = k1;
    *reinterpret_cast<float4*>(&sq[tt][8 * c8]) = q0;
    *reinterpret_cast<float4*>(&sq[tt][8 * c8 + 4]) = q1;
    const float ssk = group_sum<16>(dot4(k1, k1, dot4(k0, k0, 0.f)));
    const float ssq = group_sum<16>(dot4(q1, q1, dot4(q0, q0, 0.f)));
    if (c8 == 0) {
      const bool l2 = (a.flags & GDN_FOLD_QK_L2NORM) != 0;
      float rk = rsqrtf(l2 ? ssk + a.qk_eps : 1.f);
      float rq = rsqrtf(l2 ? ssq + a.qk_eps : 1.f) * a.qscale;
      if (tt >= tc) rk = rq = 0.f;
      srk[tt] = rk;
      srq[tt] = rq;
    }
  }
  __syncthreads();

  // decay products: thread (i, j) one entry
  const int i = tid / 16, j = tid % 16;
  float dc = j <= i ? 1.f : 0.f;
#pragma unroll
  for (int m = 1; m < kL; ++m) dc *= (m > j && m <= i) ? sal[m] : 1.f;
  {  // waves 0, 1: K K^T; waves 2, 3: Q K^T; each over four key tiles
    const bool is_h = wave >= 2;
    const int part = wave & 1;
    v4f g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 4 * part; ct < 4 * part + 4; ++ct) {
      const float4 kf = *reinterpret_cast<const float4*>(&sk[lc][16 * ct + 4 * lg]);
      const float4 af = is_h ? *reinterpret_cast<const float4*>(&sq[lc][16 * ct + 4 * lg]) : kf;
      g = mfma4(af.x, kf.x, g);
      g = mfma4(af.y, kf.y, g);
      g = mfma4(af.z, kf.z, g);
      g = mfma4(af.w, kf.w, g);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (is_h) sHp[part][4 * lg + r][lc] = g[r];
      else sGp[part][4 * lg + r][lc] = g[r];
    }
  }
  __syncthreads();

  {  // Ls, Hd and the per-token scales
    const float gij = sGp[0][i][j] + sGp[1][i][j], hij = sHp[0][i][j] + sHp[1][i][j];
    sLs[i][j] = j < i ? sbe[i] * srk[i] * gij * srk[j] * dc : 0.f;
    rec[kRecH + 16 * i + j] = j <= i ? srq[i] * hij * srk[j] * dc : 0.f;
    if (j == 0) {
      const float gam = sal[0] * dc;
      rec[kRecSig + i] = gam * srq[i];
      rec[kRecWsc + i] = sbe[i] * gam * srk[i];
      rec[kRecBe + i] = sbe[i];
      if (i == kL - 1) rec[kRecGl] = gam;
    }
    if (i == kL - 1) rec[kRecSrs + j] = srk[j] * dc;
  }
  __syncthreads();

  // T = (I + Ls)^-1, one lane per column
  if (tid < kL) {
    float x[kL];
#pragma unroll
    for (int r = 0; r < kL; ++r) {
      float acc[4] = {r == tid ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < r; ++m) acc[m % 4] = fmaf(-sLs[r][m], x[m], acc[m % 4]);
      x[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
#pragma unroll
    for (int r = 0; r < kL; ++r) rec[kRecT + 16 * r + tid] = x[r];
  }
}

// ---------------------------------------------------------------------------
// The sequential part: products with the state, block after block.

struct StateArgs {
  const void *q, *k, *v, *z, *w;
  const float* rec;
  const float* s0;
  float* y;
  float* s_out;
  int64_t T, nblk;
  int Hk, Hv, G, nrb, head_major;
  float norm_eps;
};

// Workgroup = (value head, NA a-tiles of 16 value rows); NC waves share an
// a-tile by splitting its 8 key tiles (their partial products are summed
// through LDS).  NW = NA * NC waves.
template <int DT, int NA, int NC, bool FUSE>
__global__ __launch_bounds__(NA* NC* kWave)
__attribute__((amdgpu_waves_per_eu(NA * NC >= 8 ? 4 : 1))) void state_kernel(StateArgs a) {
  constexpr int NW = NA * NC, NT = NW * kWave, ROWS = 16 * NA, NCT = 8 / NC;
  static_assert(NT >= 256 && NW <= 8 && NC >= 1 && 8 % NC == 0, "shape");
  static_assert(!FUSE || ROWS == kD, "the fused norm needs the whole head");
  __shared__ __align__(16) float sk[kL][kPad];
  __shared__ __align__(16) float sq[kL][kPad];
  __shared__ float sv[kL][ROWS];
  __shared__ float sz[FUSE ? 2 : 1][FUSE ? kL : 1][FUSE ? kD : 1];
  __shared__ __align__(16) float so[kL][ROWS];
  __shared__ __align__(16) float srec[kRecUsed];
  __shared__ v4f spart[NC > 1 ? NW : 1][2][kWave];

  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int rb = (int)(tile % a.nrb);
  const int64_t bh = tile / a.nrb;
  const int hv = (int)(bh % a.Hv), hk = hv / a.G;
  const int64_t b = bh / a.Hv;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int lg = lane / 16, lc = lane % 16;
  const int ai = wave / NC, cp = wave % NC;  // this wave's a-tile and key-tile part
  const int64_t T = a.T;
  const bool has_z = FUSE && a.z != nullptr;
  const Bases bs = head_bases(b, hv, hk, a.Hk, a.Hv, T, a.head_major);
  const int row0 = rb * ROWS;
  const int64_t sbase = (b * a.Hv + hv) * (int64_t)(kD * kD);
  const float* rec = a.rec + record_at(bh, 0, a.nblk);

  // staging of one block: 512 items of 8 q or k elements, v pairs, z pairs
  // (fused), the record as float4
  constexpr int NQK = (2 * kL * 16 + NT - 1) / NT;
  constexpr int NVP = (kL * ROWS / 2 + NT - 1) / NT;
  constexpr int NZP = FUSE ? (kL * kD / 2 + NT - 1) / NT : 1;
  constexpr int NR4 = kRecUsed / 4;
  constexpr int NRC = (NR4 + NT - 1) / NT;
  struct Regs {
    Raw<DT, 8> qk[NQK];
    Raw<DT, 2> v[NVP];
    Raw<DT, 2> z[NZP];
    Raw<GDN_F32, 4> r[NRC];
  };
  auto chunk_load = [&](Regs& P, int64_t c, int tc) {
    const int64_t t0 = c * kL;
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int e = tid + i * NT, which = e / 256, it = e % 256, tt = it / 16, c8 = it % 16;
      if (e < 512 && tt < tc) P.qk[i].load(which ? a.q : a.k, bs.qk + (t0 + tt) * bs.qk_ts + 8 * c8);
      else P.qk[i].zero();
    }
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int e = tid + i * NT, tt = e / (ROWS / 2), r2 = e % (ROWS / 2);
      if (e < kL * ROWS / 2 && tt < tc) P.v[i].load(a.v, bs.v + (t0 + tt) * bs.v_ts + row0 + 2 * r2);
    }
    if constexpr (FUSE) {
#pragma unroll
      for (int i = 0; i < NZP; ++i) {
        const int e = tid + i * NT, tt = e / (kD / 2), r2 = e % (kD / 2);
        if (has_z && e < kL * kD / 2 && tt < tc)
          P.z[i].load(a.z, bs.v + (t0 + tt) * bs.v_ts + 2 * r2);
      }
    }
#pragma unroll
    for (int i = 0; i < NRC; ++i) {  // every lane loads (clamped): no branch around the load
      const int e = tid + i * NT < NR4 ? tid + i * NT : NR4 - 1;
      P.r[i].load(rec, c * kRec + 4 * e);
    }
  };
  auto chunk_store = [&](const Regs& P, int tc, int zbuf) {
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): the block's loads are complete
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int e = tid + i * NT, which = e / 256, it = e % 256, tt = it / 16, c8 = it % 16;
      if (e < 512) {
        float* dst = which ? &sq[tt][8 * c8] : &sk[tt][8 * c8];
        *reinterpret_cast<float4*>(dst) = P.qk[i].get4(0);
        *reinterpret_cast<float4*>(dst + 4) = P.qk[i].get4(1);
      }
    }
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int e = tid + i * NT, tt = e / (ROWS / 2), r2 = e % (ROWS / 2);
      if (e < kL * ROWS / 2) {
        sv[tt][2 * r2] = tt < tc ? P.v[i].get(0) : 0.f;
        sv[tt][2 * r2 + 1] = tt < tc ? P.v[i].get(1) : 0.f;
      }
    }
    if constexpr (FUSE) {
#pragma unroll
      for (int i = 0; i < NZP; ++i) {
        const int e = tid + i * NT, tt = e / (kD / 2), r2 = e % (kD / 2);
        if (has_z && e < kL * kD / 2 && tt < tc) {
          sz[zbuf][tt][2 * r2] = P.z[i].get(0);
          sz[zbuf][tt][2 * r2 + 1] = P.z[i].get(1);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NRC; ++i) {
      const int e = tid + i * NT;
      if (e < NR4) *reinterpret_cast<float4*>(&srec[4 * e]) = P.r[i].get4(0);
    }
  };

  // state S^T, this wave's key tiles of its a-tile, in the accumulator layout
  v4f St[NCT];
  const int arow = row0 + 16 * ai + lc;  // value row of this lane
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const float4 x = *reinterpret_cast<const float4*>(a.s0 + sbase + (int64_t)arow * kD +
                                                      16 * (cp * NCT + ct) + 4 * lg);
    St[ct] = v4f{x.x, x.y, x.z, x.w};
  }
  float wgt[2];
  if constexpr (FUSE) {
#pragma unroll
    for (int i = 0; i < 2; ++i) wgt[i] = has_z ? ld1<DT>(a.w, lane + kWave * i) : 0.f;
  }

  Regs P;
  chunk_load(P, 0, (int)(T < kL ? T : kL));
  chunk_store(P, (int)(T < kL ? T : kL), 0);

  for (int64_t c = 0;; ++c) {
    const int64_t t0 = c * kL;
    const int tc = (int)((T - t0) < kL ? (T - t0) : kL);
    const bool more = c + 1 < a.nblk;
    const int tcn = more ? (int)((T - t0 - kL) < kL ? (T - t0 - kL) : kL) : 0;
    __syncthreads();
    if (more) chunk_load(P, c + 1, tcn);

    // K S^T and Q S^T over this wave's key tiles (raw k and q)
    v4f pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int kt = cp * NCT + ct;
      const float4 kf = *reinterpret_cast<const float4*>(&sk[lc][16 * kt + 4 * lg]);
      const float4 qf = *reinterpret_cast<const float4*>(&sq[lc][16 * kt + 4 * lg]);
      pk = mfma4(kf.x, St[ct][0], pk);
      pq = mfma4(qf.x, St[ct][0], pq);
      pk = mfma4(kf.y, St[ct][1], pk);
      pq = mfma4(qf.y, St[ct][1], pq);
      pk = mfma4(kf.z, St[ct][2], pk);
      pq = mfma4(qf.z, St[ct][2], pq);
      pk = mfma4(kf.w, St[ct][3], pk);
      pq = mfma4(qf.w, St[ct][3], pq);
    }
    if constexpr (NC > 1) {
      spart[wave][0][lane] = pk;
      spart[wave][1][lane] = pq;
      __syncthreads();
      pk = spart[ai * NC][0][lane];
      pq = spart[ai * NC][1][lane];
#pragma unroll
      for (int p = 1; p < NC; ++p) {
        pk += spart[ai * NC + p][0][lane];
        pq += spart[ai * NC + p][1][lane];
      }
    }
    // C = T (diag(beta) V - diag(beta gam rk) K S^T)  (rows: tokens, columns:
    // this a-tile's value rows)
    v4f yv;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      yv[r] = srec[kRecBe + 4 * lg + r] * sv[4 * lg + r][16 * ai + lc] -
              srec[kRecWsc + 4 * lg + r] * pk[r];
    v4f cc = {0.f, 0.f, 0.f, 0.f};
    {
      const float4 tf = *reinterpret_cast<const float4*>(&srec[kRecT + 16 * lc + 4 * lg]);
      cc = mfma4(tf.x, yv[0], cc);
      cc = mfma4(tf.y, yv[1], cc);
      cc = mfma4(tf.z, yv[2], cc);
      cc = mfma4(tf.w, yv[3], cc);
    }
    // S^T = gam_15 S^T + (diag(rk Dc[15][.]) K)^T C
    const float gl = srec[kRecGl];
    float rsl[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) rsl[s2] = srec[kRecSrs + 4 * lg + s2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int kc = 16 * (cp * NCT + ct) + lc;
      v4f acc = St[ct] * gl;
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) acc = mfma4(sk[4 * lg + s2][kc] * rsl[s2], cc[s2], acc);
      St[ct] = acc;
    }
    // O = diag(gam rq) Q S^T + Hd C
    if (cp == 0) {
      v4f o = {0.f, 0.f, 0.f, 0.f};
      const float4 hf = *reinterpret_cast<const float4*>(&srec[kRecH + 16 * lc + 4 * lg]);
      o = mfma4(hf.x, cc[0], o);
      o = mfma4(hf.y, cc[1], o);
      o = mfma4(hf.z, cc[2], o);
      o = mfma4(hf.w, cc[3], o);
      const float4 sg = *reinterpret_cast<const float4*>(&srec[kRecSig + 4 * lg]);
      so[4 * lg + 0][16 * ai + lc] = fmaf(sg.x, pq[0], o[0]);
      so[4 * lg + 1][16 * ai + lc] = fmaf(sg.y, pq[1], o[1]);
      so[4 * lg + 2][16 * ai + lc] = fmaf(sg.z, pq[2], o[2]);
      so[4 * lg + 3][16 * ai + lc] = fmaf(sg.w, pq[3], o[3]);
    }
    __syncthreads();

    // next block into LDS (every block array was last read above); z is
    // double-buffered because the output below reads this block's slot
    chunk_store(P, tcn, (int)((c + 1) & 1));

    // ---- outputs of this block
    if constexpr (FUSE) {
      if (has_z) {
        constexpr int TPW = (kL + NW - 1) / NW;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          const int tt = wave + NW * u;
          if (tt < kL) {  // uniform per wave
            const int zb = (int)(c & 1);
            float x0 = so[tt][lane] * silu(sz[zb][tt][lane]);
            float x1 = so[tt][lane + kWave] * silu(sz[zb][tt][lane + kWave]);
            const float inv = rsqrtf(wave_sum(fmaf(x0, x0, x1 * x1)) * (1.0f / kD) + a.norm_eps);
            if (tt < tc) {
              const int64_t vo = bs.v + (t0 + tt) * bs.v_ts;
              a.y[vo + lane] = x0 * inv * wgt[0];
              a.y[vo + lane + kWave] = x1 * inv * wgt[1];
            }
          }
        }
      } else {
        for (int e = tid; e < tc * (kD / 4); e += NT) {
          const int tt = e / (kD / 4), r4 = e % (kD / 4);
          *reinterpret_cast<float4*>(a.y + bs.v + (t0 + tt) * bs.v_ts + 4 * r4) =
              *reinterpret_cast<const float4*>(&so[tt][4 * r4]);
        }
      }
    } else {
      constexpr int R4 = ROWS / 4;
      for (int e = tid; e < tc * R4; e += NT) {
        const int tt = e / R4, r4 = e % R4;
        *reinterpret_cast<float4*>(a.y + bs.v + (t0 + tt) * bs.v_ts + row0 + 4 * r4) =
            *reinterpret_cast<const float4*>(&so[tt][4 * r4]);
      }
    }
    if (!more) break;
  }

#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    float4 x = make_float4(St[ct][0], St[ct][1], St[ct][2], St[ct][3]);
    *reinterpret_cast<float4*>(a.s_out + sbase + (int64_t)arow * kD + 16 * (cp * NCT + ct) +
                               4 * lg) = x;
  }
}

template <int DT, int NA, int NC>
int launch_state(StateArgs a, int64_t heads, hipStream_t st) {
  constexpr int ROWS = 16 * NA;
  a.nrb = kD / ROWS;
  const dim3 grid((unsigned)(heads * a.nrb));
  if constexpr (ROWS == kD) {
    state_kernel<DT, NA, NC, true><<<grid, NA * NC * kWave, 0, st>>>(a);
  } else {
    state_kernel<DT, NA, NC, false><<<grid, NA * NC * kWave, 0, st>>>(a);
  }
  return device_status("state_kernel launch");
}

template <int DT>
int launch_prep(const PrepArgs& p, int gdt, dim3 grid, hipStream_t st) {
  switch (gdt) {
    case GDN_F32: prep_kernel<DT, GDN_F32><<<grid, 256, 0, st>>>(p); break;
    case GDN_F16: prep_kernel<DT, GDN_F16><<<grid, 256, 0, st>>>(p); break;
    default: prep_kernel<DT, GDN_BF16><<<grid, 256, 0, st>>>(p); break;
  }
  return device_status("prep_kernel launch");
}

template <int DT>
int launch_dt(const gdn_desc& d, const PrepArgs& p, const StateArgs& s, int64_t heads,
              hipStream_t st) {
  const dim3 pgrid((unsigned)(heads * p.nblk));
  const int rc = launch_prep<DT>(p, d.gate_dtype, pgrid, st);
  if (rc != GDN_OK) return rc;
  if (heads >= 256) return launch_state<DT, 8, 1>(s, heads, st);
  return launch_state<DT, 1, 4>(s, heads, st);
}

int64_t block_record_bytes(int64_t heads, int64_t T) {
  return heads * ((T + kL - 1) / kL) * (int64_t)kRec * (int64_t)sizeof(float);
}

}  // namespace

// The block-form scan for D == 128; y receives the raw o (the gated norm, when
// asked for and not fused, runs after it).  Returns whether the gated output
// was written (fused) through *gated.  The block records live in a
// stream-ordered allocation released on the same stream after the scan.
int launch_scan_chunked(const gdn_desc& d, const void* q, const void* k, const void* v,
                        const void* ld, const void* beta, const float* s0, const void* z,
                        const void* w, float* y, float* s_out, void* stream, bool* gated) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t heads = d.B * d.Hv, nblk = (d.T + kL - 1) / kL;
  *gated = heads >= 256;
  void* ws = nullptr;
  if (hipMallocAsync(&ws, (size_t)block_record_bytes(heads, d.T), st) != hipSuccess) {
    (void)hipGetLastError();
    set_error("gdn_scan: no device memory for the block records");
    return GDN_EDEVICE;
  }
  float* rec = static_cast<float*>(ws);
  const PrepArgs p{q, k, ld, beta, rec, d.T, nblk, (int)d.Hk, (int)d.Hv, (int)(d.Hv / d.Hk),
                   d.head_major, d.flags, d.qk_eps, q_scale(d)};
  const StateArgs s{q, k, v, z, w, rec, s0, y, s_out, d.T, nblk, (int)d.Hk, (int)d.Hv,
                    (int)(d.Hv / d.Hk), 1, d.head_major, d.norm_eps};
  int rc;
  switch (d.dtype) {
    case GDN_F32: rc = launch_dt<GDN_F32>(d, p, s, heads, st); break;
    case GDN_F16: rc = launch_dt<GDN_F16>(d, p, s, heads, st); break;
    default: rc = launch_dt<GDN_BF16>(d, p, s, heads, st); break;
  }
  const hipError_t fe = hipFreeAsync(ws, st);
  if (rc == GDN_OK && fe != hipSuccess) return device_status("gdn_scan: releasing the block records");
  return rc;
}

}  // namespace gdn

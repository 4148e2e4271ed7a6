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
//   prep_kernel  (one wave per key head and block, all in parallel): the
//                norms, decay products, K K^T and Q K^T on the matrix cores,
//                T = (I + Ls)^-1 by forward substitution and the masked
//                Hd = tril(Q^ K^^T) (.) Dc, written as a small block record;
//   state_kernel / rows_ws_kernel (sequential over the blocks; a workgroup
//                per head when there are many heads, per 16 value rows when
//                there are few): P = K S^T and Q S^T, C = T (diag(beta) V -
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
  int64_t T, nblk, ntask;  // ntask = B * Hk * nblk
  int Hk, Hv, G, head_major;
  uint32_t flags;
  float qk_eps, qscale;
};

// One wave per (batch, key head, block): K K^T and Q K^T once, then the
// records of the G value heads that share the key head (four at a time, one
// per 16-lane group).  No workgroup barrier: each wave owns its LDS slice.
template <int DT, int GT>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  __shared__ float sLs[4][4][kL][kL + 1];  // [wave][value head of the group][i][j]
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int lg = lane / 16, lc = lane % 16;
  const int64_t task = (int64_t)blockIdx.x * 4 + wave;
  if (task >= a.ntask) return;  // uniform per wave
  const int64_t c = task % a.nblk, bk = task / a.nblk;
  const int hk = (int)(bk % a.Hk);
  const int64_t b = bk / a.Hk, T = a.T, t0 = c * kL;
  const int tc = (int)((T - t0) < kL ? (T - t0) : kL);
  int64_t qk_base, qk_ts;
  if (a.head_major) {
    qk_base = (b * a.Hk + hk) * T * kD; qk_ts = kD;
  } else {
    qk_base = (b * T * a.Hk + hk) * kD; qk_ts = (int64_t)a.Hk * kD;
  }

  // rows of q and k: lane (lg, lc) holds row lc, elements [32 lg, 32 lg + 32)
  Raw<DT, 8> kr[4], qr[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (lc < tc) {
      kr[u].load(a.k, qk_base + (t0 + lc) * qk_ts + 32 * lg + 8 * u);
      qr[u].load(a.q, qk_base + (t0 + lc) * qk_ts + 32 * lg + 8 * u);
    } else {
      kr[u].zero();
      qr[u].zero();
    }
  }
  float ssk = 0.f, ssq = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ssk = fmaf(kr[u].get(e), kr[u].get(e), ssk);
      ssq = fmaf(qr[u].get(e), qr[u].get(e), ssq);
    }
  ssk += __shfl_xor(ssk, 16);
  ssk += __shfl_xor(ssk, 32);
  ssq += __shfl_xor(ssq, 16);
  ssq += __shfl_xor(ssq, 32);
  const bool l2 = (a.flags & GDN_FOLD_QK_L2NORM) != 0;
  float rk = rsqrtf(l2 ? ssk + a.qk_eps : 1.f);          // of row lc
  float rq = rsqrtf(l2 ? ssq + a.qk_eps : 1.f) * a.qscale;
  if (lc >= tc) rk = rq = 0.f;

  // G = K K^T and H = Q K^T (raw) on the matrix cores; product m contracts
  // key index 32 lg + m.  Lane (lg, lc), register r: entry [4 lg + r][lc].
  v4f G4 = {0.f, 0.f, 0.f, 0.f}, H4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float kv = kr[u].get(e);
      G4 = mfma4(kv, kv, G4);
      H4 = mfma4(qr[u].get(e), kv, H4);
    }
  float rki[4], rqi[4];  // norms of the lane's rows i = 4 lg + r
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    rki[r] = __shfl(rk, 4 * lg + r);
    rqi[r] = __shfl(rq, 4 * lg + r);
  }

  for (int g0 = 0; g0 < a.G; g0 += 4) {
    // gates: lane (lg, lc) loads token lc of value head g0 + lg
    const int g = g0 + lg, hv = hk * a.G + g;
    const bool gv = g < a.G;
    float al = 1.f, be = 0.f;
    if (gv && lc < tc) {
      const int64_t gi = a.head_major ? (b * a.Hv + hv) * T + t0 + lc
                                      : (b * T + t0 + lc) * a.Hv + hv;
      Raw<GT, 1> l1, b1;
      l1.load(a.ld, gi);
      b1.load(a.beta, gi);
      al = expf(l1.get(0));
      be = b1.get(0);
    }
    // decay products of token lc of each 16-lane row's value head: from the
    // block start through lc, and after lc to the block end
    const float gam = row_prefix_prod(al), tail = dpp_or_one<0x101, 0xF>(row_suffix_prod(al));
    const int ng = a.G - g0 < 4 ? a.G - g0 : 4;
    for (int gq = 0; gq < ng; ++gq) {  // Ls and Hd of value head g0 + gq, all lanes
      float als[kL];
#pragma unroll
      for (int m = 0; m < kL; ++m)
        als[m] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 16 * gq + m));
      float* rec = a.rec + record_at(b * a.Hv + hk * a.G + g0 + gq, c, a.nblk);
      // Dc[i][j] for j = lc and the rows i = 4 lg .. 4 lg + 3: the product up to
      // row 4 lg, then one decay per row
      const int j = lc;
      float dc = j <= 4 * lg ? 1.f : 0.f;
#pragma unroll
      for (int m = 1; m < kL; ++m) dc *= (m > j && m <= 4 * lg) ? als[m] : 1.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * lg + r;
        if (r > 0) {
          const float ai = lg == 0 ? als[r] : lg == 1 ? als[4 + r] : lg == 2 ? als[8 + r] : als[12 + r];
          dc = j < i ? dc * ai : (j == i ? 1.f : 0.f);
        }
        const float bei = __shfl(be, 16 * gq + i);
        sLs[wave][gq][i][j] = j < i ? bei * rki[r] * G4[r] * rk * dc : 0.f;
        rec[kRecH + 16 * i + j] = j <= i ? rqi[r] * H4[r] * rk * dc : 0.f;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (gv) {  // lane group lg: value head g; lane lc: token lc and column lc
      float* rec = a.rec + record_at(b * a.Hv + hv, c, a.nblk);
      rec[kRecSig + lc] = gam * rq;
      rec[kRecWsc + lc] = be * gam * rk;
      rec[kRecBe + lc] = be;
      rec[kRecSrs + lc] = rk * tail;
      if (lc == kL - 1) rec[kRecGl] = gam;
      // column lc of T = (I + Ls)^-1 by forward substitution
      float x[kL];
#pragma unroll
      for (int r = 0; r < kL; ++r) {
        float acc[4] = {r == lc ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < r; ++m) acc[m % 4] = fmaf(-sLs[wave][lg][r][m], x[m], acc[m % 4]);
        x[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      }
#pragma unroll
      for (int r = 0; r < kL; ++r) rec[kRecT + 16 * r + lc] = x[r];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

// The many-head shape: one workgroup per value head, its 8 waves one a-tile
// (16 value rows) each over all 8 key tiles, two workgroups per CU; the gated
// norm is fused.  The loads of block c + 1 are issued while block c is
// computed.
template <int DT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void state_kernel(
    StateArgs a) {
  constexpr int NW = 8, NT = NW * kWave, ROWS = kD, NCT = 8;
  __shared__ __align__(16) float sk[kL][kPad];
  __shared__ __align__(16) float sq[kL][kPad];
  __shared__ float sv[kL][ROWS];
  __shared__ float sz[2][kL][kD];
  __shared__ __align__(16) float so[2][kL][ROWS];
  __shared__ __align__(16) float srec[kRecUsed];

  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t bh = tile;
  const int hv = (int)(bh % a.Hv), hk = hv / a.G;
  const int64_t b = bh / a.Hv;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int lg = lane / 16, lc = lane % 16;
  const int ai = wave;  // this wave's a-tile (value rows 16 ai ..), all key tiles
  const int64_t T = a.T;
  const bool has_z = a.z != nullptr;
  const Bases bs = head_bases(b, hv, hk, a.Hk, a.Hv, T, a.head_major);
  const int64_t sbase = (b * a.Hv + hv) * (int64_t)(kD * kD);
  const float* rec = a.rec + record_at(bh, 0, a.nblk);

  // staging of one block: 512 items of 8 q or k elements, v pairs, z pairs
  // (fused), the record as float4
  constexpr int NQK = (2 * kL * 16 + NT - 1) / NT;
  constexpr int NVP = (kL * ROWS / 2 + NT - 1) / NT;
  constexpr int NZP = (kL * kD / 2 + NT - 1) / NT;
  constexpr int NR4 = kRecUsed / 4;
  constexpr int NRC = (NR4 + NT - 1) / NT;
  struct Regs {
    Raw<DT, 8> qk[NQK];
    Raw<DT, 2> v[NVP];
    Raw<DT, 2> z[NZP];
    Raw<GDN_F32, 4> r[NRC];
  };
  // Every lane issues every load of a block (token and item indices clamped
  // into range; the excess is zeroed or dropped when the block is written to
  // LDS), so no branch skips a load.
  auto clamp_t = [&](int tt, int tc) { return tt < tc ? tt : tc - 1; };
  auto chunk_load = [&](Regs& P, int64_t c, int tc) {
    const int64_t t0 = c * kL;
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int e = (tid + i * NT) % 512, which = e / 256, it = e % 256, tt = it / 16, c8 = it % 16;
      P.qk[i].load(which ? a.q : a.k, bs.qk + (t0 + clamp_t(tt, tc)) * bs.qk_ts + 8 * c8);
    }
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int e = (tid + i * NT) % (kL * ROWS / 2), tt = e / (ROWS / 2), r2 = e % (ROWS / 2);
      P.v[i].load(a.v, bs.v + (t0 + clamp_t(tt, tc)) * bs.v_ts + 2 * r2);
    }
    if (has_z) {
#pragma unroll
      for (int i = 0; i < NZP; ++i) {
        const int e = (tid + i * NT) % (kL * kD / 2), tt = e / (kD / 2), r2 = e % (kD / 2);
        P.z[i].load(a.z, bs.v + (t0 + clamp_t(tt, tc)) * bs.v_ts + 2 * r2);
      }
    }
#pragma unroll
    for (int i = 0; i < NRC; ++i) {
      const int e = tid + i * NT < NR4 ? tid + i * NT : NR4 - 1;
      P.r[i].load(rec, c * kRec + 4 * e);
    }
  };
  // Every lane also writes every item it loaded (lanes past the item count
  // repeat an item with the same value), so no path leaves a load unread.
  // Rows past the last token repeat its inputs; the block record gives them
  // beta = rk = rq = 0, so they add nothing to C, O or the state.
  auto chunk_store = [&](const Regs& P, int zbuf) {
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int e = (tid + i * NT) % 512, which = e / 256, it = e % 256, tt = it / 16, c8 = it % 16;
      float* dst = which ? &sq[tt][8 * c8] : &sk[tt][8 * c8];
      *reinterpret_cast<float4*>(dst) = P.qk[i].get4(0);
      *reinterpret_cast<float4*>(dst + 4) = P.qk[i].get4(1);
    }
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int e = (tid + i * NT) % (kL * ROWS / 2), tt = e / (ROWS / 2), r2 = e % (ROWS / 2);
      sv[tt][2 * r2] = P.v[i].get(0);
      sv[tt][2 * r2 + 1] = P.v[i].get(1);
    }
    if (has_z) {
#pragma unroll
      for (int i = 0; i < NZP; ++i) {
        const int e = (tid + i * NT) % (kL * kD / 2), tt = e / (kD / 2), r2 = e % (kD / 2);
        sz[zbuf][tt][2 * r2] = P.z[i].get(0);
        sz[zbuf][tt][2 * r2 + 1] = P.z[i].get(1);
      }
    }
#pragma unroll
    for (int i = 0; i < NRC; ++i) {
      const int e = tid + i * NT < NR4 ? tid + i * NT : NR4 - 1;
      *reinterpret_cast<float4*>(&srec[4 * e]) = P.r[i].get4(0);
    }
  };

  // state S^T, this wave's key tiles of its a-tile, in the accumulator layout
  v4f St[NCT];
  const int arow = 16 * ai + lc;  // value row of this lane
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const float4 x = *reinterpret_cast<const float4*>(a.s0 + sbase + (int64_t)arow * kD +
                                                      16 * ct + 4 * lg);
    St[ct] = v4f{x.x, x.y, x.z, x.w};
  }
  float wgt[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) wgt[i] = has_z ? ld1<DT>(a.w, lane + kWave * i) : 0.f;
  const int64_t nblk = a.nblk;
  auto tc_of = [&](int64_t c) { return (int)((T - c * kL) < kL ? (T - c * kL) : kL); };

  // Outputs of block c from LDS (a fixed number of stores per lane).  They
  // run after the top barrier of the next block, before its loads, so the
  // waits on those loads never have to cover these stores.
  auto outputs = [&](int64_t c) {
    const int64_t t0 = c * kL;
    const int tc = tc_of(c);
    if (has_z) {  // the gated norm: two tokens per wave, 128 values each
#pragma unroll
      for (int u = 0; u < kL / NW; ++u) {
        const int tt = wave + NW * u, zb = (int)(c & 1);
        float x0 = so[c & 1][tt][lane] * silu(sz[zb][tt][lane]);
        float x1 = so[c & 1][tt][lane + kWave] * silu(sz[zb][tt][lane + kWave]);
        const float inv = rsqrtf(wave_sum(fmaf(x0, x0, x1 * x1)) * (1.0f / kD) + a.norm_eps);
        if (tt < tc) {
          const int64_t vo = bs.v + (t0 + tt) * bs.v_ts;
          a.y[vo + lane] = x0 * inv * wgt[0];
          a.y[vo + lane + kWave] = x1 * inv * wgt[1];
        }
      }
      return;
    }
    constexpr int R4 = ROWS / 4, NO = (kL * R4 + NT - 1) / NT;
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int e = tid + u * NT, tt = e / R4, r4 = e % R4;
      if (e < kL * R4 && tt < tc)
        *reinterpret_cast<float4*>(a.y + bs.v + (t0 + tt) * bs.v_ts + 4 * r4) =
            *reinterpret_cast<const float4*>(&so[c & 1][tt][4 * r4]);
    }
  };

  // One block: LDS holds block c; the loads of block c + 1 go into P (issued
  // first) and reach LDS after the block's last LDS read.
  // Loads and LDS writes run unconditionally (past the end they repeat the
  // last block), so every path through the loop leaves the same loads in
  // flight and the waits before the LDS writes only cover the older block.
  auto step = [&](int64_t c, Regs& P) {
    const int64_t cl = c + 1 < nblk ? c + 1 : nblk - 1;
    __syncthreads();
    if (c > 0) outputs(c - 1);
    chunk_load(P, cl, tc_of(cl));

    // K S^T then Q S^T over this wave's key tiles (raw k and q); K S^T first:
    // only it is on the chain to the next block
    v4f pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float4 kf = *reinterpret_cast<const float4*>(&sk[lc][16 * ct + 4 * lg]);
      pk = mfma4(kf.x, St[ct][0], pk);
      pk = mfma4(kf.y, St[ct][1], pk);
      pk = mfma4(kf.z, St[ct][2], pk);
      pk = mfma4(kf.w, St[ct][3], pk);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float4 qf = *reinterpret_cast<const float4*>(&sq[lc][16 * ct + 4 * lg]);
      pq = mfma4(qf.x, St[ct][0], pq);
      pq = mfma4(qf.y, St[ct][1], pq);
      pq = mfma4(qf.z, St[ct][2], pq);
      pq = mfma4(qf.w, St[ct][3], pq);
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
    // S^T = gam_15 S^T + K^T diag(rk Dc[15][.]) C: the key scales on C's rows
    // (4 products per lane) rather than on K (4 per key tile)
    const float gl = srec[kRecGl];
    v4f cs;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) cs[s2] = cc[s2] * srec[kRecSrs + 4 * lg + s2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int kc = 16 * ct + lc;
      v4f acc = St[ct] * gl;
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) acc = mfma4(sk[4 * lg + s2][kc], cs[s2], acc);
      St[ct] = acc;
    }
    // O = diag(gam rq) Q S^T + Hd C
    {
      const float4 hf = *reinterpret_cast<const float4*>(&srec[kRecH + 16 * lc + 4 * lg]);
      const float4 sg = *reinterpret_cast<const float4*>(&srec[kRecSig + 4 * lg]);
      v4f o = {0.f, 0.f, 0.f, 0.f};
      o = mfma4(hf.x, cc[0], o);
      o = mfma4(hf.y, cc[1], o);
      o = mfma4(hf.z, cc[2], o);
      o = mfma4(hf.w, cc[3], o);
      so[c & 1][4 * lg + 0][16 * ai + lc] = fmaf(sg.x, pq[0], o[0]);
      so[c & 1][4 * lg + 1][16 * ai + lc] = fmaf(sg.y, pq[1], o[1]);
      so[c & 1][4 * lg + 2][16 * ai + lc] = fmaf(sg.z, pq[2], o[2]);
      so[c & 1][4 * lg + 3][16 * ai + lc] = fmaf(sg.w, pq[3], o[3]);
    }
    __syncthreads();

    // next block into LDS (every block array was last read above); z and o
    // are double-buffered: the outputs of this block are written at the
    // start of the next one
    chunk_store(P, (int)((c + 1) & 1));

  };

  Regs P;
  chunk_load(P, 0, tc_of(0));
  chunk_store(P, 0);
  for (int64_t c = 0; c < nblk; ++c) step(c, P);
  __syncthreads();
  outputs(nblk - 1);

#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    float4 x = make_float4(St[ct][0], St[ct][1], St[ct][2], St[ct][3]);
    *reinterpret_cast<float4*>(a.s_out + sbase + (int64_t)arow * kD + 16 * ct +
                               4 * lg) = x;
  }
}

// The few-head shape with two waves per SIMD in different roles.  Waves 0-3
// ("chain" waves, one per SIMD) hold the state, two key tiles each, and run
// only the products with it: K S^T, its sum over the four waves, C, the
// update, and Q S^T.  Waves 4-7 ("helper" waves, one per SIMD) move the data:
// they load the blocks two ahead, write them to LDS, form O of the previous
// block (from the C the first chain wave leaves in LDS, one product per
// helper) and store y.  On every SIMD the helper's vector and memory work then
// overlaps the chain wave's matrix-core work.  Two barriers per block, taken
// by all waves.
template <int DT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void rows_ws_kernel(
    StateArgs a) {
  constexpr int NC = 4, NCT = 8 / NC, ROWS = 16, HT = NC * kWave;
  __shared__ __align__(16) float sk[2][kL][kPad];
  __shared__ __align__(16) float sq[2][kL][kPad];
  __shared__ __align__(16) float sv[2][kL][ROWS];
  __shared__ __align__(16) float srec[2][kRecUsed];
  __shared__ __align__(16) float scc[2][kL][ROWS];  // C of a block, for its O
  __shared__ v4f sop[2][NC][kWave];  // O of a block: one part per helper
  __shared__ v4f spart[NC][3][kWave];  // [chain wave][K S^T | Q S^T of even | odd blocks][lane]

  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int rb = (int)(tile % a.nrb);
  const int64_t bh = tile / a.nrb;
  const int hv = (int)(bh % a.Hv), hk = hv / a.G;
  const int64_t b = bh / a.Hv;
  // the wave index through readfirstlane: the compiler then treats the role
  // branches as uniform (no exec-mask merge of the two roles' registers)
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const bool chain = wave < NC;
  const int cp = wave % NC;      // chain: key-tile part; helper: helper index
  const int ht = tid - HT;       // helper thread index (helpers only)
  const int lg = lane / 16, lc = lane % 16;
  const int64_t T = a.T, nblk = a.nblk;
  const Bases bs = head_bases(b, hv, hk, a.Hk, a.Hv, T, a.head_major);
  const int row0 = rb * ROWS;
  const int64_t sbase = (b * a.Hv + hv) * (int64_t)(kD * kD);
  const float* rec = a.rec + record_at(bh, 0, nblk);
  auto tc_of = [&](int64_t c) { return (int)((T - c * kL) < kL ? (T - c * kL) : kL); };

  // ---- helpers: one block in registers (2 q/k items, a v pair, a record
  // float4 per helper lane; indices clamped, every lane loads and writes)
  constexpr int NR4 = kRecUsed / 4;
  struct Regs {
    Raw<DT, 8> qk[2];
    Raw<DT, 2> v;
    Raw<GDN_F32, 4> r;
  };
  const int qtt = (ht & (HT - 1)) / 16, qc8 = ht % 16;
  const int ve = (ht & (HT - 1)) % (kL * ROWS / 2), vtt = ve / (ROWS / 2), vr2 = ve % (ROWS / 2);
  const int tcl = tc_of(nblk - 1);
  const int64_t qk_blk = kL * bs.qk_ts, v_blk = kL * bs.v_ts;
  const int64_t qk_off = bs.qk + qtt * bs.qk_ts + 8 * qc8;
  const int64_t v_off = bs.v + vtt * bs.v_ts + row0 + 2 * vr2;
  const int64_t qk_last = bs.qk + (nblk - 1) * qk_blk + (qtt < tcl ? qtt : tcl - 1) * bs.qk_ts + 8 * qc8;
  const int64_t v_last = bs.v + (nblk - 1) * v_blk + (vtt < tcl ? vtt : tcl - 1) * bs.v_ts + row0 + 2 * vr2;
  const int rec_e = 4 * ((ht & (HT - 1)) < NR4 ? (ht & (HT - 1)) : NR4 - 1);
  auto chunk_load = [&](Regs& P, int64_t c) {
    const bool last = c == nblk - 1;
    const int64_t oq = last ? qk_last : qk_off + c * qk_blk;
    P.qk[0].load(a.k, oq);
    P.qk[1].load(a.q, oq);
    P.v.load(a.v, last ? v_last : v_off + c * v_blk);
    P.r.load(rec, c * kRec + rec_e);
  };
  auto chunk_store = [&](const Regs& P, int buf) {
    *reinterpret_cast<float4*>(&sk[buf][qtt][8 * qc8]) = P.qk[0].get4(0);
    *reinterpret_cast<float4*>(&sk[buf][qtt][8 * qc8 + 4]) = P.qk[0].get4(1);
    *reinterpret_cast<float4*>(&sq[buf][qtt][8 * qc8]) = P.qk[1].get4(0);
    *reinterpret_cast<float4*>(&sq[buf][qtt][8 * qc8 + 4]) = P.qk[1].get4(1);
    sv[buf][vtt][2 * vr2] = P.v.get(0);
    sv[buf][vtt][2 * vr2 + 1] = P.v.get(1);
    *reinterpret_cast<float4*>(&srec[buf][rec_e]) = P.r.get4(0);
  };
  // O of block cb = Hd C + diag(gam rq) Q S^T.  Before the block's second
  // barrier each helper h forms the part of Hd C over the tokens 4 i + h (one
  // product on its SIMD); after it, helper lane (t, j) sums the four parts and
  // the four Q S^T parts and stores y[t][j] (16 lanes write a token's values).
  const int ot = (ht & (HT - 1)) / 16, oj = ht % 16;
  const int pl = 4 * ((ot / 4) * 16 + oj) + ot % 4;  // element (ot, oj) of a part
  auto o_part = [&](int64_t cb) {  // before the barrier; returns gam_t rq_t of (ot, oj)
    const int ob = (int)(cb & 1);
    const float hd = srec[ob][kRecH + 16 * lc + 4 * lg + cp];
    const v4f o = mfma4(hd, scc[ob][4 * lg + cp][lc], v4f{0.f, 0.f, 0.f, 0.f});
    sop[ob][cp][lane] = o;
    return srec[ob][kRecSig + ot];
  };
  auto out_y = [&](int64_t cb, float sig) {  // after the barrier
    const int ob = (int)(cb & 1), sl = 1 + ob;
    float pqs = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NC; ++w) {
      pqs += reinterpret_cast<const float*>(&spart[w][sl][0])[pl];
      o += reinterpret_cast<const float*>(&sop[ob][w][0])[pl];
    }
    if (ot < tc_of(cb)) a.y[bs.v + (cb * kL + ot) * bs.v_ts + row0 + oj] = fmaf(sig, pqs, o);
  };

  // ---- chain waves: the state, two key tiles of the 16 rows, accumulator layout
  v4f St[NCT];
  const int arow = row0 + lc;
  if (chain) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float4 x = *reinterpret_cast<const float4*>(a.s0 + sbase + (int64_t)arow * kD +
                                                        16 * (cp * NCT + ct) + 4 * lg);
      St[ct] = v4f{x.x, x.y, x.z, x.w};
    }
  }

  // Each role runs its own loop; both take the same two barriers per block in
  // the same order, so the workgroup stays in step while each role's
  // registers (the state, the staged blocks) stay out of the other's code.
  const int64_t npair = nblk / 2;
  if (chain) {
    // block c: LDS buffer c & 1 holds it
    auto step = [&](int64_t c) {
      const int bf = (int)(c & 1);
      __syncthreads();
      v4f pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float4 kf = *reinterpret_cast<const float4*>(&sk[bf][lc][16 * (cp * NCT + ct) + 4 * lg]);
        pk = mfma4(kf.x, St[ct][0], pk);
        pk = mfma4(kf.y, St[ct][1], pk);
        pk = mfma4(kf.z, St[ct][2], pk);
        pk = mfma4(kf.w, St[ct][3], pk);
      }
      float bei[4], wsci[4], vi[4], srsi[4], ka[NCT][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bei[r] = srec[bf][kRecBe + 4 * lg + r];
        wsci[r] = srec[bf][kRecWsc + 4 * lg + r];
        srsi[r] = srec[bf][kRecSrs + 4 * lg + r];
        vi[r] = sv[bf][4 * lg + r][lc];
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
          ka[ct][s2] = sk[bf][4 * lg + s2][16 * (cp * NCT + ct) + lc];
      const float4 tf = *reinterpret_cast<const float4*>(&srec[bf][kRecT + 16 * lc + 4 * lg]);
      const float gl = srec[bf][kRecGl];
      spart[cp][0][lane] = pk;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float4 qf = *reinterpret_cast<const float4*>(&sq[bf][lc][16 * (cp * NCT + ct) + 4 * lg]);
        pq = mfma4(qf.x, St[ct][0], pq);
        pq = mfma4(qf.y, St[ct][1], pq);
        pq = mfma4(qf.z, St[ct][2], pq);
        pq = mfma4(qf.w, St[ct][3], pq);
      }
      __syncthreads();
      const v4f k0 = spart[0][0][lane], k1 = spart[1][0][lane];
      const v4f k2 = spart[2][0][lane], k3 = spart[3][0][lane];
      pk = (k0 + k1) + (k2 + k3);
      v4f yv;
#pragma unroll
      for (int r = 0; r < 4; ++r) yv[r] = bei[r] * vi[r] - wsci[r] * pk[r];
      v4f cc = {0.f, 0.f, 0.f, 0.f};
      cc = mfma4(tf.x, yv[0], cc);
      cc = mfma4(tf.y, yv[1], cc);
      cc = mfma4(tf.z, yv[2], cc);
      cc = mfma4(tf.w, yv[3], cc);
      v4f cs;  // C with the key scales of the update on its rows
#pragma unroll
      for (int r = 0; r < 4; ++r) cs[r] = cc[r] * srsi[r];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        v4f acc = St[ct] * gl;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = mfma4(ka[ct][s2], cs[s2], acc);
        St[ct] = acc;
      }
      spart[cp][1 + bf][lane] = pq;
      if (cp == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) scc[bf][4 * lg + r][lc] = cc[r];
      }
    };
    for (int64_t p = 0; p < npair; ++p) {
      step(2 * p);
      step(2 * p + 1);
    }
    if (nblk & 1) step(nblk - 1);
    __syncthreads();
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float4 x = make_float4(St[ct][0], St[ct][1], St[ct][2], St[ct][3]);
      *reinterpret_cast<float4*>(a.s_out + sbase + (int64_t)arow * kD + 16 * (cp * NCT + ct) +
                                 4 * lg) = x;
    }
  } else {
    // block c: the loads of block c + 2 go into Pl, O and y of block c - 1
    // are formed, Ps (block c + 1) reaches the other LDS buffer after the
    // block's second barrier
    auto step = [&](int64_t c, Regs& Pl, const Regs& Ps) {
      const int bf = (int)(c & 1);
      __syncthreads();
      chunk_load(Pl, c + 2 < nblk ? c + 2 : nblk - 1);
      const float sig = c >= 1 ? o_part(c - 1) : 0.f;
      __syncthreads();
      chunk_store(Ps, bf ^ 1);
      // y after the staging: the wait before the staging then never covers a
      // store issued in the same block
      if (c >= 1) out_y(c - 1, sig);
    };
    Regs P0, P1;
    chunk_load(P0, 0);
    chunk_load(P1, nblk > 1 ? 1 : 0);
    chunk_store(P0, 0);
    // nothing in flight on entry, and no exit inside the loop body: the
    // loop's own loads are then the only ones its waits have to count
    __builtin_amdgcn_s_waitcnt(0xF70);
    for (int64_t p = 0; p < npair; ++p) {
      step(2 * p, P0, P1);
      step(2 * p + 1, P1, P0);
    }
    if (nblk & 1) step(nblk - 1, P0, P1);
    __syncthreads();
    const float sig = o_part(nblk - 1);
    __syncthreads();
    out_y(nblk - 1, sig);
  }
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
  const dim3 pgrid((unsigned)((p.ntask + 3) / 4));
  const int rc = launch_prep<DT>(p, d.gate_dtype, pgrid, st);
  if (rc != GDN_OK) return rc;
  // many heads: whole-head workgroups, two per CU, the norm fused; few heads:
  // a workgroup per 16 value rows (rows_ws_kernel)
  StateArgs r = s;
  if (heads >= 256) {
    r.nrb = 1;
    state_kernel<DT><<<dim3((unsigned)heads), 512, 0, st>>>(r);
    return device_status("state_kernel launch");
  }
  r.nrb = kD / 16;
  rows_ws_kernel<DT><<<dim3((unsigned)(heads * r.nrb)), 512, 0, st>>>(r);
  return device_status("rows_ws_kernel launch");
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
  const PrepArgs p{q, k, ld, beta, rec, d.T, nblk, d.B * d.Hk * nblk, (int)d.Hk, (int)d.Hv,
                   (int)(d.Hv / d.Hk), d.head_major, d.flags, d.qk_eps, q_scale(d)};
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

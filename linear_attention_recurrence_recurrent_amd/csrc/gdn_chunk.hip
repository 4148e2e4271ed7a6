// Time-axis scan of the Gated DeltaNet recurrence in block form on the matrix
// cores (gfx950 MFMA, FP32 in and out), for D = 32, 64, 128 and 256.
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
//                Hd = tril(Q^ K^^T) (.) Dc, written as a small block record
//                (for few heads also K and Q products across blocks);
//   state_kernel (many heads, a workgroup per head) / rows_la_kernel (few
//                heads, a workgroup per 16 value rows; the products with S
//                taken one block ahead, off the sequential chain): P = K S^T
//                and Q S^T, C = T (diag(beta) V - diag(beta gam rk) P),
//                O = diag(gam rq) Q S^T + Hd C and the rank-16 update of S^T,
//                on raw q and k with the norms folded into per-token scales.
//                With f32 inputs these are v_mfma_f32_16x16x4f32 products.
//                With 16-bit inputs the products with the f32 state run on
//                the bf16 matrix cores over bf16 parts of the state and of
//                Cs: by default two parts rounded to nearest (split_bf2
//                below; each term within 2^-16 relative of the f32
//                product), with GDN_SCAN_EXACT three exact ones (split_bf3:
//                every term an exact f32 product, the sums differing from
//                f32 products only in their order); f16 q and k enter as two
//                exact bf16 parts, bf16 ones as they are.
// The sequential chain then holds only the products with S.  S^T stays in the
// accumulator layout for the whole time axis: lane l, register r of a 16 x 16
// tile holds S^T[4(l/16) + r][l%16] (key row within the tile, value column),
// which is also a valid B operand of the next product when the contraction
// index is taken in the matching order (the kernels with bf16 parts take a
// tile's keys in a permuted order, stated where they do).  Decays are
// products (never quotients), so alpha = 0 needs no special case.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kL = 16;        // tokens per block (the MFMA tile)
// (from kManyHeads value heads on, a workgroup per head fills the chip)

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

// 16x16x16 product of 16-bit operands (bf16 or f16), f32 accumulation: a lane
// holds 4 elements of the contraction index packed in a uint2.  The products
// of 16-bit values are exact in f32, so this equals the f32 product of the
// widened operands up to the order of the sums.
typedef short v4s16 __attribute__((ext_vector_type(4)));
typedef _Float16 v4h16 __attribute__((ext_vector_type(4)));
template <int DT>
__device__ __forceinline__ v4f mm16(uint2 a, uint2 b, v4f c = v4f{0.f, 0.f, 0.f, 0.f}) {
  if constexpr (DT == GDN_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4s16, a),
                                                      __builtin_bit_cast(v4s16, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4h16, a),
                                                  __builtin_bit_cast(v4h16, b), c, 0, 0, 0);
}

// 16x16x32 product of bf16 operands, f32 accumulation: a lane holds 8
// elements of the contraction index packed in a uint4, the same 8 for A's
// row and B's column.
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v4f mm32bf(uint4 a, uint4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf16, a),
                                                 __builtin_bit_cast(v8bf16, b), c, 0, 0, 0);
}

// An f32 value as the exact sum of three bf16 values.  hi keeps the top 8
// significant bits (truncation), the rest x - hi has at most 16 significant
// bits, its own truncation mid takes 8 of them and lo = x - hi - mid the last
// 8 or fewer, so lo is a bf16 value as it stands.  Both subtractions are
// exact.  (That holds for |x| >= 2^-110; below, lo reaches f32's subnormal
// range and its high half drops bits under 2^-133.)  With bf16 q and k the
// products against the three parts are exact in f32, so a state product
// through them is an f32 product up to the order of the sums.  Two values are
// packed per word, the first in the low half.
struct Bf3 {
  uint32_t h, m, l;
};
__device__ __forceinline__ Bf3 split_bf3(float x0, float x1) {
  const uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
  const float r0 = x0 - __uint_as_float(u0 & 0xffff0000u);
  const float r1 = x1 - __uint_as_float(u1 & 0xffff0000u);
  const uint32_t w0 = __float_as_uint(r0), w1 = __float_as_uint(r1);
  const uint32_t t0 = __float_as_uint(r0 - __uint_as_float(w0 & 0xffff0000u));
  const uint32_t t1 = __float_as_uint(r1 - __uint_as_float(w1 & 0xffff0000u));
  // the high halves of two words, the first word's in the low half
  return Bf3{__builtin_amdgcn_perm(u1, u0, 0x07060302u), __builtin_amdgcn_perm(w1, w0, 0x07060302u),
             __builtin_amdgcn_perm(t1, t0, 0x07060302u)};
}

// An f32 value as the sum hi + lo of two bf16 values, each rounded to nearest
// even (gfx950's v_cvt_pk_bf16_f32): hi = RN(x), lo = RN(x - hi).  x - hi is
// exact, and each rounding keeps 8 significant bits, so
// |x - hi - lo| <= 2^-16 |x|: a product through the two parts is the f32
// product up to that relative error per term (the default for the state and
// Cs with 16-bit q and k; split_bf3 keeps them exact).  Two values are packed
// per word, the first in the low half.
struct Bf2 {
  uint32_t h, l;
};
__device__ __forceinline__ Bf2 split_bf2(float x0, float x1) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x0, x1}, b2));
  const f2 r = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u)};
  return Bf2{h, __builtin_bit_cast(uint32_t, __builtin_convertvector(r, b2))};
}

// 16-bit fragments widened on the matrix cores.  With lane (lg, lc) holding
// X[lc][4 lg .. 4 lg + 3] of a 16 x 16 tile packed (its raw A-operand fragment)
// and E the identity in the same packing, mm16(E, X) leaves X[lc][4 lg + s] in
// register s (the f32 A-operand fragment) and mm16(X, E) leaves X[4 lg + s][lc]
// (the transposed one), exactly.  A product right behind vector work of the
// same wave issues only once the matrix pipe has drained, so widening with
// vector instructions between the products cost more than these products do.
template <int DT>
__device__ __forceinline__ uint2 eye16(int lg, int lc) {  // the identity, packed as above
  const uint32_t one = DT == GDN_BF16 ? 0x3F80u : 0x3C00u;
  uint32_t e[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) e[s] = 4 * lg + s == lc ? one : 0u;
  return make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
}
// The bf16 values of four f32 results of mm16(X, E) (bf16 values already),
// packed two per word
__device__ __forceinline__ uint2 pack_bf16(const v4f& x) {
  return make_uint2(__builtin_amdgcn_perm(__float_as_uint(x[1]), __float_as_uint(x[0]), 0x07060302u),
                    __builtin_amdgcn_perm(__float_as_uint(x[3]), __float_as_uint(x[2]), 0x07060302u));
}

struct Bases {
  int64_t qk, qk_ts, v, v_ts, g, g_ts;
};

__device__ __forceinline__ Bases head_bases(int64_t b, int hv, int hk, int Hk, int Hv, int64_t T,
                                            int head_major, int D) {
  Bases r;
  if (head_major) {
    r.qk = (b * Hk + hk) * T * D; r.qk_ts = D;
    r.v = (b * Hv + hv) * T * D; r.v_ts = D;
    r.g = (b * Hv + hv) * T; r.g_ts = 1;
  } else {
    r.qk = (b * T * Hk + hk) * D; r.qk_ts = (int64_t)Hk * D;
    r.v = (b * T * Hv + hv) * D; r.v_ts = (int64_t)Hv * D;
    r.g = b * T * Hv + hv; r.g_ts = Hv;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Block pieces that do not depend on the state.

// Entry (row, col) of a 16 x 16 block written as two bf16 parts rounded to
// nearest (hi = RN(x), lo = RN(x - hi)), in 16-byte chunks of four columns:
// chunk 4 row + col / 4 holds the four hi values, then the four lo values.
// A lane reading chunk 4 lc + lg then has the hi and lo A fragments of a
// 16x16x16 bf16 product over row lc (the few-head chain wave's T and M1).
__device__ __forceinline__ void store_parts16(float* base, int row, int col, float x) {
  const uint16_t h = __builtin_bit_cast(uint16_t, (__bf16)x);
  const uint16_t l = __builtin_bit_cast(uint16_t, (__bf16)(x - __uint_as_float((uint32_t)h << 16)));
  uint16_t* p = reinterpret_cast<uint16_t*>(base) + 8 * (4 * row + col / 4) + col % 4;
  p[0] = h;
  p[4] = l;
}

struct PrepArgs {
  const void *q, *k, *ld, *beta;
  float* rec;
  int64_t T, nblk, ntask;  // ntask = B * Hk * nblk
  int Hk, Hv, G, head_major;
  uint32_t flags;
  float qk_eps, qscale;
  float* mx;  // null, or [B][Hk][nblk][3][16][16]: K_c K_(c-1)^T, K_c K_(c-2)^T, Q_c K_(c-1)^T (raw)
};

// One wave per (batch, key head, block): K K^T and Q K^T once, then the
// records of the G value heads that share the key head (four at a time, one
// per 16-lane group).  No workgroup barrier: each wave owns its LDS slice.
// XB: also the products across blocks into a.mx (the few-head kernel's; a
// separate instance, so the many-head prep keeps its register count).
// TP: T, Hd, M1, M2 and N written as two rounded bf16 parts (store_parts16)
// for the few-head kernel's default products.
template <int DT, int GT, int D, bool XB, bool TP>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  static_assert(XB || !TP, "the parts layout is the few-head kernel's");
  // a lane holds D / 4 elements of a row: NU loads of 8, taken in NCH chunks
  // of NUC (more than 32 elements per lane, 16 for f32 rows at D = 256, would
  // not fit beside the cross-block products: those rows are loaded and their
  // products accumulated a chunk at a time)
  constexpr int NU = D / 32, NUC = DT == GDN_F32 && D > 128 ? 2 : (NU < 4 ? NU : 4), NCH = NU / NUC;
  static_assert(NU >= 1 && D % 32 == 0, "head dim a multiple of 32");
  static_assert(NCH == 1 || XB, "chunked rows: few heads (D = 256)");
  __shared__ float sLs[4][4][kL][kL + 1];  // [wave][value head of the group][i][j]
  __shared__ __align__(16) float sAB[4][2][4][kL];  // [wave][alpha, beta][value head][token]
  // the wave index through readfirstlane: everything derived from the task
  // is then uniform (scalar), not computed per lane; the task count is below
  // 2^31 (B * T * Hv is), so 32-bit divisions suffice
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, lc = lane % 16;
  const int64_t task = (int64_t)blockIdx.x * 4 + wave;
  if (task >= a.ntask) return;  // uniform per wave
  const uint32_t tk = (uint32_t)task, nb = (uint32_t)a.nblk;
  const int64_t c = tk % nb, bk = tk / nb;
  const int hk = (int)((uint32_t)bk % (uint32_t)a.Hk);
  const int64_t b = (uint32_t)bk / (uint32_t)a.Hk, T = a.T, t0 = c * kL;
  const int tc = (int)((T - t0) < kL ? (T - t0) : kL);
  int64_t qk_base, qk_ts;
  if (a.head_major) {
    qk_base = (b * a.Hk + hk) * T * D; qk_ts = D;
  } else {
    qk_base = (b * T * a.Hk + hk) * D; qk_ts = (int64_t)a.Hk * D;
  }

  // Every load of the wave is issued here, before any of them is used, so
  // that their latencies overlap (one round trip instead of one per use).
  // Rows of q and k: lane (lg, lc) holds row lc, elements [D/4 lg, D/4 (lg + 1))
  // Addresses: a block base (uniform) plus a 32-bit offset per lane, so no
  // lane computes a 64-bit product.
  const uint32_t loff = (uint32_t)lc * (uint32_t)qk_ts + (uint32_t)(D / 4) * (uint32_t)lg;
  Raw<DT, 8> kr[NUC], qr[NUC];
  const int64_t rowb = qk_base + t0 * qk_ts;
  auto load_rows = [&](int ch) {
#pragma unroll
    for (int u = 0; u < NUC; ++u) {
      if (lc < tc) {
        kr[u].load(a.k, rowb + (int64_t)(loff + 8u * (ch * NUC + u)));
        qr[u].load(a.q, rowb + (int64_t)(loff + 8u * (ch * NUC + u)));
      } else {
        kr[u].zero();
        qr[u].zero();
      }
    }
  };
  load_rows(0);
  // XB: the key rows of the two blocks before (block 0's where there is
  // none; those products are replaced by zero below)
  [[maybe_unused]] Raw<DT, 8> kp1[NUC], kp2[NUC];
  const int64_t c1 = c > 0 ? c - 1 : 0, c2 = c > 1 ? c - 2 : 0;
  const int64_t b1r = qk_base + c1 * kL * qk_ts, b2r = qk_base + c2 * kL * qk_ts;
  auto load_prev = [&](int ch) {
#pragma unroll
    for (int u = 0; u < NUC; ++u) {
      kp1[u].load(a.k, b1r + (int64_t)(loff + 8u * (ch * NUC + u)));
      kp2[u].load(a.k, b2r + (int64_t)(loff + 8u * (ch * NUC + u)));
    }
  };
  if constexpr (XB) load_prev(0);
  // gates: lane (lg, lc) loads token lc of value head g0 + lg
  Raw<GT, 1> l1, b1;
  bool gld = false;
  auto gates_load = [&](int g0) {
    const int g = g0 + lg;
    gld = g < a.G && lc < tc;
    const int64_t hv0 = (int64_t)hk * a.G + g0;  // first value head of the group
    const int64_t gb = a.head_major ? (b * a.Hv + hv0) * T + t0 : (b * T + t0) * a.Hv + hv0;
    const uint32_t go = a.head_major ? (uint32_t)lg * (uint32_t)T + (uint32_t)lc
                                     : (uint32_t)lc * (uint32_t)a.Hv + (uint32_t)lg;
    if (gld) {
      l1.load(a.ld, gb + (int64_t)go);
      b1.load(a.beta, gb + (int64_t)go);
    }
  };
  gates_load(0);
  // squared norms of row lc (16-bit inputs: below, from the products; f32
  // ones chunk by chunk, summed over the lane groups at the end)
  float ssk = 0.f, ssq = 0.f;
  [[maybe_unused]] auto norms = [&]() {
#pragma unroll
    for (int u = 0; u < NUC; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ssk = fmaf(kr[u].get(e), kr[u].get(e), ssk);
        ssq = fmaf(qr[u].get(e), qr[u].get(e), ssq);
      }
  };
  if constexpr (DT == GDN_F32) norms();

  // X Y^T of 16 raw rows each on the matrix cores; lane (lg, lc), register
  // r: entry [4 lg + r][lc].  The contraction runs over the lane's own D / 4
  // elements: f32, one element per 16x16x4 product; 16-bit, four per 16x16x16
  // product straight from the loaded words (no widening).
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  auto gram = [&](const Raw<DT, 8>* x, const Raw<DT, 8>* y, v4f d) {
    if constexpr (DT == GDN_F32) {
#pragma unroll
      for (int u = 0; u < NUC; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) d = mfma4(x[u].get(e), y[u].get(e), d);
    } else {
#pragma unroll
      for (int m = 0; m < 2 * NUC; ++m)
        d = mm16<DT>(make_uint2(x[m / 2].w[2 * (m % 2)], x[m / 2].w[2 * (m % 2) + 1]),
                     make_uint2(y[m / 2].w[2 * (m % 2)], y[m / 2].w[2 * (m % 2) + 1]), d);
    }
    return d;
  };
  // chunked rows: every product accumulated chunk by chunk (Q Q^T and the
  // cross-block ones too, since the chunk's rows are gone afterwards)
  [[maybe_unused]] v4f Q4c = zero, M1c = zero, M2c = zero, N1c = zero;
  v4f G4 = gram(kr, kr, zero), H4 = gram(qr, kr, zero);
  if constexpr (NCH > 1) {
    if constexpr (DT != GDN_F32) Q4c = gram(qr, qr, zero);  // (f32: the norms come from the rows)
    M1c = gram(kr, kp1, zero);
    N1c = gram(qr, kp1, zero);
    M2c = gram(kr, kp2, zero);
#pragma unroll
    for (int ch = 1; ch < NCH; ++ch) {
      load_rows(ch);
      load_prev(ch);
      if constexpr (DT == GDN_F32) norms();
      G4 = gram(kr, kr, G4);
      H4 = gram(qr, kr, H4);
      if constexpr (DT != GDN_F32) Q4c = gram(qr, qr, Q4c);
      M1c = gram(kr, kp1, M1c);
      N1c = gram(qr, kp1, N1c);
      M2c = gram(kr, kp2, M2c);
    }
  }
  if constexpr (DT == GDN_F32) {
    ssk += __shfl_xor(ssk, 16);
    ssk += __shfl_xor(ssk, 32);
    ssq += __shfl_xor(ssq, 16);
    ssq += __shfl_xor(ssq, 32);
  } else {
    // 16-bit inputs: the squared norms are the diagonals of K K^T (above) and
    // Q Q^T (one more product on the otherwise idle matrix cores instead of
    // 64 widening multiply-adds per lane): entry [lc][lc] sits in register
    // lc % 4 of lane (lc / 4) * 16 + lc
    const v4f Q4 = NCH > 1 ? Q4c : gram(qr, qr, zero);
    auto diag = [&](const v4f& m) {
      const int r = lc % 4;
      const float v = r == 0 ? m[0] : (r == 1 ? m[1] : (r == 2 ? m[2] : m[3]));
      return __shfl(v, (lc / 4) * 16 + lc);
    };
    ssk = diag(G4);
    ssq = diag(Q4);
  }
  const bool l2 = (a.flags & GDN_FOLD_QK_L2NORM) != 0;
  float rk = rsqrtf(l2 ? ssk + a.qk_eps : 1.f);          // of row lc
  float rq = rsqrtf(l2 ? ssq + a.qk_eps : 1.f) * a.qscale;
  if (lc >= tc) rk = rq = 0.f;
  if constexpr (XB) {
    // Products of raw rows across blocks (zero where the earlier block does
    // not exist), row-major: M1 = K_c K_(c-1)^T, M2 = K_c K_(c-2)^T and
    // N = Q_c K_(c-1)^T.  The few-head kernel forms K S^T and Q S^T of a
    // newer state from an older one with them.
    v4f M1, N1, M2;
    if constexpr (NCH > 1) {
      M1 = c > 0 ? M1c : zero;
      N1 = c > 0 ? N1c : zero;
      M2 = c > 1 ? M2c : zero;
    } else {
      M1 = c > 0 ? gram(kr, kp1, zero) : zero;
      N1 = c > 0 ? gram(qr, kp1, zero) : zero;
      M2 = c > 1 ? gram(kr, kp2, zero) : zero;
    }
    float* mx = a.mx + task * (3 * kL * kL);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (TP) {
        store_parts16(mx, 4 * lg + r, lc, M1[r]);
        store_parts16(mx + kL * kL, 4 * lg + r, lc, M2[r]);
        store_parts16(mx + 2 * kL * kL, 4 * lg + r, lc, N1[r]);
      } else {
        mx[16 * (4 * lg + r) + lc] = M1[r];
        mx[kL * kL + 16 * (4 * lg + r) + lc] = M2[r];
        mx[2 * kL * kL + 16 * (4 * lg + r) + lc] = N1[r];
      }
    }
  }
  float rki[4], rqi[4];  // norms of the lane's rows i = 4 lg + r
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    rki[r] = __shfl(rk, 4 * lg + r);
    rqi[r] = __shfl(rq, 4 * lg + r);
  }

  for (int g0 = 0; g0 < a.G; g0 += 4) {
    if (g0 > 0) gates_load(g0);
    const int g = g0 + lg;
    const bool gv = g < a.G;
    const float al = gld ? expf(l1.get(0)) : 1.f, be = gld ? b1.get(0) : 0.f;
    // decay products of token lc of each 16-lane row's value head: from the
    // block start through lc, and after lc to the block end
    const float gam = row_prefix_prod(al), tail = dpp_or_one<0x101, 0xF>(row_suffix_prod(al));
    const int ng = a.G - g0 < 4 ? a.G - g0 : 4;
    // every lane's alpha and beta into the wave's LDS slice ([value head of
    // the group][token]); each lane then reads what it needs in a few vector
    // reads (cross-lane shuffles one row at a time formed a chain of LDS
    // round trips)
    sAB[wave][0][lg][lc] = al;
    sAB[wave][1][lg][lc] = be;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int gq = 0; gq < ng; ++gq) {  // Ls and Hd of value head g0 + gq, all lanes
      float als[kL];  // the 16 alphas of value head g0 + gq (the same in every lane)
#pragma unroll
      for (int m4 = 0; m4 < kL / 4; ++m4) {
        const float4 x = *reinterpret_cast<const float4*>(&sAB[wave][0][gq][4 * m4]);
        als[4 * m4] = x.x, als[4 * m4 + 1] = x.y, als[4 * m4 + 2] = x.z, als[4 * m4 + 3] = x.w;
      }
      // alpha and beta of the lane's rows i = 4 lg .. 4 lg + 3
      const float4 ar = *reinterpret_cast<const float4*>(&sAB[wave][0][gq][4 * lg]);
      const float4 br = *reinterpret_cast<const float4*>(&sAB[wave][1][gq][4 * lg]);
      const float ari[4] = {ar.x, ar.y, ar.z, ar.w}, bri[4] = {br.x, br.y, br.z, br.w};
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
        if (r > 0) dc = j < i ? dc * ari[r] : (j == i ? 1.f : 0.f);
        sLs[wave][gq][i][j] = j < i ? bri[r] * rki[r] * G4[r] * rk * dc : 0.f;
        const float hd = j <= i ? rqi[r] * H4[r] * rk * dc : 0.f;
        if constexpr (TP) store_parts16(rec + kRecH, i, j, hd);
        else rec[kRecH + 16 * i + j] = hd;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (gv) {  // lane group lg: value head g; lane lc: token lc and column lc
      float* rec = a.rec + record_at(b * a.Hv + hk * a.G + g0, c, a.nblk) +
                   (int64_t)lg * (a.nblk * kRec);
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
      for (int r = 0; r < kL; ++r) {
        if constexpr (TP) store_parts16(rec + kRecT, r, lc, x[r]);
        else rec[kRecT + 16 * r + lc] = x[r];
      }
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
  const float* mx;  // the prep's K_c K_(c-1)^T blocks (lookahead kernel only)
};

// The many-head shape: one workgroup per value head, its 8 waves one a-tile
// (16 value rows) each over all 8 key tiles, two workgroups per CU; the gated
// norm is fused.  The loads of block c + 1 are issued while block c is
// computed.  NSP: parts of the state and of Cs in the products of 16-bit
// inputs (3: exact, split_bf3; 2: rounded, split_bf2).
template <int DT, int NSP, int D>
__global__ __launch_bounds__(4 * D) __attribute__((amdgpu_waves_per_eu(4))) void state_kernel(
    StateArgs a) {
  static_assert(NSP == 2 || NSP == 3, "two or three parts");
  static_assert(D % 32 == 0 && D <= 128, "head dim 32, 64 or 128");
  // a wave per 16 value rows (a-tile), each over all D / 16 key tiles
  constexpr int NW = D / 16, NT = NW * kWave, ROWS = D, NCT = D / 16;
  // 16-bit inputs: q and k in LDS as bf16 parts (bf16: the value; f16: its
  // exact split into two bf16 values), the products on the bf16 matrix cores
  // against the three exact bf16 parts of the state; f32 inputs: f32 products
  constexpr bool W16 = DT != GDN_F32;
  constexpr int NPART = DT == GDN_F16 ? 2 : 1, KP16 = D + 8, KPF = D + 4;
  __shared__ __align__(16) float sk[kL][KPF];
  __shared__ __align__(16) float sq[kL][KPF];
  __shared__ __align__(16) uint16_t sk16[NPART][kL][KP16];
  __shared__ __align__(16) uint16_t sq16[NPART][kL][KP16];
  __shared__ float sv[kL][ROWS];
  __shared__ float sz[2][kL][D];
  __shared__ __align__(16) float so[2][kL][ROWS];
  __shared__ __align__(16) float srec[kRecUsed];

  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t bh = tile;
  const int hv = (int)(bh % a.Hv), hk = hv / a.G;
  const int64_t b = bh / a.Hv;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: scalar index math
  const int lg = lane / 16, lc = lane % 16;
  const int ai = wave;  // this wave's a-tile (value rows 16 ai ..), all key tiles
  const int64_t T = a.T;
  const bool has_z = a.z != nullptr;
  const Bases bs = head_bases(b, hv, hk, a.Hk, a.Hv, T, a.head_major, D);
  const int64_t sbase = (b * a.Hv + hv) * (int64_t)(D * D);
  const float* rec = a.rec + record_at(bh, 0, a.nblk);

  // staging of one block: items of 8 q or k elements (IPR per row, NI in
  // all, k first), v pairs, z pairs (fused), the record as float4
  constexpr int IPR = D / 8, NI = 2 * kL * IPR;
  constexpr int NQK = (NI + NT - 1) / NT;
  constexpr int NVP = (kL * ROWS / 2 + NT - 1) / NT;
  constexpr int NZP = (kL * D / 2 + NT - 1) / NT;
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
  // addresses: the block's base (uniform) plus a 32-bit offset per lane, so
  // no 64-bit per-lane address stays live across the loop
  auto chunk_load = [&](Regs& P, int64_t c, int tc) {
    const int64_t t0 = c * kL;
    const int64_t qkb = bs.qk + t0 * bs.qk_ts, vb = bs.v + t0 * bs.v_ts;
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int e = (tid + i * NT) % NI, it = e % (NI / 2), tt = it / IPR, c8 = it % IPR;
      const int which = __builtin_amdgcn_readfirstlane(e / (NI / 2));  // uniform per wave
      const uint32_t off = (uint32_t)clamp_t(tt, tc) * (uint32_t)bs.qk_ts + 8u * (uint32_t)c8;
      P.qk[i].load(which ? a.q : a.k, qkb + (int64_t)off);
    }
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int e = (tid + i * NT) % (kL * ROWS / 2), tt = e / (ROWS / 2), r2 = e % (ROWS / 2);
      const uint32_t off = (uint32_t)clamp_t(tt, tc) * (uint32_t)bs.v_ts + 2u * (uint32_t)r2;
      P.v[i].load(a.v, vb + (int64_t)off);
    }
    if (has_z) {
#pragma unroll
      for (int i = 0; i < NZP; ++i) {
        const int e = (tid + i * NT) % (kL * D / 2), tt = e / (D / 2), r2 = e % (D / 2);
        const uint32_t off = (uint32_t)clamp_t(tt, tc) * (uint32_t)bs.v_ts + 2u * (uint32_t)r2;
        P.z[i].load(a.z, vb + (int64_t)off);
      }
    }
#pragma unroll
    for (int i = 0; i < NRC; ++i) {
      const int e = tid + i * NT < NR4 ? tid + i * NT : NR4 - 1;
      P.r[i].load(rec, c * kRec + (int64_t)(uint32_t)(4 * e));
    }
  };
  // Every lane also writes every item it loaded (lanes past the item count
  // repeat an item with the same value), so no path leaves a load unread.
  // Rows past the last token repeat its inputs; the block record gives them
  // beta = rk = rq = 0, so they add nothing to C, O or the state.
  auto chunk_store = [&](const Regs& P, int zbuf) {
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int e = (tid + i * NT) % NI, which = e / (NI / 2), it = e % (NI / 2), tt = it / IPR, c8 = it % IPR;
      if constexpr (DT == GDN_F32) {
        float* dst = which ? &sq[tt][8 * c8] : &sk[tt][8 * c8];
        *reinterpret_cast<float4*>(dst) = P.qk[i].get4(0);
        *reinterpret_cast<float4*>(dst + 4) = P.qk[i].get4(1);
      } else if constexpr (DT == GDN_BF16) {
        uint16_t* dst = which ? &sq16[0][tt][8 * c8] : &sk16[0][tt][8 * c8];
        *reinterpret_cast<uint4*>(dst) = make_uint4(P.qk[i].w[0], P.qk[i].w[1], P.qk[i].w[2], P.qk[i].w[3]);
      } else {
        // an f16 value x is hi + lo exactly: hi its top 8 significant bits
        // (truncation), lo the other 3 or fewer
        uint32_t h[4], l[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float x0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(P.qk[i].w[w] & 0xffffu));
          const float x1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(P.qk[i].w[w] >> 16));
          const uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
          const uint32_t r0 = __float_as_uint(x0 - __uint_as_float(u0 & 0xffff0000u));
          const uint32_t r1 = __float_as_uint(x1 - __uint_as_float(u1 & 0xffff0000u));
          h[w] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
          l[w] = __builtin_amdgcn_perm(r1, r0, 0x07060302u);
        }
        *reinterpret_cast<uint4*>(which ? &sq16[0][tt][8 * c8] : &sk16[0][tt][8 * c8]) = make_uint4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<uint4*>(which ? &sq16[1][tt][8 * c8] : &sk16[1][tt][8 * c8]) = make_uint4(l[0], l[1], l[2], l[3]);
      }
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
        const int e = (tid + i * NT) % (kL * D / 2), tt = e / (D / 2), r2 = e % (D / 2);
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

  // state S^T, this wave's key tiles of its a-tile, in the accumulator layout.
  // 16-bit inputs: the keys in the order that makes lane (lg, lc) hold keys
  // 32 g + 8 lg .. + 7 of its row in tiles 2 g and 2 g + 1 (tile ct keeps
  // key 32 (ct / 2) + 8 (i / 4) + 4 (ct % 2) + i % 4 at tile row i): the two
  // tiles' registers are then the B operand of a 16x16x32 product whose A
  // operand is 8 consecutive elements of a q or k row.
  v4f St[NCT];
  const int arow = 16 * ai + lc;  // value row of this lane
  auto key0 = [&](int ct) { return W16 ? 32 * (ct / 2) + 8 * lg + 4 * (ct % 2) : 16 * ct + 4 * lg; };
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const float4 x = *reinterpret_cast<const float4*>(a.s0 + sbase + (int64_t)arow * D + key0(ct));
    St[ct] = v4f{x.x, x.y, x.z, x.w};
  }
  [[maybe_unused]] const uint2 eye = eye16<GDN_BF16>(lg, lc);
  // 16-bit inputs: the decay is applied lazily, the state being gsc * St
  // (gsc uniform; St rescaled and gsc reset to 1 only when gsc would drop
  // under 2^-80, a zero decay included), so each block scales the four
  // values of K S^T and Q S^T and Cs instead of the 32 of St
  float gsc = 1.f;
  // the gated norm: a lane holds EPL of a token's D values (lanes past D,
  // below 64, hold none)
  constexpr int EPL = D >= kWave ? D / kWave : 1;
  const bool nact = D >= kWave || lane < D;
  float wgt[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) wgt[i] = has_z && nact ? ld1<DT>(a.w, lane + kWave * i) : 0.f;
  const int64_t nblk = a.nblk;
  auto tc_of = [&](int64_t c) { return (int)((T - c * kL) < kL ? (T - c * kL) : kL); };

  // Outputs of block c from LDS (a fixed number of stores per lane).  They
  // run after the top barrier of the next block, before its loads, so the
  // waits on those loads never have to cover these stores.
  auto outputs = [&](int64_t c) {
    const int64_t t0 = c * kL;
    const int tc = tc_of(c);
    if (has_z) {  // the gated norm: kL / NW tokens per wave, D values each
#pragma unroll
      for (int u = 0; u < kL / NW; ++u) {
        const int tt = wave + NW * u, zb = (int)(c & 1);
        float x[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          x[i] = nact ? so[c & 1][tt][lane + kWave * i] * silu(sz[zb][tt][lane + kWave * i]) : 0.f;
        float ss = x[EPL - 1] * x[EPL - 1];
#pragma unroll
        for (int i = EPL - 2; i >= 0; --i) ss = fmaf(x[i], x[i], ss);
        const float inv = rsqrtf(wave_sum(ss) * (1.0f / D) + a.norm_eps);
        if (tt < tc && nact) {
          const int64_t vo = bs.v + (t0 + tt) * bs.v_ts;
#pragma unroll
          for (int i = 0; i < EPL; ++i) a.y[vo + lane + kWave * i] = x[i] * inv * wgt[i];
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
    if constexpr (W16) {
      // per group of 32 keys: the parts of S (small first) against each part
      // of k and q
#pragma unroll
      for (int g4 = 0; g4 < NCT / 2; ++g4) {
        uint4 sh, sm, sl;
        if constexpr (NSP == 3) {
          const Bf3 a0 = split_bf3(St[2 * g4][0], St[2 * g4][1]), a1 = split_bf3(St[2 * g4][2], St[2 * g4][3]);
          const Bf3 b0 = split_bf3(St[2 * g4 + 1][0], St[2 * g4 + 1][1]);
          const Bf3 b1 = split_bf3(St[2 * g4 + 1][2], St[2 * g4 + 1][3]);
          sh = make_uint4(a0.h, a1.h, b0.h, b1.h);
          sm = make_uint4(a0.m, a1.m, b0.m, b1.m);
          sl = make_uint4(a0.l, a1.l, b0.l, b1.l);
        } else {
          const Bf2 a0 = split_bf2(St[2 * g4][0], St[2 * g4][1]), a1 = split_bf2(St[2 * g4][2], St[2 * g4][3]);
          const Bf2 b0 = split_bf2(St[2 * g4 + 1][0], St[2 * g4 + 1][1]);
          const Bf2 b1 = split_bf2(St[2 * g4 + 1][2], St[2 * g4 + 1][3]);
          sh = make_uint4(a0.h, a1.h, b0.h, b1.h);
          sl = make_uint4(a0.l, a1.l, b0.l, b1.l);
        }
#pragma unroll
        for (int p = 0; p < NPART; ++p) {
          const uint4 kA = *reinterpret_cast<const uint4*>(&sk16[p][lc][32 * g4 + 8 * lg]);
          const uint4 qA = *reinterpret_cast<const uint4*>(&sq16[p][lc][32 * g4 + 8 * lg]);
          pk = mm32bf(kA, sl, pk);
          pq = mm32bf(qA, sl, pq);
          if constexpr (NSP == 3) {
            pk = mm32bf(kA, sm, pk);
            pq = mm32bf(qA, sm, pq);
          }
          pk = mm32bf(kA, sh, pk);
          pq = mm32bf(qA, sh, pq);
        }
        // one group at a time: the accumulators pass through an empty asm, so
        // no product of a later group moves above it (interleaved, the
        // groups' parts overflow the 128 registers of four waves per SIMD)
        asm volatile("" : "+v"(pk), "+v"(pq));
      }
    } else {
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
    }
    if constexpr (W16) {
      pk *= gsc;
      pq *= gsc;
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
    if constexpr (W16) {
      // S' = gl S + K^T Cs with S = gsc St: St' = St + K^T (Cs / g) and
      // gsc' = g for g = gl gsc, or (g under 2^-80) St' = g St + K^T Cs and
      // gsc' = 1
      const float g = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gl))) * gsc;
      float cscale;
      if (g < 0x1p-80f) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) St[ct] *= g;
        gsc = 1.f;
        cscale = 1.f;
      } else {
        gsc = g;
        cscale = __builtin_amdgcn_rcpf(g);  // 1 ulp
      }
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) cs[s2] = cc[s2] * (srec[kRecSrs + 4 * lg + s2] * cscale);
    } else {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) cs[s2] = cc[s2] * srec[kRecSrs + 4 * lg + s2];
    }
    if constexpr (W16) {
      // the parts of Cs against the parts of k, transposed on the matrix
      // cores (mm16(X, E)); with two parts of k both go into one 16x16x32
      // product (contraction: 16 tokens x 2 parts, Cs's part given twice)
      uint32_t c0h, c0m = 0, c0l, c1h, c1m = 0, c1l;
      if constexpr (NSP == 3) {
        const Bf3 c0 = split_bf3(cs[0], cs[1]), c1 = split_bf3(cs[2], cs[3]);
        c0h = c0.h, c0m = c0.m, c0l = c0.l, c1h = c1.h, c1m = c1.m, c1l = c1.l;
      } else {
        const Bf2 c0 = split_bf2(cs[0], cs[1]), c1 = split_bf2(cs[2], cs[3]);
        c0h = c0.h, c0l = c0.l, c1h = c1.h, c1l = c1.l;
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        uint2 kt[NPART];
#pragma unroll
        for (int p = 0; p < NPART; ++p)
          kt[p] = pack_bf16(mm16<GDN_BF16>(*reinterpret_cast<const uint2*>(&sk16[p][lc][key0(ct)]), eye));
        v4f acc = St[ct];
        if constexpr (NPART == 1 && NSP == 2) {
          // k's four tokens twice against the two parts of Cs side by side
          acc = mm32bf(make_uint4(kt[0].x, kt[0].y, kt[0].x, kt[0].y), make_uint4(c0l, c1l, c0h, c1h), acc);
        } else if constexpr (NPART == 1) {
          acc = mm16<GDN_BF16>(kt[0], make_uint2(c0l, c1l), acc);
          acc = mm16<GDN_BF16>(kt[0], make_uint2(c0m, c1m), acc);
          acc = mm16<GDN_BF16>(kt[0], make_uint2(c0h, c1h), acc);
        } else {
          const uint4 ka = make_uint4(kt[0].x, kt[0].y, kt[1].x, kt[1].y);
          acc = mm32bf(ka, make_uint4(c0l, c1l, c0l, c1l), acc);
          if constexpr (NSP == 3) acc = mm32bf(ka, make_uint4(c0m, c1m, c0m, c1m), acc);
          acc = mm32bf(ka, make_uint4(c0h, c1h, c0h, c1h), acc);
        }
        St[ct] = acc;
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int kc = 16 * ct + lc;
        v4f acc = St[ct] * gl;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = mfma4(sk[4 * lg + s2][kc], cs[s2], acc);
        St[ct] = acc;
      }
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
    if constexpr (W16) St[ct] *= gsc;
    float4 x = make_float4(St[ct][0], St[ct][1], St[ct][2], St[ct][3]);
    *reinterpret_cast<float4*>(a.s_out + sbase + (int64_t)arow * D + key0(ct)) = x;
  }
}

// K and Q of a block sit in LDS in the input's format (16-bit inputs as
// their raw halves: LDS writes, not reads, limit the few-head kernel) and
// are widened to f32 as they are read.
template <int DT>
using LdsElem = typename std::conditional<DT == GDN_F32, float, uint16_t>::type;
template <int DT, int D>
constexpr int lds_row() {  // padded row, elements: rows 4 banks apart
  return DT == GDN_F32 ? D + 4 : D + 8;
}

// State waves of the few-head kernel: D / 32 of 32 keys each.  Threads: the
// state waves, then the chain, O and two staging waves.
template <int DT, int D>
constexpr int rows_nc() { return D / 32; }
template <int DT, int D>
constexpr int rows_la_threads() { return (rows_nc<DT, D>() + 4) * kWave; }

// The sum of the state waves' partial products, pairwise
template <int N>
__device__ __forceinline__ v4f sum_parts(const v4f (*p)[kWave], int lane) {
  if constexpr (N == 1) return p[0][lane];
  else return sum_parts<N / 2>(p, lane) + sum_parts<N / 2>(p + N / 2, lane);
}
template <int DT>
__device__ __forceinline__ float half_lo(uint32_t x) {
  if constexpr (DT == GDN_BF16) return __uint_as_float(x << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
}
template <int DT>
__device__ __forceinline__ float half_hi(uint32_t x) {
  if constexpr (DT == GDN_BF16) return __uint_as_float(x & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
}
template <int DT>
__device__ __forceinline__ float4 lds_get4(const LdsElem<DT>* row, int e) {  // e % 4 == 0
  if constexpr (DT == GDN_F32) {
    return *reinterpret_cast<const float4*>(row + e);
  } else {
    const uint2 u = *reinterpret_cast<const uint2*>(row + e);
    return make_float4(half_lo<DT>(u.x), half_hi<DT>(u.x), half_lo<DT>(u.y), half_hi<DT>(u.y));
  }
}
template <int DT>
__device__ __forceinline__ float lds_get(const LdsElem<DT>* row, int e) {
  if constexpr (DT == GDN_F32) return row[e];
  else return half_lo<DT>(row[e]);
}

// The few-head shape: a workgroup per 16 value rows of a head, the block
// recurrence taken apart so that each round (one 16-token block) has no
// chain of products through the state.  With B_(r+1) = K_(r+1) S_(r-1)^T and
// P_r = Q_r S_(r-1)^T formed from the state before round r's update, and
// C-scaled_c = diag(rk Dc[15][.]) C_c:
//   K_(r+1) S_(r+1)^T = gam(r) (gam(r-1) B_(r+1) + M2_(r+1) Cs_(r-1))
//                       + M1_(r+1) Cs_r,
//   Q_r S_r^T = gam(r-1) P_r + N_r Cs_(r-1),
// gam(c) = gam_15 of block c, M1, M2, N the prep's 16 x 16 products of raw
// rows.  Round r, after one workgroup barrier:
//   waves 0-3 (state, 32 keys each): their parts of P_r and B_(r+1), then
//     S_r = gam(r-1) S_(r-1) + K_(r-1)^T Cs_(r-1) (bf16 inputs: on the bf16
//     parts of S and Cs, with their own q and k loaded four blocks ahead);
//   wave 4 (chain): C_r from the B_r parts, Y_r and its own Cs_(r-1), then
//     M1_(r+1) Cs_r for the next round (and Cs_r's bf16 parts);
//   wave 5: O and y of block r - 1;
//   wave 6: Y_(r+1) = M2_(r+1) Cs_(r-1);  wave 7: Z_r = N_r Cs_(r-1);
//   waves 6-7: block r + 2 into a four-slot LDS ring (v, the record, M1 M2
//     N, and q and k unless the state waves load them), the loads of block
//     r + 5 (three register sets).
// Every operand a wave needs from LDS is read at the start of the round
// before it or right after its own barrier, so each role issues its matrix
// products back to back.  A prologue round forms A_0 = K_0 S_0^T; the last
// round finishes the state and O.  Each role runs its own loop with the same
// barriers.
template <int DT, int NSP, int D>
__global__ __launch_bounds__((rows_la_threads<DT, D>())) __attribute__((amdgpu_waves_per_eu(2))) void
rows_la_kernel(StateArgs a) {
  static_assert(NSP == 2 || NSP == 3, "two or three parts of the state and Cs");
  static_assert(D % 32 == 0 && D <= 256, "head dim 32 to 256");
  // NC state waves of two 16-key tiles each
  constexpr int NC = rows_nc<DT, D>(), NCT = 2, ROWS = 16, KP = lds_row<DT, D>(), NM = 3 * kL * kL;
  typedef LdsElem<DT> KT;
  // f32 q and k rows staged in LDS up to D = 128 (16-bit inputs, and f32 ones
  // at D = 256, whose rows would take 133 KB: the state waves load their own;
  // at D = 256 the unused slots shrink to a token)
  constexpr int SKS = D <= 128 ? 4 : 1, SKP = D <= 128 ? KP : 8;
  __shared__ __align__(16) KT sk[SKS][kL][SKP];
  __shared__ __align__(16) KT sq[SKS][kL][SKP];
  __shared__ __align__(16) float sv[4][kL][ROWS];
  __shared__ __align__(16) float srec[4][kRecUsed];
  __shared__ __align__(16) float smx[4][NM];  // M1, M2, N of a block
  __shared__ v4f sb[2][NC][kWave];  // parts of B (of A_0 in the prologue)
  __shared__ v4f sp[2][NC][kWave];  // parts of P
  __shared__ v4f scs[2][kWave];     // C-scaled
  __shared__ uint2 scp[2][NSP][kWave];  // its bf16 parts (16-bit inputs): lo, (mid,) hi
  __shared__ v4f scc[2][kWave];     // C
  // chain, Y and Z products on bf16 parts (16-bit inputs, two parts): the
  // prep then writes T, M1, M2 and N as parts (store_parts16), staged like
  // the f32 values
  constexpr bool BFCHAIN = DT != GDN_F32 && NSP == 2;
  __shared__ v4f sy[2][kWave];      // Y
  __shared__ v4f sz[2][kWave];      // Z

  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int rb = (int)(tile % a.nrb);
  const int64_t bh = tile / a.nrb;
  const int hv = (int)(bh % a.Hv), hk = hv / a.G;
  const int64_t b = bh / a.Hv;
  const int tid = threadIdx.x, lane = tid % kWave;
  // the wave index through readfirstlane: the compiler then treats the role
  // branches as uniform (no exec-mask merge of the roles' registers)
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int cp = wave % NC;
  const int lg = lane / 16, lc = lane % 16;
  const int64_t T = a.T, nblk = a.nblk;
  const Bases bs = head_bases(b, hv, hk, a.Hk, a.Hv, T, a.head_major, D);
  const int row0 = rb * ROWS;
  const int64_t sbase = (b * a.Hv + hv) * (int64_t)(D * D);
  const float* rec = a.rec + record_at(bh, 0, nblk);
  const float* mxh = a.mx + (b * a.Hk + hk) * nblk * NM;
  auto tc_of = [&](int64_t c) { return (int)((T - c * kL) < kL ? (T - c * kL) : kL); };
  auto clampb = [&](int64_t c) { return c < nblk ? c : nblk - 1; };
  const int tcl = tc_of(nblk - 1);

  if constexpr (DT != GDN_F32) {
    if (wave < NC) {
      // ---- state waves, 16-bit inputs.  The wave's 32 key columns go in the
      // order that makes lane (lg, lc) hold columns 32 cp + 8 lg .. + 7 of
      // its row: tile ct keeps S^T row 32 cp + 8 (i / 4) + 4 ct + i % 4 at
      // tile row i.  Its registers are then the B operand of a 16x16x32
      // product whose A operand is 8 consecutive elements of a q or k row
      // (bf16: raw; f16: its exact hi or lo bf16 part, split from the raw
      // row after one 16-byte load).  X S^T runs on the three bf16 parts of S,
      // and the update on those of Cs, against the transposed k (parts).  The
      // wave loads its own q and k slices from global memory (LDS writes, not
      // reads, bound the staging), four blocks ahead.
      v4f St[NCT];
      const int64_t soff = sbase + (int64_t)(row0 + lc) * D + 32 * cp + 8 * lg;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float4 x = *reinterpret_cast<const float4*>(a.s0 + soff + 4 * ct);
        St[ct] = v4f{x.x, x.y, x.z, x.w};
      }
      uint4 Sh, Sm, Sl;
      auto split_state = [&]() {
        if constexpr (NSP == 3) {
          const Bf3 p0 = split_bf3(St[0][0], St[0][1]), p1 = split_bf3(St[0][2], St[0][3]);
          const Bf3 p2 = split_bf3(St[1][0], St[1][1]), p3 = split_bf3(St[1][2], St[1][3]);
          Sh = make_uint4(p0.h, p1.h, p2.h, p3.h);
          Sm = make_uint4(p0.m, p1.m, p2.m, p3.m);
          Sl = make_uint4(p0.l, p1.l, p2.l, p3.l);
        } else {
          const Bf2 p0 = split_bf2(St[0][0], St[0][1]), p1 = split_bf2(St[0][2], St[0][3]);
          const Bf2 p2 = split_bf2(St[1][0], St[1][1]), p3 = split_bf2(St[1][2], St[1][3]);
          Sh = make_uint4(p0.h, p1.h, p2.h, p3.h);
          Sl = make_uint4(p0.l, p1.l, p2.l, p3.l);
        }
      };
      // q and k of a block, row lc, raw (rows past the last token repeat it)
      struct Blk {
        uint4 q, k;
      };
      auto ld = [&](Blk& x, int64_t c) {
        const int tcc = c == nblk - 1 ? tcl : kL;
        const int64_t o = bs.qk + (c * kL + (lc < tcc ? lc : tcc - 1)) * bs.qk_ts + 32 * cp + 8 * lg;
        x.q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + o);
        x.k = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + o);
      };
      // their NPART bf16 parts: bf16 as it is; an f16 value x as hi + lo, hi
      // its top 8 significant bits (truncation), lo the other 3 or fewer
      constexpr int NPART = DT == GDN_F16 ? 2 : 1;
      auto parts = [&](const uint4& r, uint4* f) {
        if constexpr (NPART == 1) {
          f[0] = r;
        } else {
          uint32_t h[4], l[4];
          const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
            const float x1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
            const uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
            const uint32_t r0 = __float_as_uint(x0 - __uint_as_float(u0 & 0xffff0000u));
            const uint32_t r1 = __float_as_uint(x1 - __uint_as_float(u1 & 0xffff0000u));
            h[i] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
            l[i] = __builtin_amdgcn_perm(r1, r0, 0x07060302u);
          }
          f[0] = make_uint4(h[0], h[1], h[2], h[3]);
          f[1] = make_uint4(l[0], l[1], l[2], l[3]);
        }
      };
      // X S^T over this wave's key columns (the parts of X), the small parts
      // of S first
      auto xst = [&](const uint4* f) {
        v4f p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pt = NPART - 1; pt >= 0; --pt) {
          p = mm32bf(f[pt], Sl, p);
          if constexpr (NSP == 3) p = mm32bf(f[pt], Sm, p);
          p = mm32bf(f[pt], Sh, p);
        }
        return p;
      };
      // the next loads of a set stay below its last use (the inputs are
      // read-only: hoisted, they would need new registers and a copy at the
      // loop edge that waits for them)
      auto reload = [&](Blk& x, int64_t c) {
        __builtin_amdgcn_sched_barrier(0);
        int64_t cn = clampb(c);
        asm volatile("" : "+s"(cn) : : "memory");
        ld(x, cn);
      };
      // the raw rows f (this wave's 8 columns per lane) transposed, as bf16:
      // each half of f is the 16x16x16 A fragment of one tile, E turns it over
      // exactly, and the high halves of the f32 results are the bf16 values
      [[maybe_unused]] const uint2 eye = eye16<GDN_BF16>(lg, lc);
      typedef typename std::conditional<NPART == 1, uint2, uint4>::type KtT;
      auto transpose = [&](const uint4* f, KtT* kt) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int pt = 0; pt < NPART; ++pt) {
            const v4f x = mm16<GDN_BF16>(ct ? make_uint2(f[pt].z, f[pt].w) : make_uint2(f[pt].x, f[pt].y), eye);
            const uint32_t w0 = __builtin_amdgcn_perm(__float_as_uint(x[1]), __float_as_uint(x[0]), 0x07060302u);
            const uint32_t w1 = __builtin_amdgcn_perm(__float_as_uint(x[3]), __float_as_uint(x[2]), 0x07060302u);
            if constexpr (NPART == 1) kt[ct] = make_uint2(w0, w1);
            else if (pt == 0) { kt[ct].x = w0; kt[ct].y = w1; }
            else { kt[ct].z = w0; kt[ct].w = w1; }
          }
      };
      // operands of round r's update: K_(r-1) transposed (lane (lg, lc):
      // tokens 4 lg .. + 3 of the tile's column lc; f16: the hi part's four,
      // then the lo part's), formed in round r - 2, and gam(r-1), read in
      // round r - 1
      struct Ops {
        KtT kt[NCT];
        float gl;
      };
      // S_r = gam(r-1) S_(r-1) + K_(r-1)^T Cs_(r-1), then its parts; Cs comes
      // as its three bf16 parts (the chain wave splits it once for all four
      // state waves)
      struct CsParts {
        uint2 l, m, h;
      };
      auto cs_parts = [&](int sl) {
        if constexpr (NSP == 3) return CsParts{scp[sl][0][lane], scp[sl][1][lane], scp[sl][2][lane]};
        else return CsParts{scp[sl][0][lane], make_uint2(0u, 0u), scp[sl][1][lane]};
      };
      auto update = [&](const CsParts& c, const Ops& o) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          v4f acc = St[ct] * o.gl;
          if constexpr (NPART == 1 && NSP == 2) {
            // k's four tokens twice against the two parts of Cs side by side:
            // one 16x16x32 product for two 16x16x16 ones
            const uint4 kk = make_uint4(o.kt[ct].x, o.kt[ct].y, o.kt[ct].x, o.kt[ct].y);
            St[ct] = mm32bf(kk, make_uint4(c.l.x, c.l.y, c.h.x, c.h.y), acc);
          } else if constexpr (NPART == 1) {
            // three parts: three 16x16x16 products (a 16x16x16 product must not
            // take a 16x16x32 one's result as its accumulator straight away)
            acc = mm16<GDN_BF16>(o.kt[ct], c.l, acc);
            acc = mm16<GDN_BF16>(o.kt[ct], c.m, acc);
            St[ct] = mm16<GDN_BF16>(o.kt[ct], c.h, acc);
          } else {
            // one 16x16x32 product per part of Cs: k's hi and lo parts
            // against the same four tokens of Cs
            acc = mm32bf(o.kt[ct], make_uint4(c.l.x, c.l.y, c.l.x, c.l.y), acc);
            if constexpr (NSP == 3)
              acc = mm32bf(o.kt[ct], make_uint4(c.m.x, c.m.y, c.m.x, c.m.y), acc);
            St[ct] = mm32bf(o.kt[ct], make_uint4(c.h.x, c.h.y, c.h.x, c.h.y), acc);
          }
        }
        split_state();
      };
      // round r >= 1: bq holds block r, bk block r + 1; cur holds round r's
      // update operands and then takes K_(r+1)^T for round r + 2, nxt takes
      // gam(r); bq then takes the loads of block r + 4
      auto round = [&](int64_t r, Ops& cur, Ops& nxt, Blk& bq, const Blk& bk) {
        __syncthreads();
        const CsParts cs = cs_parts((int)((r - 1) & 1));
        nxt.gl = srec[r & 3][kRecGl];
        uint4 qp[NPART], kp[NPART];
        parts(bq.q, qp);
        parts(bk.k, kp);
        sp[r & 1][cp][lane] = xst(qp);
        sb[(r + 1) & 1][cp][lane] = xst(kp);
        update(cs, cur);
        transpose(kp, cur.kt);
        reload(bq, r + 4);
      };
      Ops o0, o1;
      Blk b0, b1, b2, b3;
      ld(b0, 0);
      ld(b1, clampb(1));
      ld(b2, clampb(2));
      ld(b3, clampb(3));
      split_state();
      __syncthreads();  // blocks 0 and 1 staged
      uint4 qp[NPART], kp[NPART];
      parts(b0.k, kp);
      sb[0][cp][lane] = xst(kp);  // A_0
      transpose(kp, o1.kt);       // K_0^T for round 1
      __syncthreads();
      // round 0: P_0 and B_1 from S_0, no update
      o1.gl = srec[0][kRecGl];
      parts(b0.q, qp);
      sp[0][cp][lane] = xst(qp);
      parts(b1.k, kp);
      sb[1][cp][lane] = xst(kp);
      transpose(kp, o0.kt);  // K_1^T for round 2
      reload(b0, 4);
      // rounds in fours (the ring of four sets), then up to three more
      const int64_t nq = (nblk - 1) / 4, rm = (nblk - 1) % 4;
      for (int64_t p = 0; p < nq; ++p) {
        round(4 * p + 1, o1, o0, b1, b2);
        round(4 * p + 2, o0, o1, b2, b3);
        round(4 * p + 3, o1, o0, b3, b0);
        round(4 * p + 4, o0, o1, b0, b1);
      }
      if (rm >= 1) round(4 * nq + 1, o1, o0, b1, b2);
      if (rm >= 2) round(4 * nq + 2, o0, o1, b2, b3);
      if (rm >= 3) round(4 * nq + 3, o1, o0, b3, b0);
      __syncthreads();
      update(cs_parts((int)((nblk - 1) & 1)), ((nblk - 1) & 1) ? o0 : o1);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        *reinterpret_cast<float4*>(a.s_out + soff + 4 * ct) =
            make_float4(St[ct][0], St[ct][1], St[ct][2], St[ct][3]);
      return;
    }
  }
  if constexpr (DT == GDN_F32 && D > 128) if (wave < NC) {
    // ---- state waves, f32 inputs at D = 256: the products of the branch
    // below (f32 16x16x4), two key tiles of the 16 rows per wave, with q and
    // k loaded by the wave itself from global memory, two blocks ahead in a
    // ring of two register sets (LDS would need 133 KB for the f32 rows, and
    // three waves per SIMD leave no registers for a deeper ring);
    // K^T for the update is formed from the loaded rows on the matrix cores:
    // four products per tile against slices of the identity (X E exactly;
    // lane (lg, lc) then holds X[4 lg + r][lc]).
    constexpr int NT4 = D / (16 * NC);
    v4f St[NT4];
    const int arow = row0 + lc;
    auto key0 = [&](int ct) { return 16 * (cp * NT4 + ct) + 4 * lg; };
#pragma unroll
    for (int ct = 0; ct < NT4; ++ct) {
      const float4 x = *reinterpret_cast<const float4*>(a.s0 + sbase + (int64_t)arow * D + key0(ct));
      St[ct] = v4f{x.x, x.y, x.z, x.w};
    }
    // q and k of a block: row lc, keys key0(ct) .. + 3 (rows past the last
    // token repeat it)
    struct Blk {
      float4 q[NT4], k[NT4];
    };
    auto ld = [&](Blk& x, int64_t c) {
      const int tcc = c == nblk - 1 ? tcl : kL;
      const int64_t o = bs.qk + (c * kL + (lc < tcc ? lc : tcc - 1)) * bs.qk_ts;
#pragma unroll
      for (int ct = 0; ct < NT4; ++ct) {
        x.q[ct] = *reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + o + key0(ct));
        x.k[ct] = *reinterpret_cast<const float4*>(static_cast<const float*>(a.k) + o + key0(ct));
      }
    };
    // the next loads of a set stay below its last use (see the 16-bit branch)
    auto reload = [&](Blk& x, int64_t c) {
      __builtin_amdgcn_sched_barrier(0);
      int64_t cn = clampb(c);
      asm volatile("" : "+s"(cn) : : "memory");
      ld(x, cn);
    };
    // X S^T over the wave's key tiles: two chains of dependent products
    auto xst = [&](const float4* f) {
      v4f p[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ct = 0; ct < NT4; ++ct) {
        v4f& acc = p[ct & 1];
        acc = mfma4(f[ct].x, St[ct][0], acc);
        acc = mfma4(f[ct].y, St[ct][1], acc);
        acc = mfma4(f[ct].z, St[ct][2], acc);
        acc = mfma4(f[ct].w, St[ct][3], acc);
      }
      return p[0] + p[1];
    };
    // E_e[kk][j] = (4 kk + e == j): lane (lg, lc) holds E_e[lg][lc]
    float eye[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) eye[e] = 4 * lg + e == lc ? 1.f : 0.f;
    struct Ops {
      float kt[NT4][4];
      float gl;
    };
    auto transpose = [&](const float4* f, Ops& o) {
#pragma unroll
      for (int ct = 0; ct < NT4; ++ct) {
        v4f d = {0.f, 0.f, 0.f, 0.f};
        d = mfma4(f[ct].x, eye[0], d);
        d = mfma4(f[ct].y, eye[1], d);
        d = mfma4(f[ct].z, eye[2], d);
        d = mfma4(f[ct].w, eye[3], d);
#pragma unroll
        for (int r = 0; r < 4; ++r) o.kt[ct][r] = d[r];
      }
    };
    // S_r = gam(r-1) S_(r-1) + K_(r-1)^T Cs_(r-1)
    auto update = [&](const v4f& cs, const Ops& o) {
#pragma unroll
      for (int ct = 0; ct < NT4; ++ct) {
        v4f acc = St[ct] * o.gl;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = mfma4(o.kt[ct][s2], cs[s2], acc);
        St[ct] = acc;
      }
    };
    // round r >= 1: bq holds block r, bk block r + 1; cur holds round r's
    // update operands and then takes K_(r+1)^T for round r + 2, nxt takes
    // gam(r); bq then takes the loads of block r + 2
    auto round = [&](int64_t r, Ops& cur, Ops& nxt, Blk& bq, const Blk& bk) {
      __syncthreads();
      const v4f cs = scs[(r - 1) & 1][lane];
      nxt.gl = srec[r & 3][kRecGl];
      sp[r & 1][cp][lane] = xst(bq.q);
      sb[(r + 1) & 1][cp][lane] = xst(bk.k);
      update(cs, cur);
      transpose(bk.k, cur);
      reload(bq, r + 2);
    };
    Ops o0, o1;
    Blk b0, b1;
    ld(b0, 0);
    ld(b1, clampb(1));
    __syncthreads();  // blocks 0 and 1 staged
    sb[0][cp][lane] = xst(b0.k);  // A_0
    transpose(b0.k, o1);           // K_0^T for round 1
    __syncthreads();
    // round 0: P_0 and B_1 from S_0, no update
    o1.gl = srec[0][kRecGl];
    sp[0][cp][lane] = xst(b0.q);
    sb[1][cp][lane] = xst(b1.k);
    transpose(b1.k, o0);  // K_1^T for round 2
    reload(b0, 2);
    // rounds in pairs (two register sets, two operand sets), then one more
    const int64_t npair = (nblk - 1) / 2;
    for (int64_t p = 0; p < npair; ++p) {
      round(2 * p + 1, o1, o0, b1, b0);
      round(2 * p + 2, o0, o1, b0, b1);
    }
    if ((nblk - 1) & 1) round(nblk - 1, o1, o0, b1, b0);
    __syncthreads();
    update(scs[(nblk - 1) & 1][lane], ((nblk - 1) & 1) ? o0 : o1);
#pragma unroll
    for (int ct = 0; ct < NT4; ++ct) {
      float4 x = make_float4(St[ct][0], St[ct][1], St[ct][2], St[ct][3]);
      *reinterpret_cast<float4*>(a.s_out + sbase + (int64_t)arow * D + key0(ct)) = x;
    }
    return;
  }
  if constexpr (DT == GDN_F32 && D <= 128) if (wave < NC) {
    // ---- state waves, f32 inputs: two key tiles of the 16 rows,
    // accumulator layout
    v4f St[NCT];
    const int arow = row0 + lc;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float4 x = *reinterpret_cast<const float4*>(a.s0 + sbase + (int64_t)arow * D +
                                                        16 * (cp * NCT + ct) + 4 * lg);
      St[ct] = v4f{x.x, x.y, x.z, x.w};
    }
    // Operand fragments of the 16 rows X of a slot (raw q or k) for X S^T
    typedef float4 Frag;
    auto frag = [&](const KT (*x)[KP], Frag* f) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        f[ct] = *reinterpret_cast<const float4*>(&x[lc][16 * (cp * NCT + ct) + 4 * lg]);
    };
    // as A-operand fragments
    auto widen = [&](const Frag* f, v4f* w) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) w[ct] = v4f{f[ct].x, f[ct].y, f[ct].z, f[ct].w};
    };
    // X S^T over this wave's key tiles
    auto xst = [&](const v4f* f) {
      v4f p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
      p0 = mfma4(f[0][0], St[0][0], p0);
      p1 = mfma4(f[1][0], St[1][0], p1);
      p0 = mfma4(f[0][1], St[0][1], p0);
      p1 = mfma4(f[1][1], St[1][1], p1);
      p0 = mfma4(f[0][2], St[0][2], p0);
      p1 = mfma4(f[1][2], St[1][2], p1);
      p0 = mfma4(f[0][3], St[0][3], p0);
      p1 = mfma4(f[1][3], St[1][3], p1);
      return p0 + p1;
    };
    // operands of round r, read in round r - 1 (staged at least a round
    // before that): Q_r, K_(r-1) in the update's layout, gam(r-1)
    struct Ops {
      Frag qf[NCT];
      float kt[NCT][4];
      float gl;
    };
    auto fetch = [&](int64_t r, Ops& o) {
      const int sp_ = (int)((r - 1) & 3);
      frag(sq[r & 3], o.qf);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) o.kt[ct][s2] = sk[sp_][4 * lg + s2][16 * (cp * NCT + ct) + lc];
      o.gl = srec[sp_][kRecGl];
    };
    // S_r = gam(r-1) S_(r-1) + K_(r-1)^T Cs_(r-1)
    auto update = [&](const v4f& cs, const Ops& o) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const v4f kt = v4f{o.kt[ct][0], o.kt[ct][1], o.kt[ct][2], o.kt[ct][3]};
        v4f acc = St[ct] * o.gl;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = mfma4(kt[s2], cs[s2], acc);
        St[ct] = acc;
      }
    };
    // round r >= 1: cur holds round r's operands, nxt takes round r + 1's
    auto round = [&](int64_t r, const Ops& cur, Ops& nxt) {
      __syncthreads();
      const v4f cs = scs[(r - 1) & 1][lane];
      Frag kf[NCT];
      frag(sk[(r + 1) & 3], kf);
      fetch(r + 1, nxt);
      v4f qw[NCT], kw[NCT];
      widen(cur.qf, qw);
      sp[r & 1][cp][lane] = xst(qw);
      widen(kf, kw);
      sb[(r + 1) & 1][cp][lane] = xst(kw);
      update(cs, cur);
    };
    Ops o0, o1;
    Frag kf[NCT];
    v4f kw[NCT], qw[NCT];
    __syncthreads();  // blocks 0 and 1 staged
    frag(sk[0], kf);
    widen(kf, kw);
    sb[0][cp][lane] = xst(kw);  // A_0
    fetch(0, o0);               // Q_0 (its K and gam parts are not used)
    __syncthreads();
    // round 0: P_0 and B_1 from S_0, no update
    frag(sk[1], kf);
    fetch(1, o1);
    widen(o0.qf, qw);
    sp[0][cp][lane] = xst(qw);
    widen(kf, kw);
    sb[1][cp][lane] = xst(kw);
    const int64_t npair = (nblk - 1) / 2;
    for (int64_t p = 0; p < npair; ++p) {
      round(1 + 2 * p, o1, o0);
      round(2 + 2 * p, o0, o1);
    }
    if ((nblk - 1) & 1) round(nblk - 1, o1, o0);
    __syncthreads();
    update(scs[(nblk - 1) & 1][lane], ((nblk - 1) & 1) ? o0 : o1);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float4 x = make_float4(St[ct][0], St[ct][1], St[ct][2], St[ct][3]);
      *reinterpret_cast<float4*>(a.s_out + sbase + (int64_t)arow * D + 16 * (cp * NCT + ct) +
                                 4 * lg) = x;
    }
    return;
  }

  if (wave == NC) {
    // ---- chain wave: C of block r.  K_r S_r^T = gam(r-1) (gam(r-2) sum B_r
    // + Y_r) + M1_r Cs_(r-1); the last term is formed at the start of round
    // r, the record of block r read at the start of round r - 1.  With two
    // bf16 parts (BFCHAIN) both products run as three 16x16x16 bf16 products
    // over the rounded parts (hi.hi + hi.lo + lo.hi; the prep writes T and M1
    // as parts, this wave splits Y and Cs), instead of four f32 16x16x4 ones
    // each: the SIMD's issue is shared with a state wave.
    __builtin_amdgcn_s_setprio(3);  // ahead of the state wave on its SIMD
    struct Cops {
      float4 tf, m1;
      uint2 th, tl, mh, ml;
      float be[4], wsc[4], srs[4], v[4];
      float g1, g2;
      v4f mc;
    };
    v4f csp = {0.f, 0.f, 0.f, 0.f};
    uint2 cph = make_uint2(0u, 0u), cpl = make_uint2(0u, 0u);  // csp's parts (BFCHAIN)
    auto fetch = [&](int64_t r, Cops& o, float g1, float g2) {
      const int s = (int)(r & 3);
      if constexpr (BFCHAIN) {  // T[lc][4 lg ..] and M1[lc][4 lg ..]: four hi, four lo
        const uint4 t = *reinterpret_cast<const uint4*>(&srec[s][kRecT + 16 * lc + 4 * lg]);
        const uint4 m = *reinterpret_cast<const uint4*>(&smx[s][16 * lc + 4 * lg]);
        o.th = make_uint2(t.x, t.y);
        o.tl = make_uint2(t.z, t.w);
        o.mh = make_uint2(m.x, m.y);
        o.ml = make_uint2(m.z, m.w);
      } else {
        o.tf = *reinterpret_cast<const float4*>(&srec[s][kRecT + 16 * lc + 4 * lg]);
        o.m1 = *reinterpret_cast<const float4*>(&smx[s][16 * lc + 4 * lg]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o.be[i] = srec[s][kRecBe + 4 * lg + i];
        o.wsc[i] = srec[s][kRecWsc + 4 * lg + i];
        o.srs[i] = srec[s][kRecSrs + 4 * lg + i];
        o.v[i] = sv[s][4 * lg + i][lc];
      }
      o.g1 = g1;
      o.g2 = g2;
    };
    auto step = [&](int64_t r, const Cops& o, const v4f& bsum, const v4f& y) {
      v4f yv;  // beta V - (beta gam rk) K S^T
#pragma unroll
      for (int i = 0; i < 4; ++i)
        yv[i] = o.be[i] * o.v[i] - o.wsc[i] * fmaf(o.g1, fmaf(o.g2, bsum[i], y[i]), o.mc[i]);
      v4f cc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BFCHAIN) {
        const Bf2 y0 = split_bf2(yv[0], yv[1]), y1 = split_bf2(yv[2], yv[3]);
        const uint2 yh = make_uint2(y0.h, y1.h), yl = make_uint2(y0.l, y1.l);
        cc = mm16<GDN_BF16>(o.tl, yh, cc);
        cc = mm16<GDN_BF16>(o.th, yl, cc);
        cc = mm16<GDN_BF16>(o.th, yh, cc);
      } else {
        const float4 tf = o.tf;
        cc = mfma4(tf.x, yv[0], cc);
        cc = mfma4(tf.y, yv[1], cc);
        cc = mfma4(tf.z, yv[2], cc);
        cc = mfma4(tf.w, yv[3], cc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) csp[i] = cc[i] * o.srs[i];
      if constexpr (!BFCHAIN) scs[r & 1][lane] = csp;  // (BFCHAIN: Y and Z take its parts)
      scc[r & 1][lane] = cc;
      if constexpr (DT != GDN_F32 && NSP == 3) {
        const Bf3 p0 = split_bf3(csp[0], csp[1]), p1 = split_bf3(csp[2], csp[3]);
        scp[r & 1][0][lane] = make_uint2(p0.l, p1.l);
        scp[r & 1][1][lane] = make_uint2(p0.m, p1.m);
        scp[r & 1][2][lane] = make_uint2(p0.h, p1.h);
      } else if constexpr (DT != GDN_F32) {
        const Bf2 p0 = split_bf2(csp[0], csp[1]), p1 = split_bf2(csp[2], csp[3]);
        cpl = make_uint2(p0.l, p1.l);
        cph = make_uint2(p0.h, p1.h);
        scp[r & 1][0][lane] = cpl;
        scp[r & 1][1][lane] = cph;
      }
    };
    auto m1cs = [&](Cops& o) {  // M1 of o's block times the newest Cs (the one before)
      v4f d = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BFCHAIN) {
        d = mm16<GDN_BF16>(o.ml, cph, d);
        d = mm16<GDN_BF16>(o.mh, cpl, d);
        d = mm16<GDN_BF16>(o.mh, cph, d);
      } else {
        d = mfma4(o.m1.x, csp[0], d);
        d = mfma4(o.m1.y, csp[1], d);
        d = mfma4(o.m1.z, csp[2], d);
        d = mfma4(o.m1.w, csp[3], d);
      }
      o.mc = d;
    };
    auto bparts = [&](int64_t r) { return sum_parts<NC>(sb[r & 1], lane); };
    // M1_r Cs_(r-1) goes right after the barrier, in the shadow of the
    // round's LDS reads, rather than in front of the barrier
    auto round = [&](int64_t r, Cops& cur, Cops& nxt) {
      __syncthreads();
      const v4f bsum = bparts(r);
      const v4f y = sy[r & 1][lane];
      fetch(r + 1, nxt, srec[r & 3][kRecGl], srec[(r - 1) & 3][kRecGl]);
      m1cs(cur);
      step(r, cur, bsum, y);
    };
    Cops c0, c1;
    __syncthreads();  // blocks 0 and 1 staged
    fetch(0, c0, 1.f, 1.f);
    c0.mc = v4f{0.f, 0.f, 0.f, 0.f};
    __syncthreads();  // A_0 formed
    {
      const v4f bsum = bparts(0);
      fetch(1, c1, srec[0][kRecGl], 1.f);
      step(0, c0, bsum, v4f{0.f, 0.f, 0.f, 0.f});
    }
    const int64_t npair = (nblk - 1) / 2;
    for (int64_t p = 0; p < npair; ++p) {
      round(1 + 2 * p, c1, c0);
      round(2 + 2 * p, c0, c1);
    }
    if ((nblk - 1) & 1) round(nblk - 1, c1, c0);
    __syncthreads();
    return;
  }

  if (wave == NC + 1) {
    // ---- O and y of the previous block.  This wave loads nothing: with
    // only stores in its memory queue it never waits on it.
    // O_c = diag(gam rq) (gam(c-1) sum P_c + Z_c) + Hd C_c: lane (lg, lc)
    // register i is token 4 lg + i, row lc
    auto o_block = [&](int64_t cb, float g) {
      const int s = (int)(cb & 3), ob = (int)(cb & 1);
      const v4f pq = sum_parts<NC>(sp[ob], lane);
      const v4f z = sz[ob][lane];
      const v4f cc = scc[ob][lane];
      v4f o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = srec[s][kRecSig + 4 * lg + i] * fmaf(g, pq[i], z[i]);
      if constexpr (BFCHAIN) {  // Hd as parts (prep), C split here: three bf16 products
        const uint4 hp = *reinterpret_cast<const uint4*>(&srec[s][kRecH + 16 * lc + 4 * lg]);
        const Bf2 c0 = split_bf2(cc[0], cc[1]), c1 = split_bf2(cc[2], cc[3]);
        const uint2 ch = make_uint2(c0.h, c1.h), cl = make_uint2(c0.l, c1.l);
        o = mm16<GDN_BF16>(make_uint2(hp.z, hp.w), ch, o);
        o = mm16<GDN_BF16>(make_uint2(hp.x, hp.y), cl, o);
        o = mm16<GDN_BF16>(make_uint2(hp.x, hp.y), ch, o);
      } else {
        const float4 hf = *reinterpret_cast<const float4*>(&srec[s][kRecH + 16 * lc + 4 * lg]);
        o = mfma4(hf.x, cc[0], o);
        o = mfma4(hf.y, cc[1], o);
        o = mfma4(hf.z, cc[2], o);
        o = mfma4(hf.w, cc[3], o);
      }
      return o;
    };
    auto o_store = [&](int64_t cb, const v4f& o, int tc) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * lg + i < tc) a.y[bs.v + (cb * kL + 4 * lg + i) * bs.v_ts + row0 + lc] = o[i];
    };
    __syncthreads();  // blocks 0 and 1 staged
    __syncthreads();  // A_0 formed
    float g = 1.f;    // gam(r-2) in round r
    for (int64_t r = 1; r < nblk; ++r) {
      __syncthreads();
      const float gn = srec[(r - 1) & 3][kRecGl];
      o_store(r - 1, o_block(r - 1, g), kL);
      g = gn;
    }
    __syncthreads();
    o_store(nblk - 1, o_block(nblk - 1, g), tc_of(nblk - 1));
    return;
  }

  // ---- waves 6 and 7: the staging, and Y (wave 6) or Z (wave 7).  Lane st:
  // q and k of token st / 8, elements 16 (st % 8) .. + 15 (not with bf16
  // inputs: the state waves load their own); two v values; two float4 of the
  // record and of M1 M2 N.
  constexpr int NR4 = kRecUsed / 4, NM4 = NM / 4;
  constexpr bool QK = DT == GDN_F32 && D <= 128;
  struct Regs {
    Raw<DT, 8> k[2], q[2];
    Raw<DT, 2> v;
    Raw<GDN_F32, 4> r[2], m[2];
  };
  const int st = tid - (NC + 2) * kWave;
  // f32 q and k: CPR chunks of 16 elements per row, a chunk per lane (lanes
  // past the kL * CPR chunks load the last one and do not write it); v: two
  // values of one token per lane
  constexpr int CPR = D / 16;
  constexpr bool QKALL = kL * CPR >= 2 * kWave;  // every staging lane writes a chunk
  const int sqi = st < kL * CPR ? st : kL * CPR - 1;
  const int qtt = sqi / CPR, qc = 16 * (sqi % CPR), vtt = st / 8, vr = 2 * (st % 8);
  int rec_e[2], mx_e[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    rec_e[u] = 4 * (st + 2 * kWave * u < NR4 ? st + 2 * kWave * u : NR4 - 1);
    mx_e[u] = 4 * (st + 2 * kWave * u < NM4 ? st + 2 * kWave * u : NM4 - 1);
  }
  // branch-free addresses (a branch here splits the loop body, and the
  // registers of a load then no longer carry over the loop edge)
  auto load = [&](Regs& P, int64_t c) {
    const int tcc = c == nblk - 1 ? tcl : kL;  // tokens in block c
    const int64_t t = c * kL + (qtt < tcc ? qtt : tcc - 1);
    const int64_t tv = c * kL + (vtt < tcc ? vtt : tcc - 1);
    const int64_t o = bs.qk + t * bs.qk_ts + qc;
    if constexpr (QK) {
      P.k[0].load(a.k, o);
      P.k[1].load(a.k, o + 8);
      P.q[0].load(a.q, o);
      P.q[1].load(a.q, o + 8);
    }
    P.v.load(a.v, bs.v + tv * bs.v_ts + row0 + vr);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      P.r[u].load(rec, c * kRec + rec_e[u]);
      P.m[u].load(mxh, c * NM + mx_e[u]);
    }
  };
  // the loaded words pass through an empty asm first: the conversions for
  // the LDS writes then stay below the barrier before them (hoisted above
  // it, they would wait on the loads a round early)
  auto pin = [](auto& raw) {
#pragma unroll
    for (int i = 0; i < (int)(sizeof(raw.w) / sizeof(raw.w[0])); ++i) asm volatile("" : "+v"(raw.w[i]));
  };
  // each LDS element is written once (the clamped lanes load but do not write)
  auto store = [&](Regs& P, int sl) {
    if constexpr (QK) {
      pin(P.k[0]);
      pin(P.k[1]);
      pin(P.q[0]);
      pin(P.q[1]);
    }
    pin(P.v);
    pin(P.r[0]);
    pin(P.r[1]);
    pin(P.m[0]);
    pin(P.m[1]);
    if (QKALL || st < kL * CPR) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (DT == GDN_F32 && QK) {
          *reinterpret_cast<float4*>(&sk[sl][qtt][qc + 8 * h]) = P.k[h].get4(0);
          *reinterpret_cast<float4*>(&sk[sl][qtt][qc + 8 * h + 4]) = P.k[h].get4(1);
          *reinterpret_cast<float4*>(&sq[sl][qtt][qc + 8 * h]) = P.q[h].get4(0);
          *reinterpret_cast<float4*>(&sq[sl][qtt][qc + 8 * h + 4]) = P.q[h].get4(1);
        } else if constexpr (QK) {
          *reinterpret_cast<uint4*>(&sk[sl][qtt][qc + 8 * h]) =
              make_uint4(P.k[h].w[0], P.k[h].w[1], P.k[h].w[2], P.k[h].w[3]);
          *reinterpret_cast<uint4*>(&sq[sl][qtt][qc + 8 * h]) =
              make_uint4(P.q[h].w[0], P.q[h].w[1], P.q[h].w[2], P.q[h].w[3]);
        }
      }
    }
    *reinterpret_cast<float2*>(&sv[sl][vtt][vr]) = make_float2(P.v.get(0), P.v.get(1));
    *reinterpret_cast<float4*>(&srec[sl][rec_e[0]]) = P.r[0].get4(0);
    if (st + 2 * kWave < NR4) *reinterpret_cast<float4*>(&srec[sl][rec_e[1]]) = P.r[1].get4(0);
    *reinterpret_cast<float4*>(&smx[sl][mx_e[0]]) = P.m[0].get4(0);
    if (st + 2 * kWave < NM4) *reinterpret_cast<float4*>(&smx[sl][mx_e[1]]) = P.m[1].get4(0);
  };
  // P's loads are kept below its LDS writes: its registers then carry over
  // the loop edge, and no copy there waits for the loads of the last round.
  // (The inputs are read-only, so the compiler would otherwise hoist the
  // loads across the writes and the barrier; the block index passes through
  // an empty asm after the writes.)
  auto restage = [&](Regs& P, int sl, int64_t c) {
    store(P, sl);
    __builtin_amdgcn_sched_barrier(0);
    int64_t cn = clampb(c);
    asm volatile("" : "+s"(cn) : : "memory");
    load(P, cn);
  };
  const bool ywave = wave == NC + 2;
  // round r >= 1: Y_(r+1) = M2_(r+1) Cs_(r-1) (wave 6) or Z_r = N_r Cs_(r-1)
  // (wave 7); P holds block r + 2, loaded three rounds before (right after
  // its previous contents went to LDS, so two whole rounds hide the load
  // latency); it goes to its slot, then takes the loads of block r + 5.
  // Three register sets in turn, the loop unrolled by three.
  // The two LDS reads go first, the block's LDS writes right behind them,
  // and the products last: the writes, the longer part, then start at the
  // barrier instead of after the products.
  auto round = [&](int64_t r, Regs& P) {
    __syncthreads();
    const float* m = ywave ? &smx[(r + 1) & 3][kL * kL] : &smx[r & 3][2 * kL * kL];
    v4f d = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BFCHAIN) {
      // M2 or N as two bf16 parts (prep), Cs as its parts (chain wave):
      // three 16x16x16 bf16 products
      const uint2 cl = scp[(r - 1) & 1][0][lane], ch = scp[(r - 1) & 1][1][lane];
      const uint4 mp = *reinterpret_cast<const uint4*>(&m[16 * lc + 4 * lg]);
      restage(P, (int)((r + 2) & 3), r + 5);
      d = mm16<GDN_BF16>(make_uint2(mp.z, mp.w), ch, d);
      d = mm16<GDN_BF16>(make_uint2(mp.x, mp.y), cl, d);
      d = mm16<GDN_BF16>(make_uint2(mp.x, mp.y), ch, d);
    } else {
      const v4f cs = scs[(r - 1) & 1][lane];
      const float4 mf = *reinterpret_cast<const float4*>(&m[16 * lc + 4 * lg]);
      restage(P, (int)((r + 2) & 3), r + 5);
      d = mfma4(mf.x, cs[0], d);
      d = mfma4(mf.y, cs[1], d);
      d = mfma4(mf.z, cs[2], d);
      d = mfma4(mf.w, cs[3], d);
    }
    if (ywave) sy[(r + 1) & 1][lane] = d;
    else sz[r & 1][lane] = d;
  };
  Regs P0, P1, P2;
  load(P0, 0);
  load(P1, clampb(1));
  store(P0, 0);
  store(P1, 1);
  load(P0, clampb(2));
  load(P1, clampb(3));
  load(P2, clampb(4));
  __syncthreads();  // blocks 0 and 1 staged
  __syncthreads();  // A_0 formed
  // round 0: Y_1 = Z_0 = 0 (no C-scaled before block 0)
  restage(P0, 2, 5);
  if (ywave) sy[1][lane] = v4f{0.f, 0.f, 0.f, 0.f};
  else sz[0][lane] = v4f{0.f, 0.f, 0.f, 0.f};
  // nothing but the loads of blocks 3 to 5 in flight on entry, and no exit
  // inside the loop body
  const int64_t ntri = (nblk - 1) / 3, rem = (nblk - 1) % 3;
  for (int64_t p = 0; p < ntri; ++p) {
    round(1 + 3 * p, P1);
    round(2 + 3 * p, P2);
    round(3 + 3 * p, P0);
  }
  if (rem >= 1) round(1 + 3 * ntri, P1);
  if (rem >= 2) round(2 + 3 * ntri, P2);
  __syncthreads();
}

template <int DT, int GT, int D, bool TP>
void launch_prep_gt(const PrepArgs& p, dim3 grid, hipStream_t st) {
  if (p.mx != nullptr) prep_kernel<DT, GT, D, true, TP><<<grid, 256, 0, st>>>(p);
  else if constexpr (D <= 128) prep_kernel<DT, GT, D, false, false><<<grid, 256, 0, st>>>(p);
}

template <int DT, int D, bool TP>
int launch_prep(const PrepArgs& p, int gdt, dim3 grid, hipStream_t st) {
  switch (gdt) {
    case GDN_F32: launch_prep_gt<DT, GDN_F32, D, TP>(p, grid, st); break;
    case GDN_F16: launch_prep_gt<DT, GDN_F16, D, TP>(p, grid, st); break;
    default: launch_prep_gt<DT, GDN_BF16, D, TP>(p, grid, st); break;
  }
  return device_status("prep_kernel launch");
}

template <int DT, int NSP, int D>
int launch_dt(const gdn_desc& d, const PrepArgs& p, const StateArgs& s, int64_t heads,
              hipStream_t st) {
  const int64_t pblocks = (p.ntask + 3) / 4;
  const bool rows = D > 128 || scan_uses_key_products(d);
  if (!launch_fits(pblocks, 256, "prep_kernel") ||
      !(rows ? launch_fits(heads * (D / 16), rows_la_threads<DT, D>(), "rows_la_kernel")
             : launch_fits(heads, 4 * D, "state_kernel")))
    return GDN_ESHAPE;
  const dim3 pgrid((unsigned)pblocks);
  // the few-head kernel's default products take T and M1 as bf16 parts
  const int rc = launch_prep<DT, D, DT != GDN_F32 && NSP == 2>(p, d.gate_dtype, pgrid, st);
  if (rc != GDN_OK) return rc;
  // many heads: whole-head workgroups, the norm fused; few heads (and D =
  // 256, whose whole-head state would overflow the registers): a workgroup
  // per 16 value rows with the one-block lookahead
  StateArgs r = s;
  if constexpr (D <= 128) {
    if (!scan_uses_key_products(d)) {
      r.nrb = 1;
      state_kernel<DT, NSP, D><<<dim3((unsigned)heads), 4 * D, 0, st>>>(r);
      return device_status("state_kernel launch");
    }
  }
  r.nrb = D / 16;
  rows_la_kernel<DT, NSP, D><<<dim3((unsigned)(heads * r.nrb)), rows_la_threads<DT, D>(), 0, st>>>(r);
  return device_status("rows_la_kernel launch");
}

template <int DT, int NSP>
int launch_d(const gdn_desc& d, const PrepArgs& p, const StateArgs& s, int64_t heads,
             hipStream_t st) {
  switch (d.Dk) {
    case 32: return launch_dt<DT, NSP, 32>(d, p, s, heads, st);
    case 64: return launch_dt<DT, NSP, 64>(d, p, s, heads, st);
    case 256: return launch_dt<DT, NSP, 256>(d, p, s, heads, st);
    default: return launch_dt<DT, NSP, 128>(d, p, s, heads, st);
  }
}

}  // namespace

// The block-form scan at the head dims block_form_fits admits; y receives the
// raw o (the gated norm, when asked for and not fused, runs after it).  Returns whether the gated output
// was written (fused) through *gated.  The block records (and, for few heads,
// the cross-block key products) live in the caller's workspace, laid out as
// scan_workspace_bytes() sizes it: records first, then the key products.
int launch_scan_chunked(const gdn_desc& d, const void* q, const void* k, const void* v,
                        const void* ld, const void* beta, const float* s0, const void* z,
                        const void* w, float* y, float* s_out, void* workspace, void* stream,
                        bool* gated) {
  static_assert(kRec * sizeof(float) == kBlockRecordBytes, "record size");
  static_assert(kL == kBlockTokens, "block length");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t heads = d.B * d.Hv, nblk = (d.T + kL - 1) / kL;
  *gated = !scan_uses_key_products(d);
  float* rec = static_cast<float*>(workspace);
  float* mx = *gated ? nullptr : rec + scan_record_bytes(d) / (int64_t)sizeof(float);
  const PrepArgs p{q, k, ld, beta, rec, d.T, nblk, d.B * d.Hk * nblk, (int)d.Hk, (int)d.Hv,
                   (int)(d.Hv / d.Hk), d.head_major, d.flags, d.qk_eps, q_scale(d), mx};
  const StateArgs s{q, k, v, z, w, rec, s0, y, s_out, d.T, nblk, (int)d.Hk, (int)d.Hv,
                    (int)(d.Hv / d.Hk), 1, d.head_major, d.norm_eps, mx};
  // 16-bit inputs: the state and Cs in two rounded bf16 parts, or three
  // exact ones with GDN_SCAN_EXACT; f32 inputs use f32 products either way
  const bool exact = (d.flags & GDN_SCAN_EXACT) != 0;
  switch (d.dtype) {
    case GDN_F32: return launch_d<GDN_F32, 3>(d, p, s, heads, st);
    case GDN_F16:
      return exact ? launch_d<GDN_F16, 3>(d, p, s, heads, st)
                   : launch_d<GDN_F16, 2>(d, p, s, heads, st);
    default:
      return exact ? launch_d<GDN_BF16, 3>(d, p, s, heads, st)
                   : launch_d<GDN_BF16, 2>(d, p, s, heads, st);
  }
}

}  // namespace gdn

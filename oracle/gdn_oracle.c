/*
 * gdn_oracle.c -- slow, plain float64 CPU oracle of the Gated DeltaNet (GDN)
 * recurrence.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this library.  It shares no code, header,
 * table or helper with the HIP implementation, and it never reads anything the
 * HIP path produced.
 *
 * What it computes (the pages, cited by page title and section):
 *   - "Module gdn" (logicaffeine codegen_cuda/gdn), module description: each
 *     value head keeps a D x D memory S; per token u = S.k, then
 *     S = alpha*S + beta*(v - alpha*u) k^T, then o = S.q taken after that
 *     update (the memory of this token, not the previous one), then
 *     o = rmsnorm(o * silu(z)) * GN with the gate multiplied in before the
 *     normalisation.
 *   - Same page, "The fusion": unfused, a token visits S three times (the
 *     product with k, the rank-1 update, the product with q).  This oracle
 *     makes exactly those three visits, on purpose, so that the fused kernels
 *     are checked against the unfused definition.
 *   - "gated_delta" (torch-to-nnef op reference), native_gdn_reject_reason: the
 *     fused decode operator folds the q/k L2 norm and the 1/sqrt(head_dim)
 *     scale; l2norm: the L2 normalisation of the last axis uses HF's eps.
 *   - Same page, emit_native_gdn_recurrent: operands (q, k, v, log_decay, beta,
 *     s0); token-major layout [B, S, H, W] for q/k/v, [B, S, H] for log_decay
 *     and beta; state [B, H, W, W]; outputs (output, final_state).
 *
 * Readings taken where the pages leave a step open:
 *   - alpha = exp(log_decay); beta is used as given.
 *   - state row a is a value lane, column c a key lane: s0/s_out are
 *     [B, Hv, Dv, Dk] with u[a] = sum_c S[a][c] k[c].
 *   - key head of value head hv is hv / (Hv / Hk) (contiguous groups).
 *   - l2norm(x) = x / sqrt(sum x^2 + eps); the q scale multiplies q-hat by
 *     1/sqrt(Dk) after normalisation.
 *   - gated norm: x = o * z * sigmoid(z); y[a] = x[a] / sqrt(mean_a x^2 + eps)
 *     * w[a], the mean taken over the Dv lanes of one head; w may be NULL
 *     (unit weight).
 *
 * All arithmetic is float64.  Every array argument is float64, dense,
 * token-major.  Work is split over (batch, value head) pairs, which are
 * independent, with plain pthreads; the per-head arithmetic is sequential and
 * identical for any thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_FOLD_QK_L2NORM 1u
#define ORACLE_FOLD_Q_SCALE 2u

/* L2-normalise x[0..n) in place: x / sqrt(sum x^2 + eps).
 * "gated_delta" page, l2norm (HF's use_qk_l2norm_in_kernel eps). */
void gdn_oracle_l2norm(double* x, int64_t n, double eps) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss + eps);
  for (int64_t i = 0; i < n; ++i) x[i] *= inv;
}

/* Gated RMSNorm of one head, gate first: x = o * silu(z);
 * y = x / sqrt(mean(x^2) + eps) * w.  "Module gdn" page, last equation of the
 * module description.  w == NULL means unit weight. */
void gdn_oracle_gated_rmsnorm(const double* o, const double* z, const double* w, int64_t n,
                              double eps, double* y) {
  double* x = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double silu = z[i] / (1.0 + exp(-z[i]));
    x[i] = o[i] * silu;
    ss += x[i] * x[i];
  }
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) y[i] = x[i] * inv * (w ? w[i] : 1.0);
  free(x);
}

/* Gate producer: log_decay = -decay_scale * softplus(a), beta = sigmoid(b), for
 * n elements.  "Module gdn" page, QWEN38_KERNELS (both gates from one launch);
 * the formulas are the workloads' own recipe, the pages do not give them.
 * softplus(x) = log(1 + exp(x)) and sigmoid(x) = 1 / (1 + exp(-x)), written in
 * forms that do not overflow for large |x|. */
void gdn_oracle_gates(int64_t n, const double* a, const double* b, double decay_scale,
                      double* log_decay, double* beta) {
  for (int64_t i = 0; i < n; ++i) {
    const double x = a[i];
    const double sp = (x > 0 ? x : 0.0) + log1p(exp(-fabs(x)));
    log_decay[i] = -decay_scale * sp;
    const double y = b[i];
    beta[i] = y >= 0 ? 1.0 / (1.0 + exp(-y)) : exp(y) / (1.0 + exp(y));
  }
}

/* Causal depthwise convolution over the time axis, optionally followed by
 * silu: the producer of q, k and v ("Module gdn" page, QWEN38_KERNELS: the
 * convolution carries the silu).  The pages give neither the width nor the
 * weight layout; the reading used here is the usual causal form, one filter of
 * W taps per channel with the last tap on the current token:
 *   pre[b,t,c] = bias[c] + sum_{i<W} w[c][i] * xx(b, t - (W-1) + i, c)
 *   xx(b,t',c) = x[b][t'][c] for t' >= 0, else the carried context
 *                state_in[b][c][(W-1) + t'] (zero when there is none)
 *   y = pre * sigmoid(pre)  (act != 0)  or  y = pre
 *   state_out[b][c][j] = xx(b, T - (W-1) + j, c)  for j < W-1
 * x, y: [B][T][C]; w: [C][W]; bias: [C] or NULL; state_in, state_out:
 * [B][C][W-1] or NULL. */
void gdn_oracle_conv(int64_t B, int64_t T, int64_t C, int64_t W, int act, const double* x,
                     const double* w, const double* bias, const double* state_in, double* y,
                     double* state_out) {
  const int64_t K = W - 1; /* carried context per channel */
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t c = 0; c < C; ++c) {
      for (int64_t t = -K; t < T; ++t) {
        /* xx at time t, for the state output */
        if (state_out && t >= T - K) {
          double v = 0.0;
          if (t >= 0) v = x[(b * T + t) * C + c];
          else if (state_in) v = state_in[(b * C + c) * K + (K + t)];
          state_out[(b * C + c) * K + (t - (T - K))] = v;
        }
        if (t < 0) continue;
        double pre = bias ? bias[c] : 0.0;
        for (int64_t i = 0; i < W; ++i) {
          const int64_t tt = t - K + i;
          double v = 0.0;
          if (tt >= 0) v = x[(b * T + tt) * C + c];
          else if (state_in) v = state_in[(b * C + c) * K + (K + tt)];
          pre += w[c * W + i] * v;
        }
        y[(b * T + t) * C + c] = act ? pre / (1.0 + exp(-pre)) : pre;
      }
    }
  }
}

typedef struct {
  int64_t B, T, Hk, Hv, Dk, Dv;
  uint32_t flags;
  double qk_eps, norm_eps;
  const double *q, *k, *v, *log_decay, *beta, *s0, *z, *w;
  double *y, *s_out;
  int64_t first, last; /* range of (b, hv) pairs for one worker */
} oracle_job;

/* One (batch, value head) pair over the whole time axis. */
static void run_head(const oracle_job* J, int64_t b, int64_t hv) {
  const int64_t Dk = J->Dk, Dv = J->Dv, T = J->T, Hk = J->Hk, Hv = J->Hv;
  const int64_t hk = hv / (Hv / Hk);
  double* S = (double*)malloc(sizeof(double) * (size_t)(Dv * Dk > 0 ? Dv * Dk : 1));
  double* qv = (double*)malloc(sizeof(double) * (size_t)(Dk > 0 ? Dk : 1));
  double* kv = (double*)malloc(sizeof(double) * (size_t)(Dk > 0 ? Dk : 1));
  double* u = (double*)malloc(sizeof(double) * (size_t)(Dv > 0 ? Dv : 1));
  double* o = (double*)malloc(sizeof(double) * (size_t)(Dv > 0 ? Dv : 1));

  memcpy(S, J->s0 + (b * Hv + hv) * Dv * Dk, sizeof(double) * (size_t)(Dv * Dk));
  for (int64_t t = 0; t < T; ++t) {
    const int64_t qk_off = ((b * T + t) * Hk + hk) * Dk;
    const int64_t v_off = ((b * T + t) * Hv + hv) * Dv;
    const int64_t g_off = (b * T + t) * Hv + hv;
    memcpy(qv, J->q + qk_off, sizeof(double) * (size_t)Dk);
    memcpy(kv, J->k + qk_off, sizeof(double) * (size_t)Dk);
    if (J->flags & ORACLE_FOLD_QK_L2NORM) {
      gdn_oracle_l2norm(qv, Dk, J->qk_eps);
      gdn_oracle_l2norm(kv, Dk, J->qk_eps);
    }
    if (J->flags & ORACLE_FOLD_Q_SCALE) {
      const double sc = 1.0 / sqrt((double)Dk);
      for (int64_t c = 0; c < Dk; ++c) qv[c] *= sc;
    }
    const double alpha = exp(J->log_decay[g_off]);
    const double beta = J->beta[g_off];
    const double* vt = J->v + v_off;

    /* pass 1: u = S.k -- what the memory predicts for this key */
    for (int64_t a = 0; a < Dv; ++a) {
      double acc = 0.0;
      for (int64_t c = 0; c < Dk; ++c) acc += S[a * Dk + c] * kv[c];
      u[a] = acc;
    }
    /* pass 2: S = alpha*S + beta*(v - alpha*u) k^T -- decay, then correct */
    for (int64_t a = 0; a < Dv; ++a) {
      const double corr = beta * (vt[a] - alpha * u[a]);
      for (int64_t c = 0; c < Dk; ++c) S[a * Dk + c] = alpha * S[a * Dk + c] + corr * kv[c];
    }
    /* pass 3: o = S.q on the state this token just produced */
    for (int64_t a = 0; a < Dv; ++a) {
      double acc = 0.0;
      for (int64_t c = 0; c < Dk; ++c) acc += S[a * Dk + c] * qv[c];
      o[a] = acc;
    }
    double* yt = J->y + v_off;
    if (J->z) {
      gdn_oracle_gated_rmsnorm(o, J->z + v_off, J->w, Dv, J->norm_eps, yt);
    } else {
      memcpy(yt, o, sizeof(double) * (size_t)Dv);
    }
  }
  memcpy(J->s_out + (b * Hv + hv) * Dv * Dk, S, sizeof(double) * (size_t)(Dv * Dk));
  free(S);
  free(qv);
  free(kv);
  free(u);
  free(o);
}

static void* worker(void* arg) {
  const oracle_job* J = (const oracle_job*)arg;
  for (int64_t p = J->first; p < J->last; ++p) run_head(J, p / J->Hv, p % J->Hv);
  return NULL;
}

/* The whole recurrence over the time axis for every (batch, value head).
 * Arrays: q, k [B,T,Hk,Dk]; v, z, y [B,T,Hv,Dv]; log_decay, beta [B,T,Hv];
 * s0, s_out [B,Hv,Dv,Dk]; w [Dv].  z and w may be NULL (then y = o).
 * Returns 0, or -1 on an invalid shape. */
int gdn_oracle_scan(int64_t B, int64_t T, int64_t Hk, int64_t Hv, int64_t Dk, int64_t Dv,
                    uint32_t flags, double qk_eps, double norm_eps, const double* q,
                    const double* k, const double* v, const double* log_decay,
                    const double* beta, const double* s0, const double* z, const double* w,
                    double* y, double* s_out, int nthreads) {
  if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0 || Hv % Hk) return -1;
  const int64_t pairs = B * Hv;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > pairs) nthreads = (int)(pairs > 0 ? pairs : 1);
  oracle_job base = {B, T, Hk, Hv, Dk, Dv, flags, qk_eps, norm_eps, q, k, v, log_decay,
                     beta, s0, z, w, y, s_out, 0, 0};
  oracle_job* jobs = (oracle_job*)malloc(sizeof(oracle_job) * (size_t)nthreads);
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = base;
    jobs[i].first = pairs * i / nthreads;
    jobs[i].last = pairs * (i + 1) / nthreads;
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&tid[i], NULL, worker, &jobs[i]);
  worker(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(tid[i], NULL);
  free(jobs);
  free(tid);
  return 0;
}

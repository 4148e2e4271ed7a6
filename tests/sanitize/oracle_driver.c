/*
 * Runs the float64 oracle's entry points on operands read from a file, so that
 * a build of oracle/gdn_oracle.c with AddressSanitizer and
 * UndefinedBehaviorSanitizer can be exercised from a test (the test compares
 * the outputs with the ordinary build's).  Test infrastructure only.
 *
 *   oracle_driver scan  B T Hk Hv Dk Dv flags gated threads  in out
 *   oracle_driver gates n decay_scale                          in out
 *   oracle_driver conv  B T C W act has_bias has_state        in out
 *   oracle_driver norms rows n                                 in out
 *
 * `in` holds the float64 operands back to back in the order of the entry
 * point's arguments; `out` receives its float64 outputs the same way.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn_oracle_scan(int64_t B, int64_t T, int64_t Hk, int64_t Hv, int64_t Dk, int64_t Dv,
                    uint32_t flags, double qk_eps, double norm_eps, const double* q,
                    const double* k, const double* v, const double* log_decay,
                    const double* beta, const double* s0, const double* z, const double* w,
                    double* y, double* s_out, int nthreads);
void gdn_oracle_gates(int64_t n, const double* a, const double* b, double decay_scale,
                      double* log_decay, double* beta);
void gdn_oracle_conv(int64_t B, int64_t T, int64_t C, int64_t W, int act, const double* x,
                     const double* w, const double* bias, const double* state_in, double* y,
                     double* state_out);
void gdn_oracle_l2norm(double* x, int64_t n, double eps);
void gdn_oracle_gated_rmsnorm(const double* o, const double* z, const double* w, int64_t n,
                              double eps, double* y);

static FILE* fin;
static FILE* fout;

/* exactly n doubles from the input (NULL for n == 0: an absent operand) */
static double* take(int64_t n) {
  if (n <= 0) return NULL;
  double* p = (double*)malloc(sizeof(double) * (size_t)n);
  if (!p || fread(p, sizeof(double), (size_t)n, fin) != (size_t)n) {
    fprintf(stderr, "short input\n");
    exit(2);
  }
  return p;
}

static double* room(int64_t n) { return (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1)); }

static void put(const double* p, int64_t n) {
  if (n > 0 && fwrite(p, sizeof(double), (size_t)n, fout) != (size_t)n) exit(3);
}

static int64_t arg(char** argv, int i) { return strtoll(argv[i], NULL, 10); }

int main(int argc, char** argv) {
  if (argc < 4) return 1;
  const char* mode = argv[1];
  fin = fopen(argv[argc - 2], "rb");
  fout = fopen(argv[argc - 1], "wb");
  if (!fin || !fout) return 1;
  if (!strcmp(mode, "scan") && argc == 13) {
    const int64_t B = arg(argv, 2), T = arg(argv, 3), Hk = arg(argv, 4), Hv = arg(argv, 5);
    const int64_t Dk = arg(argv, 6), Dv = arg(argv, 7), gated = arg(argv, 9);
    const uint32_t flags = (uint32_t)arg(argv, 8);
    const int threads = (int)arg(argv, 10);
    double* q = take(B * T * Hk * Dk);
    double* k = take(B * T * Hk * Dk);
    double* v = take(B * T * Hv * Dv);
    double* g = take(B * T * Hv);
    double* be = take(B * T * Hv);
    double* s0 = take(B * Hv * Dv * Dk);
    double* z = gated ? take(B * T * Hv * Dv) : NULL;
    double* w = gated ? take(Dv) : NULL;
    double* y = room(B * T * Hv * Dv);
    double* s = room(B * Hv * Dv * Dk);
    if (gdn_oracle_scan(B, T, Hk, Hv, Dk, Dv, flags, 1e-6, 1e-6, q, k, v, g, be, s0, z, w, y, s,
                        threads) != 0)
      return 4;
    put(y, B * T * Hv * Dv);
    put(s, B * Hv * Dv * Dk);
    free(q), free(k), free(v), free(g), free(be), free(s0), free(z), free(w), free(y), free(s);
  } else if (!strcmp(mode, "gates") && argc == 6) {
    const int64_t n = arg(argv, 2);
    const double scale = strtod(argv[3], NULL);
    double* a = take(n);
    double* b = take(n);
    double* ld = room(n);
    double* bt = room(n);
    gdn_oracle_gates(n, a, b, scale, ld, bt);
    put(ld, n);
    put(bt, n);
    free(a), free(b), free(ld), free(bt);
  } else if (!strcmp(mode, "conv") && argc == 11) {
    const int64_t B = arg(argv, 2), T = arg(argv, 3), C = arg(argv, 4), W = arg(argv, 5);
    const int act = (int)arg(argv, 6), has_bias = (int)arg(argv, 7), has_state = (int)arg(argv, 8);
    double* x = take(B * T * C);
    double* w = take(C * W);
    double* bias = has_bias ? take(C) : NULL;
    double* st = has_state ? take(B * C * (W - 1)) : NULL;
    double* y = room(B * T * C);
    double* so = room(B * C * (W - 1));
    gdn_oracle_conv(B, T, C, W, act, x, w, bias, st, y, so);
    put(y, B * T * C);
    put(so, B * C * (W - 1));
    free(x), free(w), free(bias), free(st), free(y), free(so);
  } else if (!strcmp(mode, "norms") && argc == 6) {
    const int64_t rows = arg(argv, 2), n = arg(argv, 3);
    double* x = take(rows * n);
    double* z = take(rows * n);
    double* w = take(n);
    double* y = room(rows * n);
    for (int64_t r = 0; r < rows; ++r) {
      gdn_oracle_gated_rmsnorm(x + r * n, z + r * n, (r & 1) ? w : NULL, n, 1e-6, y + r * n);
      gdn_oracle_l2norm(x + r * n, n, 1e-6);
    }
    put(x, rows * n);
    put(y, rows * n);
    free(x), free(z), free(w), free(y);
  } else {
    fprintf(stderr, "bad arguments\n");
    return 1;
  }
  fclose(fin);
  fclose(fout);
  return 0;
}

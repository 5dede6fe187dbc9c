/* Host-only AddressSanitizer and UndefinedBehaviorSanitizer run of the oracle's C entry
 * points: the forward, the decode step, the gradients and the diagonal-plus-low-rank
 * forward, for every gate and write rule, on small packed inputs with an empty and a
 * ragged sequence.  Exits 0 when every call returns 0 and every output is finite; the
 * sanitizers abort on any out-of-bounds access, leak or undefined operation. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_fwd(int N, const int64_t *start, const int64_t *len, int H, int dk, int dv, int gate, int write,
               const double *q, const double *k, const double *v, const double *beta, const double *log_alpha,
               const double *initial_state, double *o, double *final_state, int nthreads);
int oracle_step(int N, int H, int dk, int dv, int gate, int write, const double *q, const double *k,
                const double *v, const double *beta, const double *log_alpha, double *state, double *o);
int oracle_bwd(int N, const int64_t *start, const int64_t *len, int H, int dk, int dv, int gate, int write,
               const double *q, const double *k, const double *v, const double *beta, const double *log_alpha,
               const double *initial_state, const double *dout, const double *dfinal, double *dq, double *dk_out,
               double *dv_out, double *dbeta, double *dlog_alpha, double *dinit, int nthreads);
int oracle_fwd_dplr(int N, const int64_t *start, const int64_t *len, int H, int dk, int dv, int gate,
                    const double *q, const double *k, const double *v, const double *a, const double *b,
                    const double *log_alpha, const double *initial_state, double *o, double *final_state,
                    int nthreads);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *filled(size_t n, double lo, double hi) {
  double *x = malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * 0.5 * (urand() + 1.0);
  return x;
}
static double *zeros(size_t n) { return calloc(n, sizeof(double)); }
static int all_finite(const double *x, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

int main(void) {
  enum { N = 3, H = 2, DK = 4, DV = 3 };
  const int64_t start[N] = {0, 5, 5}, len[N] = {5, 0, 70};
  const size_t T = 75, th = T * H, st = (size_t)N * H * DK * DV;
  int bad = 0;
  double *q = filled(th * DK, -0.5, 0.5), *k = filled(th * DK, -0.5, 0.5), *v = filled(th * DV, -1, 1);
  double *a = filled(th * DK, -0.5, 0.5), *b = filled(th * DK, -0.5, 0.5);
  double *beta = filled(th, 0.0, 1.0), *la_h = filled(th, -0.5, 0.0), *la_k = filled(th * DK, -0.5, 0.0);
  double *s0 = filled(st, -0.1, 0.1), *dout = filled(th * DV, -1, 1), *dfin = filled(st, -0.1, 0.1);
  for (int gate = 0; gate < 3; ++gate) {
    const double *la = gate == 0 ? NULL : gate == 1 ? la_h : la_k;
    const size_t nla = gate == 0 ? 0 : gate == 1 ? th : th * DK;
    for (int write = 0; write < 2; ++write) {
      const double *bt = write == 0 ? beta : NULL;
      double *o = zeros(th * DV), *fs = zeros(st);
      if (oracle_fwd(N, start, len, H, DK, DV, gate, write, q, k, v, bt, la, s0, o, fs, 2) != 0 ||
          !all_finite(o, th * DV) || !all_finite(fs, st)) {
        fprintf(stderr, "forward gate %d write %d\n", gate, write);
        bad = 1;
      }
      double *dq = zeros(th * DK), *dk = zeros(th * DK), *dv = zeros(th * DV), *db = write == 0 ? zeros(th) : NULL;
      double *dla = nla ? zeros(nla) : NULL, *di = zeros(st);
      if (oracle_bwd(N, start, len, H, DK, DV, gate, write, q, k, v, bt, la, s0, dout, dfin, dq, dk, dv, db, dla, di,
                     2) != 0 ||
          !all_finite(dq, th * DK) || !all_finite(dk, th * DK) || !all_finite(dv, th * DV) || !all_finite(di, st) ||
          (db && !all_finite(db, th)) || (dla && !all_finite(dla, nla))) {
        fprintf(stderr, "gradients gate %d write %d\n", gate, write);
        bad = 1;
      }
      double *state = filled((size_t)4 * H * DK * DV, -0.1, 0.1), *os = zeros((size_t)4 * H * DV);
      if (oracle_step(4, H, DK, DV, gate, write, q, k, v, bt, la, state, os) != 0 ||
          !all_finite(os, (size_t)4 * H * DV) || !all_finite(state, (size_t)4 * H * DK * DV)) {
        fprintf(stderr, "step gate %d write %d\n", gate, write);
        bad = 1;
      }
      free(o), free(fs), free(dq), free(dk), free(dv), free(db), free(dla), free(di), free(state), free(os);
    }
    double *o = zeros(th * DV), *fs = zeros(st);
    if (oracle_fwd_dplr(N, start, len, H, DK, DV, gate, q, k, v, a, b, la, s0, o, fs, 2) != 0 ||
        !all_finite(o, th * DV) || !all_finite(fs, st)) {
      fprintf(stderr, "dplr gate %d\n", gate);
      bad = 1;
    }
    free(o), free(fs);
  }
  free(q), free(k), free(v), free(a), free(b), free(beta), free(la_h), free(la_k), free(s0), free(dout), free(dfin);
  if (!bad) printf("oracle sanitizer run: clean\n");
  return bad;
}

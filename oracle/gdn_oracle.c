/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the (gated) delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no code,
 * header, table or helper with the GPU library and must never be used as a
 * fallback for it.
 *
 * What it computes (one sequence, one head, token by token, in fp64):
 *
 *   The state is kept as M = S^T, a d_k x d_v matrix: M[i][j] maps key channel i
 *   to value channel j ("Decoding Hybrid Linear Attention Architectures", sec. 1,
 *   state of size d_k x d_v).  For each token t with key k, value v, query q,
 *   write strength beta and decay a = exp(log_alpha):
 *
 *     1. decay:    M[i][:] *= a_i   (a_i = 1 without a gate, one scalar per head
 *                                    for the gated rule, one value per key channel
 *                                    for the channel-wise rule)
 *     2. retrieve: r = M^T k        (what key k currently maps to)
 *     3. write:    M += beta * k (v - r)^T
 *     4. read:     o = M^T q        (the read uses the state after the write)
 *
 *   With the additive write (write = ORACLE_WRITE_ADD) steps 2-3 are replaced by
 *
 *     2'. write:   M += k v^T       (no erase, no beta)
 *
 *   which is the gated-linear-attention update of the same sec. 3, item 4
 *   (channel-wise forgetting without overwriting), RetNet's retention with a fixed
 *   per-head decay ("Linear Attention Variants", RetNet section) and, without a
 *   gate, the plain linear-transformer sum of that page's "The Shared Machinery".
 *
 *   Steps 1-3 are the single-step update of "Decoding Hybrid Linear Attention
 *   Architectures", sec. 3 item 6 (decay, directional erase, overwriting write),
 *   which for a scalar gate is item 3 (gated delta rule) and without a gate is
 *   item 2 (delta rule).  Step 2-3 is the retrieve / subtract / write reading of
 *   the DeltaNet update on "Linear Attention Variants (RetNet, GLA, DeltaNet,
 *   Based)", section "DeltaNet: Error-Correcting Writes".  Step 4 is the read
 *   y_t = q_t^T S_t of the same page's "The Shared Machinery" section (no feature
 *   map and no normalizer for the delta rule).
 *
 * Layout: tokens of all sequences are packed; sequence n covers packed tokens
 * [start[n], start[n] + len[n]).  q,k: [tokens][H][d_k], v,o: [tokens][H][d_v],
 * beta: [tokens][H] (NULL with the additive write), log_alpha: NULL | [tokens][H] |
 * [tokens][H][d_k],
 * states: [N][H][d_k][d_v].  All arrays are fp64 and contiguous.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_GATE_NONE = 0, ORACLE_GATE_HEAD = 1, ORACLE_GATE_KEY = 2 };
enum { ORACLE_WRITE_DELTA = 0, ORACLE_WRITE_ADD = 1 };

/* One token of the recurrence on one head's state M (d_k x d_v, row-major). */
static void oracle_token(int dk, int dv, int gate, int write, const double *q, const double *k,
                         const double *v, double beta, const double *log_alpha,
                         double *M, double *r, double *o) {
  int i, j;
  /* 1. decay (key rows) */
  if (gate == ORACLE_GATE_HEAD) {
    double a = exp(log_alpha[0]);
    for (i = 0; i < dk * dv; ++i) M[i] *= a;
  } else if (gate == ORACLE_GATE_KEY) {
    for (i = 0; i < dk; ++i) {
      double a = exp(log_alpha[i]);
      for (j = 0; j < dv; ++j) M[i * dv + j] *= a;
    }
  }
  if (write == ORACLE_WRITE_ADD) {
    /* 2'. additive write M += k v^T */
    for (i = 0; i < dk; ++i)
      for (j = 0; j < dv; ++j) M[i * dv + j] += k[i] * v[j];
  } else {
  /* 2. retrieve r = M^T k */
  for (j = 0; j < dv; ++j) r[j] = 0.0;
  for (i = 0; i < dk; ++i)
    for (j = 0; j < dv; ++j) r[j] += M[i * dv + j] * k[i];
  /* 3. write M += beta k (v - r)^T */
  for (i = 0; i < dk; ++i) {
    double bk = beta * k[i];
    for (j = 0; j < dv; ++j) M[i * dv + j] += bk * (v[j] - r[j]);
  }
  }
  /* 4. read o = M^T q */
  for (j = 0; j < dv; ++j) o[j] = 0.0;
  for (i = 0; i < dk; ++i)
    for (j = 0; j < dv; ++j) o[j] += M[i * dv + j] * q[i];
}

/* Whole sequences.  Returns 0, or -1 on a bad argument / allocation failure. */
int oracle_fwd(int N, const int64_t *start, const int64_t *len, int H, int dk, int dv,
               int gate, int write, const double *q, const double *k, const double *v,
               const double *beta, const double *log_alpha, const double *initial_state,
               double *o, double *final_state, int nthreads) {
  int64_t pair;
  int failed = 0;
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (gate != ORACLE_GATE_NONE && log_alpha == NULL) return -1;
  if (write != ORACLE_WRITE_ADD && beta == NULL) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
  for (pair = 0; pair < (int64_t)N * H; ++pair) {
    int n = (int)(pair / H), h = (int)(pair % H);
    double *M = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *r = (double *)malloc(sizeof(double) * (size_t)dv);
    int64_t t;
    if (!M || !r) { free(M); free(r); failed = 1; continue; }
    if (initial_state)
      memcpy(M, initial_state + ((size_t)n * H + h) * dk * dv, sizeof(double) * dk * dv);
    else
      memset(M, 0, sizeof(double) * dk * dv);
    for (t = start[n]; t < start[n] + len[n]; ++t) {
      size_t th = (size_t)t * H + h;
      const double *la = NULL;
      if (gate == ORACLE_GATE_HEAD) la = log_alpha + th;
      if (gate == ORACLE_GATE_KEY) la = log_alpha + th * dk;
      oracle_token(dk, dv, gate, write, q + th * dk, k + th * dk, v + th * dv, beta ? beta[th] : 0.0,
                   la, M, r, o + th * dv);
    }
    if (final_state) memcpy(final_state + ((size_t)n * H + h) * dk * dv, M, sizeof(double) * dk * dv);
    free(M);
    free(r);
  }
  return failed ? -1 : 0;
}

/* One token per stream, state updated in place: q,k [N][H][d_k], v,o [N][H][d_v],
 * beta [N][H], log_alpha NULL | [N][H] | [N][H][d_k], state [N][H][d_k][d_v]. */
int oracle_step(int N, int H, int dk, int dv, int gate, int write, const double *q, const double *k,
                const double *v, const double *beta, const double *log_alpha, double *state,
                double *o) {
  int64_t pair;
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (gate != ORACLE_GATE_NONE && log_alpha == NULL) return -1;
  if (write != ORACLE_WRITE_ADD && beta == NULL) return -1;
  for (pair = 0; pair < (int64_t)N * H; ++pair) {
    double *r = (double *)malloc(sizeof(double) * (size_t)dv);
    const double *la = NULL;
    if (!r) return -1;
    if (gate == ORACLE_GATE_HEAD) la = log_alpha + pair;
    if (gate == ORACLE_GATE_KEY) la = log_alpha + pair * dk;
    oracle_token(dk, dv, gate, write, q + pair * dk, k + pair * dk, v + pair * dv,
                 beta ? beta[pair] : 0.0, la, state + pair * dk * dv, r, o + pair * dv);
    free(r);
  }
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

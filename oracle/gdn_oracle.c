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

/*
 * Gradients of the token recurrence above (reverse mode, fp64), for the delta write and
 * the additive write with no gate, one decay per (token, head) or one decay per (token,
 * head, key channel).  For one token of the delta write, with M' = a M_{t-1} (row i
 * scaled by a_i for the per-channel gate),
 * r = M'^T k, e = v - r, M_t = M' + beta k e^T, o = M_t^T q, and the gradient G of
 * the loss with respect to M_t (everything that later tokens and the final state
 * pass back) plus do:
 *   G    += q do^T                    dq = M_t do
 *   dbeta = k^T G e                   de = beta G^T k
 *   dk    = beta G e - M' de          (from the write, and from r = M'^T k, dr = -de)
 *   dv    = de
 *   G'    = G - k de^T                (gradient with respect to M')
 *   dlog_alpha = sum(G' .* M')        (M' = a M_{t-1}, d a / d log a = a)
 *   G_{t-1} = a G'
 * With one decay per key channel the last two lines hold row by row: dlog_alpha_i =
 * sum_j G'[i][j] M'[i][j] and row i of G_{t-1} is a_i times row i of G'.
 * The additive write M_t = M' + k v^T passes G to M' unchanged, with dk = G v and
 * dv = G^T k (no beta: dbeta may be NULL).
 * Each sequence's states M_t are recomputed forward and kept, then swept in reverse.
 * dfinal (NULL: zeros) is the gradient with respect to the final state; the result
 * dinit is the gradient with respect to the initial state.  Arrays as for
 * oracle_fwd; dlog_alpha is [tokens][H], [tokens][H][d_k] for the per-channel gate, or
 * NULL without a gate.
 */
int oracle_bwd(int N, const int64_t *start, const int64_t *len, int H, int dk, int dv, int gate,
               int write, const double *q, const double *k, const double *v, const double *beta,
               const double *log_alpha, const double *initial_state, const double *dout,
               const double *dfinal, double *dq, double *dk_out, double *dv_out, double *dbeta,
               double *dlog_alpha, double *dinit, int nthreads) {
  int64_t pair;
  int failed = 0;
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (write != ORACLE_WRITE_DELTA && write != ORACLE_WRITE_ADD) return -1;
  if (write == ORACLE_WRITE_DELTA && (beta == NULL || dbeta == NULL)) return -1;
  if (gate != ORACLE_GATE_NONE && gate != ORACLE_GATE_HEAD && gate != ORACLE_GATE_KEY) return -1;
  if (gate != ORACLE_GATE_NONE && (log_alpha == NULL || dlog_alpha == NULL)) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
  for (pair = 0; pair < (int64_t)N * H; ++pair) {
    int n = (int)(pair / H), h = (int)(pair % H);
    const int64_t L = len[n], S = (int64_t)dk * dv;
    double *Ms = (double *)malloc(sizeof(double) * (size_t)S * (size_t)(L + 1)); /* M_0 .. M_L */
    double *G = (double *)malloc(sizeof(double) * (size_t)S);
    double *Mp = (double *)malloc(sizeof(double) * (size_t)S);
    double *r = (double *)malloc(sizeof(double) * (size_t)dv);
    double *e = (double *)malloc(sizeof(double) * (size_t)dv);
    double *de = (double *)malloc(sizeof(double) * (size_t)dv);
    double *otmp = (double *)malloc(sizeof(double) * (size_t)dv);
    double *arow = (double *)malloc(sizeof(double) * (size_t)dk); /* decay of each key row */
    int64_t t;
    int i, j;
    if (!Ms || !G || !Mp || !r || !e || !de || !otmp || !arow) {
      free(Ms); free(G); free(Mp); free(r); free(e); free(de); free(otmp); free(arow);
      failed = 1;
      continue;
    }
    if (initial_state)
      memcpy(Ms, initial_state + ((size_t)n * H + h) * S, sizeof(double) * S);
    else
      memset(Ms, 0, sizeof(double) * S);
    /* forward: keep every state */
    for (t = 0; t < L; ++t) {
      size_t th = (size_t)(start[n] + t) * H + h;
      memcpy(Ms + (t + 1) * S, Ms + t * S, sizeof(double) * S);
      oracle_token(dk, dv, gate, write, q + th * dk, k + th * dk, v + th * dv, beta ? beta[th] : 0.0,
                   gate == ORACLE_GATE_HEAD ? log_alpha + th : gate == ORACLE_GATE_KEY ? log_alpha + th * dk : NULL,
                   Ms + (t + 1) * S, r, otmp);
    }
    /* reverse sweep */
    if (dfinal)
      memcpy(G, dfinal + ((size_t)n * H + h) * S, sizeof(double) * S);
    else
      memset(G, 0, sizeof(double) * S);
    for (t = L - 1; t >= 0; --t) {
      size_t th = (size_t)(start[n] + t) * H + h;
      const double *qt = q + th * dk, *kt = k + th * dk, *vt = v + th * dv, *dot = dout + th * dv;
      const double *Mt = Ms + (t + 1) * S, *Mprev = Ms + t * S;
      const double bt = beta ? beta[th] : 0.0;
      double db = 0.0, dla = 0.0;
      for (i = 0; i < dk; ++i)
        arow[i] = gate == ORACLE_GATE_HEAD ? exp(log_alpha[th]) : gate == ORACLE_GATE_KEY ? exp(log_alpha[th * dk + i]) : 1.0;
      for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) Mp[i * dv + j] = arow[i] * Mprev[i * dv + j];
      for (j = 0; j < dv; ++j) r[j] = 0.0;
      for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) r[j] += Mp[i * dv + j] * kt[i];
      for (j = 0; j < dv; ++j) e[j] = vt[j] - r[j];
      /* read */
      for (i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (j = 0; j < dv; ++j) {
          G[i * dv + j] += qt[i] * dot[j];
          acc += Mt[i * dv + j] * dot[j];
        }
        dq[th * dk + i] = acc;
      }
      if (write == ORACLE_WRITE_ADD) {
        /* additive write: dk = G v, dv = G^T k; G passes to M' unchanged */
        for (i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (j = 0; j < dv; ++j) acc += G[i * dv + j] * vt[j];
          dk_out[th * dk + i] = acc;
        }
        for (j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (i = 0; i < dk; ++i) acc += G[i * dv + j] * kt[i];
          dv_out[th * dv + j] = acc;
        }
        for (i = 0; i < dk; ++i) {
          double dli = 0.0;
          for (j = 0; j < dv; ++j) {
            dli += G[i * dv + j] * Mp[i * dv + j];
            G[i * dv + j] *= arow[i];
          }
          if (gate == ORACLE_GATE_KEY) dlog_alpha[th * dk + i] = dli;
          dla += dli;
        }
        if (gate == ORACLE_GATE_HEAD) dlog_alpha[th] = dla;
        continue;
      }
      /* write: de = beta G^T k, dbeta = k^T G e */
      for (j = 0; j < dv; ++j) de[j] = 0.0;
      for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) {
          de[j] += G[i * dv + j] * kt[i];
          db += kt[i] * G[i * dv + j] * e[j];
        }
      for (j = 0; j < dv; ++j) de[j] *= bt;
      for (i = 0; i < dk; ++i) {
        double acc = 0.0, acc2 = 0.0;
        for (j = 0; j < dv; ++j) {
          acc += G[i * dv + j] * e[j];
          acc2 += Mp[i * dv + j] * de[j];
        }
        dk_out[th * dk + i] = bt * acc - acc2;
      }
      for (j = 0; j < dv; ++j) dv_out[th * dv + j] = de[j];
      dbeta[th] = db;
      /* gradient with respect to M', then M_{t-1} */
      for (i = 0; i < dk; ++i) {
        double dli = 0.0;
        for (j = 0; j < dv; ++j) {
          G[i * dv + j] -= kt[i] * de[j];
          dli += G[i * dv + j] * Mp[i * dv + j];
          G[i * dv + j] *= arow[i];
        }
        if (gate == ORACLE_GATE_KEY) dlog_alpha[th * dk + i] = dli;
        dla += dli;
      }
      if (gate == ORACLE_GATE_HEAD) dlog_alpha[th] = dla;
    }
    if (dinit) memcpy(dinit + ((size_t)n * H + h) * S, G, sizeof(double) * S);
    free(Ms); free(G); free(Mp); free(r); free(e); free(de); free(otmp); free(arow);
  }
  return failed ? -1 : 0;
}

/*
 * The diagonal-plus-low-rank transition ("Decoding Hybrid Linear Attention
 * Architectures", sec. 3 item 5): S_t = S_{t-1} (Diag(alpha_t) + a_t b_t^T) + v_t k_t^T,
 * so in storage orientation (M = S^T) one token is
 *   u = a^T M_{t-1}                 (a row of d_v values, read before anything changes)
 *   M_t = Diag(alpha) M_{t-1} + b u + k v^T
 *   o = M_t^T q                     (the read follows the write)
 * alpha = exp(log_alpha): none (1), one per (token, head), or one per key channel.
 * Arrays as for oracle_fwd, with a, b: [tokens][H][d_k].
 */
int oracle_fwd_dplr(int N, const int64_t *start, const int64_t *len, int H, int dk, int dv, int gate,
                    const double *q, const double *k, const double *v, const double *a, const double *b,
                    const double *log_alpha, const double *initial_state, double *o, double *final_state,
                    int nthreads) {
  int64_t pair;
  int failed = 0;
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (gate != ORACLE_GATE_NONE && log_alpha == NULL) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
  for (pair = 0; pair < (int64_t)N * H; ++pair) {
    int n = (int)(pair / H), h = (int)(pair % H), i, j;
    double *M = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    int64_t t;
    if (!M || !u) { free(M); free(u); failed = 1; continue; }
    if (initial_state)
      memcpy(M, initial_state + ((size_t)n * H + h) * dk * dv, sizeof(double) * dk * dv);
    else
      memset(M, 0, sizeof(double) * dk * dv);
    for (t = start[n]; t < start[n] + len[n]; ++t) {
      const size_t th = (size_t)t * H + h;
      const double *qt = q + th * dk, *kt = k + th * dk, *at = a + th * dk, *bt = b + th * dk, *vt = v + th * dv;
      /* u = a^T M_{t-1} */
      for (j = 0; j < dv; ++j) u[j] = 0.0;
      for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) u[j] += at[i] * M[i * dv + j];
      /* M = Diag(alpha) M + b u + k v^T */
      for (i = 0; i < dk; ++i) {
        double al = 1.0;
        if (gate == ORACLE_GATE_HEAD) al = exp(log_alpha[th]);
        if (gate == ORACLE_GATE_KEY) al = exp(log_alpha[th * dk + i]);
        for (j = 0; j < dv; ++j) M[i * dv + j] = al * M[i * dv + j] + bt[i] * u[j] + kt[i] * vt[j];
      }
      /* o = M^T q */
      for (j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (i = 0; i < dk; ++i) acc += M[i * dv + j] * qt[i];
        o[th * dv + j] = acc;
      }
    }
    if (final_state) memcpy(final_state + ((size_t)n * H + h) * dk * dv, M, sizeof(double) * dk * dv);
    free(M);
    free(u);
  }
  return failed ? -1 : 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * gdn.h -- C ABI of the MI355X (gfx950) chunked gated delta rule: the forward, its
 * gradients, decode steps for serving, and the diagonal-plus-low-rank transition.
 *
 * The method: a linear-attention layer keeps one fixed-size matrix state per
 * (sequence, head) ("Decoding Hybrid Linear Attention Architectures", sec. 1: a
 * state of size d_k x d_v, updated and read once per token).  Per token t, with
 * query q_t, key k_t, value v_t, write strength beta_t and decay alpha_t:
 *
 *   S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
 *
 * with S in R^{d_v x d_k}.  alpha_t = 1 is the delta rule (same page, sec. 3 item 2;
 * "Linear Attention Variants (RetNet, GLA, DeltaNet, Based)", DeltaNet section),
 * one scalar per (token, head) is the gated delta rule (sec. 3 item 3) and one
 * value per key channel is the channel-wise gated delta rule (sec. 3 item 6).  The
 * decay acts first, then the erase along k_t, then the write (sec. 3 item 6 and its
 * single-step pseudocode).  The read uses the state after the write.
 *
 * The library computes this with the chunkwise-parallel algorithm of "Decoding
 * Hybrid Linear Attention Architectures", sec. 5 (chunks of C = 64 tokens; within
 * a chunk, matrix products; across chunks, a serial state recursion), with the
 * WY/UT representation of the chunk's erase-and-write products ("Linear Attention
 * Variants", DeltaNet section).  The result equals the token-by-token recurrence up
 * to rounding.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc / torch CUDA memory),
 *    dense, row-major, 16-byte aligned.  The caller owns all memory; the library
 *    allocates and frees nothing and keeps no pointer after returning.
 *  - The state is stored transposed, M = S^T, as [.., d_k, d_v] fp32:
 *    M[i][j] maps key channel i to value channel j.
 *  - beta and log_alpha are fp32 in every mode; alpha = exp(log_alpha).  Gate
 *    products are accumulated in log space (sec. 5 of the first page).
 *  - q, k, v, o share one I/O dtype (fp32 or bf16).  Arithmetic: fp32 state and
 *    accumulation; bf16 mode rounds matrix-core operands to bf16; o is rounded
 *    once (round-to-nearest-even) to the I/O dtype.
 *  - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the default
 *    stream).  Buffers must stay valid until the stream has finished the work.
 *  - Arguments are validated on the host before anything is launched.  A negative
 *    return means nothing was launched and nothing was written.  Launch failures
 *    return GDN_ERR_HIP.  No C++ exception crosses this boundary.
 *  - Results are deterministic: no atomics, fixed reduction order.
 *  - Thread safety: the only mutable global state is the per-device address of the
 *    scratch array of gdn_fwd_chunked_static, looked up once per device under a lock.
 *    Concurrent calls on different streams are independent, except calls of
 *    gdn_fwd_chunked_static that overlap on one GPU: they share that array and race.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad offsets, misalignment */
  GDN_ERR_UNSUPPORTED = -2, /* a shape or mode outside the supported set        */
  GDN_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required       */
  GDN_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed        */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype; /* dtype of q, k, v, o */

typedef enum {
  GDN_GATE_NONE = 0,      /* alpha = 1 (delta rule); log_alpha must be NULL         */
  GDN_GATE_HEAD = 1,      /* one log_alpha per (token, head) (gated delta rule)     */
  GDN_GATE_KEY = 2,       /* one log_alpha per (token, head, key channel)           */
  GDN_GATE_HEAD_CONST = 3 /* one log_alpha per head, the same at every token: [H]
                             (RetNet's fixed per-head decay, "Linear Attention
                             Variants", RetNet section)                            */
} gdn_gate;

/* How a token writes the state (S = M^T, k a key, v a value):
 *   DELTA: erase what k retrieves, then write: S <- S + beta (v - S k) k^T, after the
 *          decay ("Decoding Hybrid Linear Attention Architectures", sec. 3 items 2,
 *          3 and 6: the delta rule and its gated forms);
 *   ADD:   accumulate: S <- S + v k^T after the decay, no erase and no beta (sec. 3
 *          item 4, gated linear attention; with GDN_GATE_HEAD_CONST RetNet's
 *          retention; without a gate the plain linear-transformer sum, "Linear
 *          Attention Variants", "The Shared Machinery").  beta must be NULL.
 * A zero-initialised argument struct selects DELTA. */
typedef enum { GDN_WRITE_DELTA = 0, GDN_WRITE_ADD = 1 } gdn_write;

/*
 * Chunked forward over whole sequences ("Decoding Hybrid Linear Attention
 * Architectures", sec. 5: inter-chunk state recursion and intra-chunk output).
 *
 * Batch mode (cu_seqlens == NULL): N = B sequences of T tokens each.
 * Varlen mode (cu_seqlens != NULL): B must be 1; the T packed tokens hold
 *   N = number of sequences; sequence n is tokens [cu_seqlens[n], cu_seqlens[n+1]).
 *   cu_seqlens is int32 on the device, N+1 non-decreasing entries, cu_seqlens[0]
 *   = 0 and cu_seqlens[N] = T (checked by the kernel: a bad table leaves o and
 *   final_state of the affected sequences unwritten rather than reading out of
 *   bounds).  Empty sequences are allowed (their final state = initial state).
 * A sequence whose length is not a multiple of 64 ends in a partial chunk; the
 * result is the recurrence's, as if padded with beta = 0 and log_alpha = 0.
 */
typedef struct {
  int B, T, H;        /* batch, tokens per batch row (packed total in varlen), heads
                         (H <= 262143: offsets inside one chunk fit 32 bits)         */
  int d_k, d_v;       /* head dims: each 64 or 128, in either dtype                  */
  int chunk;          /* chunk length: must be 64                                    */
  int N;              /* number of sequences: B, or len(cu_seqlens) - 1
                         (N H d_v / 16 and (B T / 64 + N + 1) H at most 2^31 - 1,
                         the launch grids; GDN_ERR_UNSUPPORTED otherwise)           */
  gdn_dtype dtype;    /* dtype of q, k, v, o                                         */
  gdn_gate gate;      /* gate mode                                                   */
  gdn_write write;    /* write rule                                                  */
  const void *q;      /* [B, T, H, d_k]                                              */
  const void *k;      /* [B, T, H, d_k]                                              */
  const void *v;      /* [B, T, H, d_v]                                              */
  const float *beta;  /* DELTA: [B, T, H] fp32; ADD: NULL                            */
  const float *log_alpha;     /* NONE: NULL; HEAD: [B,T,H]; KEY: [B,T,H,d_k];
                                 HEAD_CONST: [H]; fp32                               */
  const float *initial_state; /* NULL (zeros) or [N, H, d_k, d_v] fp32 (M = S^T)     */
  const int32_t *cu_seqlens;  /* NULL or [N + 1] int32 (device)                      */
  void *o;                    /* out: [B, T, H, d_v], dtype                          */
  float *final_state;         /* out: NULL or [N, H, d_k, d_v] fp32; may alias
                                 initial_state (each block is read before written)  */
  void *workspace;            /* device scratch of gdn_fwd_workspace_size() bytes    */
  size_t workspace_bytes;     /* (NULL / 0 allowed when that size is 0)             */
} gdn_fwd_args;

/* One token per stream, state updated in place (the constant-cost decode update of
 * "Decoding Hybrid Linear Attention Architectures", sec. 6; the recurrent mode of
 * "Linear Attention Variants", RetNet section). */
typedef struct {
  int N, H, d_k, d_v; /* streams, heads, head dims (each 64 or 128); N H at most
                         2^31 - 1 (GDN_ERR_UNSUPPORTED otherwise)                  */
  gdn_dtype dtype;    /* dtype of q, k, v, o                                         */
  gdn_gate gate;
  gdn_write write;
  const void *q;          /* [N, H, d_k]                                             */
  const void *k;          /* [N, H, d_k]                                             */
  const void *v;          /* [N, H, d_v]                                             */
  const float *beta;      /* DELTA: [N, H]; ADD: NULL                                */
  const float *log_alpha; /* NONE: NULL; HEAD: [N,H]; KEY: [N,H,d_k]; HEAD_CONST: [H] */
  float *state;           /* in/out: [N, H, d_k, d_v] fp32, read then overwritten   */
  void *o;                /* out: [N, H, d_v], dtype                                 */
} gdn_step_args;

/* Serving decode: L tokens per stream against a pool of states, in one call.  The
 * per-token update is the one of gdn_fwd_recurrent_step (the constant-cost decode
 * update of "Decoding Hybrid Linear Attention Architectures", sec. 6); the pages fix
 * no layout for the states of many streams, so the pool and slot convention here is
 * this library's own.  Each stream's state is read once from its slot, carried
 * through its L tokens on the GPU, and written only where a slot is given:
 *   - plain decoding: dst_slots[n, L-1] = src_slots[n], the other entries -1;
 *   - speculative drafts: one spare slot per draft token; after verification the
 *     slot of the last accepted token is the next call's src slot (no copy).
 * Slots are indices into state_pool.  A stream whose src slot is outside
 * [0, pool_size) is padding: nothing is read or written for it (its o rows are left
 * as they are).  A dst entry outside [0, pool_size) stores nothing.  The dst slots of
 * one call must differ from each other and from the other streams' src slots (a
 * stream's own src slot may be reused); otherwise the pool's contents are undefined.
 * Slots are device data, so out-of-range values cannot be reported: they are
 * skipped as described. */
typedef struct {
  int N, L, H, d_k, d_v;  /* streams, tokens per stream (>= 1), heads, head dims (64/128) */
  gdn_dtype dtype;        /* dtype of q, k, v, o                                      */
  gdn_gate gate;
  gdn_write write;
  const void *q;          /* [N, L, H, d_k]                                           */
  const void *k;          /* [N, L, H, d_k]                                           */
  const void *v;          /* [N, L, H, d_v]                                           */
  const float *beta;      /* DELTA: [N, L, H]; ADD: NULL                              */
  const float *log_alpha; /* NONE: NULL; HEAD: [N,L,H]; KEY: [N,L,H,d_k]; HEAD_CONST: [H] */
  float *state_pool;      /* in/out: [pool_size, H, d_k, d_v] fp32 (M = S^T), device  */
  int pool_size;          /* number of slots (>= 1)                                   */
  const int32_t *src_slots; /* [N] device: slot each stream's state is read from     */
  const int32_t *dst_slots; /* [N, L] device: slot receiving the state after token t */
  void *o;                /* out: [N, L, H, d_v], dtype                               */
} gdn_decode_args;

/* Bytes of device workspace gdn_fwd_chunked needs for these arguments; 0 means none.
 * Returns 0 for arguments that gdn_fwd_chunked would reject.
 *   - with cu_seqlens (N <= 8192): a processing-order table, 4 N bytes rounded up to 256;
 *   - bf16 with d_k = 128, the per-key-channel gate and the delta write: the chunk
 *     operands prepared in
 *     a first, fully parallel pass (K e^G, Q e^G and K e^{g_C - G}: 3 x 256 bytes per
 *     token and head; T diag(beta) and P: 16 KiB, e^{g_C}: 512 bytes per chunk slot and
 *     head, with floor(B T / 64) + N slots), each part rounded up to 256 bytes.
 * The workspace is owned by the caller; its contents need no initialisation and are
 * meaningless after the call. */
size_t gdn_fwd_workspace_size(const gdn_fwd_args *args);

/* Chunked forward: writes o (and final_state when non-NULL). */
int gdn_fwd_chunked(const gdn_fwd_args *args, void *hip_stream);

/* The same forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): it takes no workspace
 * (args->workspace and args->workspace_bytes are ignored) and allocates nothing.  Its
 * scratch memory is one array of GDN_STATIC_SCRATCH_BYTES per GPU, part of the
 * library's device code and held until the process ends.  Calls whose
 * gdn_fwd_workspace_size() exceeds that return GDN_ERR_WORKSPACE and launch nothing
 * (a call that needs no scratch, e.g. batch mode with a scalar gate, always fits).
 * All calls on one GPU share that GPU's array: two such calls that can overlap on one
 * GPU (different streams without ordering between them) race and give undefined
 * results; calls ordered on one stream are safe.  The scratch needs no initialisation.
 * Otherwise identical to gdn_fwd_chunked (same arguments, validation and results). */
#define GDN_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
int gdn_fwd_chunked_static(const gdn_fwd_args *args, void *hip_stream);

/* One decode token per stream: writes o and updates state in place. */
int gdn_fwd_recurrent_step(const gdn_step_args *args, void *hip_stream);

/* Serving decode (see gdn_decode_args): writes o for the active streams and the
 * requested pool slots; allocates nothing. */
int gdn_fwd_decode(const gdn_decode_args *args, void *hip_stream);

/*
 * Gradients of the chunked forward (training): reverse mode through the chunk
 * equations of "Decoding Hybrid Linear Attention Architectures", sec. 5, written out
 * in this library's kernels (the pages give the forward only).  Supported: the delta
 * write and the additive write (GDN_WRITE_ADD: gated linear attention / RetNet), each
 * with every gate (GDN_GATE_NONE, GDN_GATE_HEAD, GDN_GATE_KEY, GDN_GATE_HEAD_CONST);
 * fp32 I/O with d_k = 128 only with the per-key-channel gate (GDN_ERR_UNSUPPORTED
 * otherwise).  Inputs as for gdn_fwd_chunked (the same validation rules, which
 * this call repeats), plus the gradients of its outputs;
 * the forward is recomputed inside the call (chunk-entering states into the
 * workspace), so nothing of the forward call needs to be kept.  All arithmetic is
 * fp32; dq, dk, dv are rounded once to dtype.  Deterministic (no atomics).
 */
typedef struct {
  int B, T, H, d_k, d_v, chunk, N; /* as in gdn_fwd_args                          */
  gdn_dtype dtype;
  gdn_gate gate;
  gdn_write write;
  const void *q, *k, *v;           /* as in gdn_fwd_args                          */
  const float *beta;               /* DELTA: [B, T, H]; ADD: NULL                 */
  const float *log_alpha;          /* NONE: NULL; HEAD: [B, T, H]; KEY: [B, T, H, d_k];
                                      HEAD_CONST: [H]                             */
  const float *initial_state;      /* NULL (zeros) or [N, H, d_k, d_v]            */
  const int32_t *cu_seqlens;       /* NULL or [N + 1] int32 (device)              */
  const void *dout;                /* [B, T, H, d_v], dtype: gradient of o        */
  const float *dfinal_state;       /* NULL (zeros) or [N, H, d_k, d_v]: gradient of
                                      the final state                             */
  void *dq, *dk, *dv;              /* out: [B, T, H, d_k] / [B, T, H, d_v], dtype */
  float *dbeta;                    /* out: DELTA: [B, T, H]; ADD: NULL            */
  float *dlog_alpha;               /* out: HEAD: [B, T, H]; KEY: [B, T, H, d_k];
                                      HEAD_CONST: [H] (the
                                      sum over all tokens, written also when there
                                      are none); NONE: NULL                       */
  float *dinitial_state;           /* out: NULL or [N, H, d_k, d_v]               */
  void *workspace;                 /* gdn_bwd_workspace_size() bytes, 256-aligned */
  size_t workspace_bytes;
} gdn_bwd_args;

/* Bytes of device workspace gdn_bwd_chunked needs (0 for arguments it would reject),
 * with S = floor(B T / 64) + N chunk slots, each part rounded up to 256 bytes:
 *  - every gate, per slot and head in fp32: the chunk-entering states and chunk-end
 *    state gradients (d_k d_v each), dDelta (64 d_v), T and T^T (delta write) and P^T
 *    (64 x 64 each), e^{g_C} (d_k);
 *  - no gate or a scalar gate adds Q^T and K^T (delta write) in the I/O dtype (d_k 64
 *    elements each) and e^g, e^{g_C - g} per row (2 x 64 fp32);
 *  - one decay per key channel adds instead K e^G (delta write), K e^{g_C - G} (64 d_k
 *    each), their transposes and (Q e^G)^T (d_k 64 each; K e^G's transpose for the
 *    delta write only), fp32;
 *  - one constant decay per head adds the per-token decay gradients (4 bytes per token
 *    and head).
 * Owned by the caller; no initialisation needed. */
size_t gdn_bwd_workspace_size(const gdn_bwd_args *args);

/* Gradients: writes dq, dk, dv, dbeta (DELTA), dlog_alpha (a gate) and dinitial_state
 * (if given). */
int gdn_bwd_chunked(const gdn_bwd_args *args, void *hip_stream);

/*
 * Chunked forward of the diagonal-plus-low-rank transition ("Decoding Hybrid Linear
 * Attention Architectures", sec. 3 item 5: a transition Diag(alpha_t) + a_t b_t^T
 * with an additive write).  Per token, in the state orientation M = S^T used here:
 *
 *   M_t = Diag(alpha_t) M_{t-1} + b_t (a_t^T M_{t-1}) + k_t v_t^T,   o_t = M_t^T q_t
 *
 * i.e. S_t = S_{t-1} (Diag(alpha_t) + a_t b_t^T) + v_t k_t^T.  With b_t = k_t,
 * a_t = -alpha_t beta_t k_t and v scaled by beta_t it is the (gated) delta rule of
 * gdn_fwd_chunked; with a_t = 0 it is its additive write.  Computed chunk by chunk
 * (C = 64; the pages' chunkwise algorithm of sec. 5, with the within-chunk low-rank
 * products solved in UT form as for the delta rule).  Every gate: GDN_GATE_NONE,
 * GDN_GATE_HEAD, GDN_GATE_HEAD_CONST (one log alpha per head for every token) and
 * GDN_GATE_KEY (one log alpha per key channel, alpha_t a vector as in sec. 3 item 5);
 * bf16 with d_k 64 or 128, fp32 with d_k 64 (GDN_ERR_UNSUPPORTED otherwise); d_v 64
 * or 128.  Batch and varlen modes, partial chunks, empty sequences, alignment and
 * validation as for gdn_fwd_chunked.  GDN_GATE_KEY needs a workspace of
 * gdn_dplr_workspace_size bytes (256-byte aligned, else GDN_ERR_WORKSPACE); the other
 * gates need none and ignore the two workspace fields.
 * The recurrence is stable only when the transitions are (e.g. a = -kappa,
 * b = kappa * w with |kappa| = 1 and 0 <= w <= 1); the library does not check this.
 */
typedef struct {
  int B, T, H, d_k, d_v, chunk, N; /* as in gdn_fwd_args                          */
  gdn_dtype dtype;                 /* dtype of q, k, v, a, b, o                   */
  gdn_gate gate;                   /* any gdn_gate                                */
  const void *q, *k, *a, *b;       /* [B, T, H, d_k], dtype                       */
  const void *v;                   /* [B, T, H, d_v], dtype                       */
  const float *log_alpha;          /* NONE: NULL; HEAD: [B, T, H]; HEAD_CONST: [H];
                                      KEY: [B, T, H, d_k]; fp32                   */
  const float *initial_state;      /* NULL (zeros) or [N, H, d_k, d_v] fp32       */
  const int32_t *cu_seqlens;       /* NULL or [N + 1] int32 (device)              */
  void *o;                         /* out: [B, T, H, d_v], dtype                  */
  float *final_state;              /* out: NULL or [N, H, d_k, d_v]; may alias
                                      initial_state                               */
  void *workspace;                 /* GDN_GATE_KEY: device scratch, see below     */
  size_t workspace_bytes;
} gdn_dplr_args;

/* Workspace bytes gdn_fwd_dplr needs: 0 for every gate but GDN_GATE_KEY (and for
 * invalid arguments).  With the per-channel gate, per chunk slot (floor(B T / 64) + N
 * slots) and head: (I - A_ab)^-1, A_ak, P_qb, P_qk (64 x 64 each), A e^{G_{j-1}} and
 * Q e^G (64 d_k each), (B e^{G_C - G})^T and (K e^{G_C - G})^T (d_k 64 each) and
 * e^{G_C} (d_k), fp32.  Owned by the caller; no initialisation needed. */
size_t gdn_dplr_workspace_size(const gdn_dplr_args *args);

/* Diagonal-plus-low-rank forward: writes o (and final_state when non-NULL). */
int gdn_fwd_dplr(const gdn_dplr_args *args, void *hip_stream);

/* One decode token per stream of the diagonal-plus-low-rank transition, the state
 * updated in place (the constant-cost decode update of "Decoding Hybrid Linear
 * Attention Architectures", sec. 6, with the transition of sec. 3 item 5):
 *   M' = Diag(alpha) M + b (a^T M) + k v^T,   o = M'^T q.
 * All gates (none, one decay per (stream, head), one constant decay per head [H], one
 * per key channel); any dtype; d_k, d_v in {64, 128}.  Validation as for
 * gdn_fwd_recurrent_step. */
typedef struct {
  int N, H, d_k, d_v;     /* streams, heads, head dims (each 64 or 128); N H at most
                             2^31 - 1 (GDN_ERR_UNSUPPORTED otherwise)              */
  gdn_dtype dtype;        /* dtype of q, k, a, b, v, o                                 */
  gdn_gate gate;
  const void *q, *k, *a, *b; /* [N, H, d_k]                                            */
  const void *v;          /* [N, H, d_v]                                               */
  const float *log_alpha; /* NONE: NULL; HEAD: [N,H]; KEY: [N,H,d_k]; HEAD_CONST: [H]   */
  float *state;           /* in/out: [N, H, d_k, d_v] fp32 (M = S^T), 16-byte aligned  */
  void *o;                /* out: [N, H, d_v], dtype                                   */
} gdn_dplr_step_args;

int gdn_fwd_dplr_step(const gdn_dplr_step_args *args, void *hip_stream);

/* Serving decode of the diagonal-plus-low-rank transition: L tokens per stream against
 * a pool of states, with the per-token update of gdn_fwd_dplr_step and the pool and
 * slot convention of gdn_fwd_decode (src_slots[n] read once, the state after token t
 * stored into dst_slots[n, t] when in [0, pool_size), a stream with src outside
 * [0, pool_size) is padding; the dst slots of one call must differ from each other and
 * from the other streams' src slots).  Every gate; any dtype; d_k, d_v in {64, 128}. */
typedef struct {
  int N, L, H, d_k, d_v;     /* streams, tokens per stream (>= 1), heads, head dims     */
  gdn_dtype dtype;           /* dtype of q, k, a, b, v, o                               */
  gdn_gate gate;
  const void *q, *k, *a, *b; /* [N, L, H, d_k]                                          */
  const void *v;             /* [N, L, H, d_v]                                          */
  const float *log_alpha;    /* NONE: NULL; HEAD: [N,L,H]; KEY: [N,L,H,d_k]; HEAD_CONST: [H] */
  float *state_pool;         /* in/out: [pool_size, H, d_k, d_v] fp32 (M = S^T)        */
  int pool_size;             /* number of slots (>= 1)                                  */
  const int32_t *src_slots;  /* [N] device                                              */
  const int32_t *dst_slots;  /* [N, L] device                                           */
  void *o;                   /* out: [N, L, H, d_v], dtype                              */
} gdn_dplr_decode_args;

int gdn_fwd_dplr_decode(const gdn_dplr_decode_args *args, void *hip_stream);

/* Static description of a status code (never NULL). */
const char *gdn_status_str(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */

// gdn_kernels.h -- launch interface between the host ABI and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// GATE_CONST: one decay per head, the same at every token (read with a token stride
// of 0); the pipelined kernel has an instantiation of its own for it, the other
// kernels run it as GATE_HEAD with la_stride = 0.
enum { GATE_NONE = 0, GATE_HEAD = 1, GATE_KEY = 2, GATE_CONST = 3 };

struct FwdParams {
  const void *q, *k, *v;         // [tokens, H, d_k] / [tokens, H, d_v]
  const float *beta;             // [tokens, H]
  const float *log_alpha;        // NULL | [tokens, H] | [tokens, H, d_k]
  const float *init_state;       // NULL | [N, H, d_k, d_v]
  float *final_state;            // NULL | [N, H, d_k, d_v]
  void *o;                       // [tokens, H, d_v]
  const int32_t *cu_seqlens;     // NULL (batch) | [N + 1]
  const int32_t *order;          // NULL | processing order of the sequences (varlen)
  int N, H;
  int T;                         // tokens per batch row, or packed total (varlen)
  int dv;                        // full d_v
  int nb;                        // number of d_v blocks per (sequence, head)
  // Per-key-channel gate on the pipelined kernel: operands prepared per chunk by
  // launch_key_prep (q and k then point at the pre-scaled Q e^G and K e^G).
  const void *k_hat;             // [tokens, H, d_k] K e^{g_C - G}
  const void *tp_img;            // [slots, H] 16 KiB LDS images of T diag(beta) and P
  const float *egc;              // [slots, H, d_k] e^{g_C} per key channel
  // Scalar (per-head) gate: elements between consecutive tokens of log_alpha, H
  // for one value per (token, head), 0 for one constant value per head.  Read by
  // the fused kernel only (the pipelined kernel takes per-token values).
  int la_stride;
  // Backward pass only (fused kernel): when set, every chunk's entering state is
  // stored here ([slots, H, d_k, d_v], slot of chunk c as for key_slots) and o may be
  // NULL (not written).
  float *chunk_states;
  // launch_key_window only: process the chunk window [c_lo, c_hi) of every sequence,
  // the state entering the window read from init_state and the state leaving it
  // written to final_state.
  int c_lo = 0, c_hi = 1 << 30;
};

// Chunk slots of the per-key-channel preparation: chunk c of sequence n (first token
// t0) is slot floor(t0 / 64) + c + n, unique and below floor(total / 64) + N.
inline long key_slots(long total_tokens, int N) { return total_tokens / 64 + N; }

struct StepParams {
  const void *q, *k, *v;
  const float *beta, *log_alpha;
  float *state;
  void *o;
  int N, H;
  int la_stride;  // scalar gate: elements of log_alpha between streams (H, or 0: per head)
};

// L decode tokens per stream against a pool of states: slot src[n] is read, the
// state after token t is stored into slot dst[n * L + t] when that is in [0, P).
struct DecodeParams {
  const void *q, *k, *v;
  const float *beta, *log_alpha;
  float *pool;
  const int *src, *dst;
  void *o;
  int N, L, H, P;
  int la_stride;  // scalar gate: elements of log_alpha between tokens (H, or 0: per head)
};

// Backward pass of the chunked delta rule and of the additive write (no gate, the
// scalar gate or a constant per-head decay).  The chunk states come from a forward
// launched with FwdParams::chunk_states; the slots of the chunks are numbered as for
// key_slots.
struct BwdParams {
  const void *q, *k, *v, *dout;  // [tokens, H, d_k] / [tokens, H, d_v], I/O dtype
  const float *beta, *log_alpha; // [tokens, H] (beta NULL for the additive write; log_alpha
                                 // NULL without a gate, read at t * la_stride + h)
  const float *dfinal;           // NULL | [N, H, d_k, d_v]
  const int32_t *cu_seqlens;     // NULL (batch) | [N + 1]
  // workspace: chunk-entering states and chunk-end state gradients [slots, H, d_k, d_v],
  // dDelta [slots, H, 64, d_v], T and T^T (delta write) and P^T [slots, H, 64, 64],
  // e^{G_C} [slots, H, d_k] (fp32); Q^T and K^T (delta write) [slots, H, d_k, 64] in the
  // I/O dtype; e^G and e^{G_C - G} per row [slots, H, 64] (fp32, 0 past the sequence end)
  const float *states;
  float *dmc, *dd, *tm, *tmT, *pmT, *gam, *egr, *etr;
  void *qT, *kT;
  void *dq, *dk, *dv_out;        // outputs, I/O dtype
  float *dbeta, *dlog_alpha;     // [tokens, H]; dbeta NULL for the additive write, dlog_alpha
                                 // NULL without a gate (per token also for a constant decay)
  float *dinit;                  // NULL | [N, H, d_k, d_v]
  int N, H, T, dv;
  int la_stride;                 // H, or 0 for one constant decay per head
  long slots;
};
hipError_t launch_bwd(const BwdParams &p, int dtype, int dk, int gate, bool add, hipStream_t stream);
// x[0 .. n) = 0
hipError_t launch_fill_zero(float *x, size_t n, hipStream_t stream);
// out[h] = sum over tokens of x[t, h] (deterministic order)
hipError_t launch_sum_tokens(const float *x, long tokens, int H, float *out, hipStream_t stream);

// Backward pass with one decay per key channel: four launches over a workspace of
// per-chunk operands (every array indexed by chunk slot, as for key_slots, then head).
struct BwdKeyParams {
  const void *q, *k, *v, *dout;  // [tokens, H, d_k] / [tokens, H, d_v], I/O dtype
  const float *beta;             // [tokens, H]; NULL for the additive write
  const float *log_alpha;        // [tokens, H, d_k]
  const float *init_state;       // NULL | [N, H, d_k, d_v]
  const float *dfinal;           // NULL | [N, H, d_k, d_v]
  const int32_t *cu_seqlens;     // NULL (batch) | [N + 1]
  // workspace (fp32): chunk-entering states and chunk-end state gradients [S, H, d_k, d_v],
  // dDelta [S, H, 64, d_v], T and T^T [S, H, 64, 64] (delta write), P^T [S, H, 64, 64],
  // K e^G and K e^{g_C - G} [S, H, 64, d_k], their transposes and (Q e^G)^T [S, H, d_k, 64],
  // e^{g_C} [S, H, d_k]
  float *states, *dmc, *dd, *tm, *tmT, *pmT, *kt, *kh, *ktT, *qtT, *khT, *gam;
  // the scalar gates' reverse pass (launch_bwdk_rev) reads instead of kh, qtT and ktT:
  // Q^T and K^T [S, H, d_k, 64] (I/O dtype), e^G and e^{G_C - G} per row [S, H, 64]
  const void *qT, *kT;
  const float *egr, *etr;
  void *dq, *dk, *dv_out;        // outputs, I/O dtype
  float *dbeta;                  // [tokens, H]; NULL for the additive write
  float *dlog_alpha;             // [tokens, H, d_k]
  float *dinit;                  // NULL | [N, H, d_k, d_v]
  int N, H, T, dv;
  long slots;
  int states_ready;              // the chunk-entering states are already in `states`
};
hipError_t launch_bwd_key(const BwdKeyParams &p, int dtype, int dk, bool add, hipStream_t stream);
// the scalar gates' reverse state pass (chunk-end state gradients, dDelta, dV, initial-
// state gradient) from P^T, T^T, Q^T, K^T and the row factors already in the workspace
hipError_t launch_bwdk_rev(const BwdKeyParams &p, int dtype, int dk, bool add, hipStream_t stream);

// Forward of the diagonal-plus-low-rank transition (no gate or the scalar gate).
struct DplrParams {
  const void *q, *k, *v, *a, *b;  // [tokens, H, d_k] (v: d_v), I/O dtype
  const float *log_alpha;         // NULL | [tokens, H] (read at token * la_stride + h)
  const float *init_state;        // NULL | [N, H, d_k, d_v]
  float *final_state;             // NULL | [N, H, d_k, d_v]
  void *o;                        // [tokens, H, d_v]
  const int32_t *cu_seqlens;      // NULL (batch) | [N + 1]
  int N, H, T, dv, la_stride;
};
hipError_t launch_dplr(const DplrParams &p, int dtype, int dk, int gate, hipStream_t stream);
// The same transition with one decay per key channel: a parallel preparation per
// (chunk, head) into the fp32 workspace arrays below (slot of chunk c as for key_slots),
// then one serial pass per (sequence, head, 64 or 32 value columns).
struct DplrKeyParams {
  const void *q, *k, *v, *a, *b;  // [tokens, H, d_k] (v: d_v), I/O dtype
  const float *log_alpha;         // [tokens, H, d_k]
  const float *init_state;        // NULL | [N, H, d_k, d_v]
  float *final_state;             // NULL | [N, H, d_k, d_v]
  void *o;                        // [tokens, H, d_v]
  const int32_t *cu_seqlens;      // NULL (batch) | [N + 1]
  // per slot-head, each matrix as a bf16 hi half then a bf16 lo half (hi + lo = the
  // fp32 value), row-major
  __bf16 *tm, *aak, *pqb, *pqk;   // [slots, H, 2, 64, 64]
  __bf16 *at, *qg;                // [slots, H, 2, 64, d_k]
  __bf16 *bhT, *khT;              // [slots, H, 2, d_k, 64]
  float *gam;                     // [slots, H, d_k]
  int N, H, T, dv;
  long slots;
};
hipError_t launch_dplr_key(const DplrKeyParams &p, int dtype, int dk, hipStream_t stream);
// One decode token per stream of the diagonal-plus-low-rank transition, state in place.
struct DplrStepParams {
  const void *q, *k, *v, *a, *b;  // [N, H, d_k] (v: d_v), I/O dtype
  const float *log_alpha;         // NULL | [N, H] (read at n * la_stride + h) | [N, H, d_k]
  float *state;                   // [N, H, d_k, d_v], read then overwritten
  void *o;                        // [N, H, d_v]
  int N, H, la_stride;
};
hipError_t launch_dplr_step(const DplrStepParams &p, int dtype, int dk, int dv, int gate, hipStream_t stream);
// L decode tokens per stream of the same transition against a pool of states.
struct DplrDecodeParams {
  const void *q, *k, *v, *a, *b;  // [N, L, H, d_k] (v: d_v), I/O dtype
  const float *log_alpha;         // NULL | [N, L, H] (read at token * la_stride + h) | [N, L, H, d_k]
  float *pool;                    // [P, H, d_k, d_v]
  const int32_t *src, *dst;       // [N], [N, L]
  void *o;                        // [N, L, H, d_v]
  int N, L, H, P, la_stride;
};
hipError_t launch_dplr_decode(const DplrDecodeParams &p, int dtype, int dk, int dv, int gate, hipStream_t stream);

// dtype: 0 fp32, 1 bf16.  Each launcher returns hipSuccess or the launch error.
// dvb: columns of d_v per workgroup (32 or 64).
// add: the additive write (S += v k^T; beta unused) instead of the delta rule.
hipError_t launch_fwd_fused(const FwdParams &p, int dtype, int dk, int dvb, int gate, bool add,
                            hipStream_t stream);
// Software-pipelined forward for bf16, d_k = 128, 64-column value blocks (nb = d_v / 64);
// gate: GATE_NONE, GATE_HEAD, GATE_CONST or GATE_KEY (the latter with the prepared
// operands, delta write only); add: the additive write.
// Gate NONE or HEAD; gate KEY after launch_key_prep, with the k_hat, tp_img, egc fields.
// With chunk_states set (every gate): the chunk-entering states instead of o.
hipError_t launch_fwd_pipe(const FwdParams &p, int gate, bool add, hipStream_t stream);
// Per-key-channel gate, bf16, d_k = 128: for every chunk (all in parallel) the
// pre-scaled operands K e^G, Q e^G, K e^{g_C - G}, e^{g_C}, and T diag(beta) and P as
// the LDS images the pipelined kernel loads.
struct KeyPrepParams {
  const void *q, *k;             // [tokens, H, 128] bf16
  const float *beta;             // [tokens, H]
  const float *log_alpha;        // [tokens, H, 128]
  const int32_t *cu_seqlens;     // NULL | [N + 1]
  void *q_g, *k_g, *k_hat;       // [tokens, H, 128] bf16 outputs
  void *tp_img;                  // [slots, H, 16384 B]
  float *egc;                    // [slots, H, 128]
  int N, H, T;
  int c_lo = 0, c_hi = 1 << 30;  // prepare only chunks c_lo <= c < c_hi of each sequence
  int win_items = 0;             // batch mode: walk only the window's (sequence, chunk, head)
};
// add: operands for the additive write (no beta, no T, no K e^G).
hipError_t launch_key_prep(const KeyPrepParams &p, long slots, bool add, hipStream_t stream);
// One launch: the state pass over fp's chunk window (fp.N * fp.H * fp.nb workgroups)
// and, on nprep more workgroups, the preparation of kp's chunk window.
hipError_t launch_key_window(const FwdParams &fp, const KeyPrepParams &kp, long slots, int nprep, bool add,
                             hipStream_t stream);
int device_cus();
hipError_t launch_seq_order(const int32_t *cu_seqlens, int N, int32_t *order, hipStream_t stream);
hipError_t launch_recurrent_step(const StepParams &p, int dtype, int dk, int dv, int gate, bool add,
                                 hipStream_t stream);
hipError_t launch_decode(const DecodeParams &p, int dtype, int dk, int dv, int gate, bool add,
                         hipStream_t stream);

}  // namespace gdn

// gdn_kernels.h -- launch interface between the host ABI and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

enum { GATE_NONE = 0, GATE_HEAD = 1, GATE_KEY = 2 };

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
};

struct StepParams {
  const void *q, *k, *v;
  const float *beta, *log_alpha;
  float *state;
  void *o;
  int N, H;
};

// dtype: 0 fp32, 1 bf16.  Each launcher returns hipSuccess or the launch error.
// dvb: columns of d_v per workgroup (32 or 64).
hipError_t launch_fwd_fused(const FwdParams &p, int dtype, int dk, int dvb, int gate,
                            hipStream_t stream);
// Software-pipelined forward for bf16, d_k = 128, 64-column value blocks (nb = d_v / 64),
// gate NONE or HEAD.
hipError_t launch_fwd_pipe(const FwdParams &p, int gate, hipStream_t stream);
hipError_t launch_seq_order(const int32_t *cu_seqlens, int N, int32_t *order, hipStream_t stream);
hipError_t launch_recurrent_step(const StepParams &p, int dtype, int dk, int dv, int gate,
                                 hipStream_t stream);

}  // namespace gdn

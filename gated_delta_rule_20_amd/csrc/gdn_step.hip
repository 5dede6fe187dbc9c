// gdn_step.hip -- decode: one token per stream in place, and L tokens per stream against a state pool.
//
// The recurrent mode of the (gated) delta rule ("Decoding Hybrid Linear Attention
// Architectures", sec. 6: constant-cost update of the fixed-size state per decoded
// token; sec. 3 item 6 for the order decay -> erase -> write).  With the state kept
// as M = S^T (d_k x d_v) and a = exp(log alpha):
//   r = (Diag(a) M)^T k,   w = beta (v - r),   M' = Diag(a) M + k w^T,
//   o = M'^T q = (Diag(a) M)^T q + w (q . k)
// so one read of M gives both reductions r and (Diag(a) M)^T q, and one write stores
// M'.  The kernel is bound by HBM traffic (2 * 4 * d_k * d_v bytes per stream).
// The additive write (sec. 3 item 4: gated linear attention; RetNet; the plain
// linear transformer) is the same body with w = v (no erase, no beta).
//
// One workgroup (256 threads) per (stream, head).  Thread (row group rg, column
// quad cq) holds d_k / RG rows x 4 columns of M in registers: 16-byte coalesced
// loads and stores, partial reductions combined in LDS in a fixed order.  The same
// body serves the pooled decode below (states addressed by slot, one or more tokens
// per stream).
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

template <typename E, int DK, int DV, int GATE, bool ADD>
__global__ __launch_bounds__(256) void recurrent_step_kernel(StepParams p) {
  constexpr int CQ = DV / 4;    // column quads
  constexpr int RG = 256 / CQ;  // row groups
  constexpr int RP = DK / RG;   // rows per thread
  static_assert(RP >= 1 && RG * RP == DK, "step geometry");
  __shared__ float qs[DK], ks[DK], as_[DK];
  __shared__ f32x4 red_r[RG][CQ], red_s[RG][CQ];
  __shared__ float qk_s;

  const int pair = blockIdx.x;  // stream * H + head
  const int tid = threadIdx.x, cq = tid % CQ, rg = tid / CQ;
  const E *q = (const E *)p.q + (size_t)pair * DK;
  const E *k = (const E *)p.k + (size_t)pair * DK;
  if (tid < DK) {
    qs[tid] = to_f(q[tid]);
    ks[tid] = to_f(k[tid]);
    float a = 1.f;
    if (GATE == GATE_HEAD) a = __expf(p.log_alpha[(size_t)(pair / p.H) * p.la_stride + pair % p.H]);
    if (GATE == GATE_KEY) a = __expf(p.log_alpha[(size_t)pair * DK + tid]);
    as_[tid] = a;
  }
  float *st = p.state + (size_t)pair * DK * DV;
  f32x4 m[RP];
#pragma unroll
  for (int u = 0; u < RP; ++u) m[u] = *(const f32x4 *)(st + (size_t)(rg * RP + u) * DV + 4 * cq);
  const E *vp = (const E *)p.v + (size_t)pair * DV + 4 * cq;  // needed only after the reduction
  f32x4 vv;
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = to_f(vp[e]);
  const float beta = ADD ? 1.f : p.beta[pair];
  __syncthreads();

  f32x4 r = zero4(), s = zero4();
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    const int row = rg * RP + u;
    m[u] *= as_[row];
    r += m[u] * ks[row];
    s += m[u] * qs[row];
  }
  red_r[rg][cq] = r;
  red_s[rg][cq] = s;
  if (tid < 64) {
    float d = 0.f;
    for (int i = tid; i < DK; i += 64) d += qs[i] * ks[i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
    if (tid == 0) qk_s = d;
  }
  __syncthreads();

  f32x4 R = zero4(), S = zero4();
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    R += red_r[g][cq];
    S += red_s[g][cq];
  }
  f32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = ADD ? vv[e] : beta * (vv[e] - R[e]);
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    const int row = rg * RP + u;
    *(f32x4 *)(st + (size_t)row * DV + 4 * cq) = m[u] + ks[row] * w;
  }
  if (rg == 0) {
    E *o = (E *)p.o + (size_t)pair * DV + 4 * cq;
    const float qk = qk_s;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = to_e<E>(S[e] + w[e] * qk);
  }
}

// Serving decode with one token per stream (L = 1): the body of recurrent_step_kernel
// with the state read from and written to pool slots.
template <typename E, int DK, int DV, int GATE, bool ADD>
__global__ __launch_bounds__(256) void decode_one_kernel(DecodeParams p) {
  constexpr int CQ = DV / 4;
  constexpr int RG = 256 / CQ;
  constexpr int RP = DK / RG;
  static_assert(RP >= 1 && RG * RP == DK, "decode geometry");
  __shared__ float qs[DK], ks[DK], as_[DK];
  __shared__ f32x4 red_r[RG][CQ], red_s[RG][CQ];
  __shared__ float qk_s;

  const int pair = blockIdx.x, n = pair / p.H, h = pair % p.H;  // token index == pair (L = 1)
  const int src = p.src[n];
  if (src < 0 || src >= p.P) return;  // padding stream: nothing read or written
  const int tid = threadIdx.x, cq = tid % CQ, rg = tid / CQ;
  if (tid < DK) {
    qs[tid] = to_f(((const E *)p.q)[(size_t)pair * DK + tid]);
    ks[tid] = to_f(((const E *)p.k)[(size_t)pair * DK + tid]);
    float a = 1.f;
    if (GATE == GATE_HEAD) a = __expf(p.log_alpha[(size_t)n * p.la_stride + h]);
    if (GATE == GATE_KEY) a = __expf(p.log_alpha[(size_t)pair * DK + tid]);
    as_[tid] = a;
  }
  const size_t slot = (size_t)p.H * DK * DV, head = (size_t)h * DK * DV;
  const float *st = p.pool + (size_t)src * slot + head;
  f32x4 m[RP];
#pragma unroll
  for (int u = 0; u < RP; ++u) m[u] = *(const f32x4 *)(st + (size_t)(rg * RP + u) * DV + 4 * cq);
  const E *vp = (const E *)p.v + (size_t)pair * DV + 4 * cq;  // needed only after the reduction
  f32x4 vv;
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = to_f(vp[e]);
  const float beta = ADD ? 1.f : p.beta[pair];
  __syncthreads();

  f32x4 r = zero4(), s = zero4();
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    const int row = rg * RP + u;
    m[u] *= as_[row];
    r += m[u] * ks[row];
    s += m[u] * qs[row];
  }
  red_r[rg][cq] = r;
  red_s[rg][cq] = s;
  if (tid < 64) {
    float d = 0.f;
    for (int i = tid; i < DK; i += 64) d += qs[i] * ks[i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
    if (tid == 0) qk_s = d;
  }
  __syncthreads();

  f32x4 R = zero4(), S = zero4();
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    R += red_r[g][cq];
    S += red_s[g][cq];
  }
  f32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = ADD ? vv[e] : beta * (vv[e] - R[e]);
#pragma unroll
  for (int u = 0; u < RP; ++u) m[u] += ks[rg * RP + u] * w;
  if (rg == 0) {
    E *o = (E *)p.o + (size_t)pair * DV + 4 * cq;
    const float qk = qk_s;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = to_e<E>(S[e] + w[e] * qk);
  }
  const int dst = p.dst[n];
  if (dst >= 0 && dst < p.P) {
    float *out = p.pool + (size_t)dst * slot + head;
#pragma unroll
    for (int u = 0; u < RP; ++u) *(f32x4 *)(out + (size_t)(rg * RP + u) * DV + 4 * cq) = m[u];
  }
}

// Serving decode: L tokens per stream in one launch, the state read once from its
// pool slot, kept in registers across the tokens, and stored only where a slot is
// given (every token for speculative drafts, the last one for plain decoding).  The
// per-token body is the one above.  The inputs of up to TB tokens are staged in LDS
// together, issued with the state load, so one memory latency covers them; q . k of
// every staged token is formed once per batch, and the partial sums alternate
// between two LDS buffers, so each token needs a single barrier.
template <typename E, int DK, int DV, int GATE, bool ADD>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  constexpr int CQ = DV / 4;
  constexpr int RG = 256 / CQ;
  constexpr int RP = DK / RG;
  constexpr int TB = 8;  // tokens staged in LDS at a time
  static_assert(RP >= 1 && RG * RP == DK, "decode geometry");
  __shared__ float qs[TB][DK], ks[TB][DK], as_[GATE == GATE_KEY ? TB : 1][DK], vs[TB][DV];
  __shared__ float bs[TB], ah[TB], qk_s[TB];
  __shared__ f32x4 red_r[2][RG][CQ], red_s[2][RG][CQ];

  const int n = blockIdx.x / p.H, h = blockIdx.x % p.H;
  const int src = p.src[n];
  if (src < 0 || src >= p.P) return;  // padding stream: nothing read or written
  const int tid = threadIdx.x, cq = tid % CQ, rg = tid / CQ;
  const size_t slot = (size_t)p.H * DK * DV, head = (size_t)h * DK * DV;
  const float *st = p.pool + (size_t)src * slot + head;
  f32x4 m[RP];
#pragma unroll
  for (int u = 0; u < RP; ++u) m[u] = *(const f32x4 *)(st + (size_t)(rg * RP + u) * DV + 4 * cq);

  for (int t0 = 0; t0 < p.L; t0 += TB) {
    const int nt = p.L - t0 < TB ? p.L - t0 : TB;
    if (t0 > 0) __syncthreads();  // the previous batch is done with the staged inputs
    const size_t i0 = ((size_t)n * p.L + t0) * p.H + h;  // (stream, token t0, head)
    for (int x = tid; x < nt * DK; x += 256) {
      const int tt = x / DK, c = x % DK;
      const size_t i = i0 + (size_t)tt * p.H;
      qs[tt][c] = to_f(((const E *)p.q)[i * DK + c]);
      ks[tt][c] = to_f(((const E *)p.k)[i * DK + c]);
      if (GATE == GATE_KEY) as_[tt][c] = __expf(p.log_alpha[i * DK + c]);
    }
    for (int x = tid; x < nt * DV; x += 256) {
      const int tt = x / DV, c = x % DV;
      vs[tt][c] = to_f(((const E *)p.v)[(i0 + (size_t)tt * p.H) * DV + c]);
    }
    if (tid < nt) {
      const size_t i = i0 + (size_t)tid * p.H;
      bs[tid] = ADD ? 1.f : p.beta[i];
      ah[tid] = GATE == GATE_HEAD ? __expf(p.log_alpha[((size_t)n * p.L + t0 + tid) * p.la_stride + h]) : 1.f;
    }
    __syncthreads();
    // q . k of each staged token: wave w takes tokens w, w + 4
    for (int tt = tid >> 6; tt < nt; tt += 4) {
      float d = 0.f;
      for (int c = tid & 63; c < DK; c += 64) d += qs[tt][c] * ks[tt][c];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
      if ((tid & 63) == 0) qk_s[tt] = d;
    }

    for (int tt = 0; tt < nt; ++tt) {
      const int t = t0 + tt, b = t & 1;
      f32x4 r = zero4(), s = zero4();
#pragma unroll
      for (int u = 0; u < RP; ++u) {
        const int row = rg * RP + u;
        if (GATE == GATE_KEY) m[u] *= as_[tt][row];
        if (GATE == GATE_HEAD) m[u] *= ah[tt];
        r += m[u] * ks[tt][row];
        s += m[u] * qs[tt][row];
      }
      red_r[b][rg][cq] = r;
      red_s[b][rg][cq] = s;
      __syncthreads();

      f32x4 R = zero4(), S = zero4();
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        R += red_r[b][g][cq];
        S += red_s[b][g][cq];
      }
      const float beta = bs[tt];
      const f32x4 vv = *(const f32x4 *)&vs[tt][4 * cq];
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = ADD ? vv[e] : beta * (vv[e] - R[e]);
#pragma unroll
      for (int u = 0; u < RP; ++u) m[u] += ks[tt][rg * RP + u] * w;
      if (rg == 0) {
        E *o = (E *)p.o + (i0 + (size_t)tt * p.H) * DV + 4 * cq;
        const float qk = qk_s[tt];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = to_e<E>(S[e] + w[e] * qk);
      }
      const int dst = p.dst[(size_t)n * p.L + t];
      if (dst >= 0 && dst < p.P) {
        float *out = p.pool + (size_t)dst * slot + head;
#pragma unroll
        for (int u = 0; u < RP; ++u) *(f32x4 *)(out + (size_t)(rg * RP + u) * DV + 4 * cq) = m[u];
      }
    }
  }
}

// Instantiate a kernel template K<E, DK, DV, GATE, ADD> for the run-time gate and
// write rule.
#define GDN_STEP_LAUNCH(K, P)                                                                          \
  do {                                                                                                 \
    switch (gate * 2 + (add ? 1 : 0)) {                                                                \
      case 0: hipLaunchKernelGGL((K<E, DK, DV, GATE_NONE, false>), dim3(blocks), dim3(256), 0, stream, P); break; \
      case 1: hipLaunchKernelGGL((K<E, DK, DV, GATE_NONE, true>), dim3(blocks), dim3(256), 0, stream, P); break;  \
      case 2: hipLaunchKernelGGL((K<E, DK, DV, GATE_HEAD, false>), dim3(blocks), dim3(256), 0, stream, P); break; \
      case 3: hipLaunchKernelGGL((K<E, DK, DV, GATE_HEAD, true>), dim3(blocks), dim3(256), 0, stream, P); break;  \
      case 4: hipLaunchKernelGGL((K<E, DK, DV, GATE_KEY, false>), dim3(blocks), dim3(256), 0, stream, P); break;  \
      case 5: hipLaunchKernelGGL((K<E, DK, DV, GATE_KEY, true>), dim3(blocks), dim3(256), 0, stream, P); break;   \
      default: return hipErrorInvalidValue;                                                            \
    }                                                                                                  \
  } while (0)

template <typename E, int DK, int DV>
hipError_t launch_g(const StepParams &p, int gate, bool add, hipStream_t stream) {
  const int blocks = p.N * p.H;
  if (blocks == 0) return hipSuccess;
  GDN_STEP_LAUNCH(recurrent_step_kernel, p);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const StepParams &p, int dk, int dv, int gate, bool add, hipStream_t stream) {
  if (dk == 128 && dv == 128) return launch_g<E, 128, 128>(p, gate, add, stream);
  if (dk == 128 && dv == 64) return launch_g<E, 128, 64>(p, gate, add, stream);
  if (dk == 64 && dv == 128) return launch_g<E, 64, 128>(p, gate, add, stream);
  if (dk == 64 && dv == 64) return launch_g<E, 64, 64>(p, gate, add, stream);
  return hipErrorInvalidValue;
}

template <typename E, int DK, int DV>
hipError_t launch_dg(const DecodeParams &p, int gate, bool add, hipStream_t stream) {
  const int blocks = p.N * p.H;
  if (blocks == 0) return hipSuccess;
  if (p.L == 1)
    GDN_STEP_LAUNCH(decode_one_kernel, p);
  else
    GDN_STEP_LAUNCH(decode_kernel, p);
  return hipGetLastError();
}

#undef GDN_STEP_LAUNCH

template <typename E>
hipError_t launch_de(const DecodeParams &p, int dk, int dv, int gate, bool add, hipStream_t stream) {
  if (dk == 128 && dv == 128) return launch_dg<E, 128, 128>(p, gate, add, stream);
  if (dk == 128 && dv == 64) return launch_dg<E, 128, 64>(p, gate, add, stream);
  if (dk == 64 && dv == 128) return launch_dg<E, 64, 128>(p, gate, add, stream);
  if (dk == 64 && dv == 64) return launch_dg<E, 64, 64>(p, gate, add, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int dtype, int dk, int dv, int gate, bool add,
                         hipStream_t stream) {
  return dtype == 1 ? launch_de<bf16>(p, dk, dv, gate, add, stream) : launch_de<float>(p, dk, dv, gate, add, stream);
}

hipError_t launch_recurrent_step(const StepParams &p, int dtype, int dk, int dv, int gate, bool add,
                                 hipStream_t stream) {
  return dtype == 1 ? launch_e<bf16>(p, dk, dv, gate, add, stream) : launch_e<float>(p, dk, dv, gate, add, stream);
}

}  // namespace gdn

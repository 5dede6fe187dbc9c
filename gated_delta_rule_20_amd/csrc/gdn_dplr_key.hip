// gdn_dplr_key.hip -- chunked forward of the diagonal-plus-low-rank transition with one
// decay per key channel ("Decoding Hybrid Linear Attention Architectures", sec. 3 item
// 5: S_t = S_{t-1} (Diag(alpha_t) + a_t b_t^T) + v_t k_t^T, with alpha_t per channel).
//
// In the state orientation M = S^T, token t reads u_t = a_t^T M_{t-1} and writes
// M_t = Diag(alpha_t) M_{t-1} + b_t u_t + k_t v_t^T; o_t = M_t^T q_t.  Per chunk of 64
// tokens, with G[r][c] the chunk-local inclusive prefix of log alpha of channel c and
// Gp[j] = G[j - 1] (Gp[0] = 0):
//   A_ab[j][i] = sum_c a_j[c] b_i[c] e^{Gp[j][c] - G[i][c]},  A_ak likewise with k  (i < j)
//   P_qb[r][i] = sum_c q_r[c] b_i[c] e^{G[r][c] - G[i][c]},   P_qk likewise with k  (i <= r)
//   U = (I - A_ab)^-1 ((A e^{Gp}) M0 + A_ak V)                 (the rows u_j)
//   O = (Q e^G) M0 + P_qb U + P_qk V
//   M_C = diag(e^{G_C}) M0 + (B e^{G_C - G})^T U + (K e^{G_C - G})^T V.
// The per-channel factors sit inside the contractions over the key channels, so the
// Gram products carry them on their operands, split at row m = 16a + 7 of each 16-row
// block a (e^{x[r] - G[m]} on the row operand, e^{G[m] - G[i]} on the column operand):
// no factor exceeds the decay accumulated over eight tokens.
//
// Two launches: dplrk_prep_kernel (one workgroup per (chunk, head), fully parallel)
// writes the chunk's fp32 operands to the caller's workspace -- (I - A_ab)^-1, A_ak,
// P_qb, P_qk, A e^{Gp}, Q e^G (row-major), (B e^{G_C - G})^T, (K e^{G_C - G})^T
// (channel-major) and e^{G_C}; dplrk_state_kernel (one workgroup per (sequence, head,
// 32 value columns)) walks the chunks in order with the fp32 state block in LDS.
// Products run on the bf16 matrix cores with every fp32 operand split into hi + lo bf16
// terms (about 2^-17 relative error per product); accumulation in fp32.
#include "gdn_common.h"
#include "gdn_kernels.h"
#include "gdn_tile.h"

namespace gdn {

namespace {

constexpr int KC = 64;
constexpr int KBV = 32;
constexpr int SV = KBV + 4;
constexpr int SC = KC + 1;

template <int K, class FA, class FB>
__device__ __forceinline__ f32x4 dprod(FA fa, FB fb, int kbeg = 0, int kend = K) {
  f32x4 acc = zero4();
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32)
    if (k0 + 32 > kbeg && k0 < kend) acc = mm(split8(fa(k0)), split8(fb(k0)), acc);
  return acc;
}

__device__ __forceinline__ bool seq_extent_d(const DplrKeyParams &p, int n, long &tok0, int &len) {
  if (p.cu_seqlens) {
    const int a = p.cu_seqlens[n], b = p.cu_seqlens[n + 1];
    if (a < 0 || b < a || b > p.T) return false;
    tok0 = a;
    len = b - a;
  } else {
    tok0 = (long)n * p.T;
    len = p.T;
  }
  return true;
}

__device__ __forceinline__ bool slot_chunk_d(const DplrKeyParams &p, long slot, long &tb, int &nv) {
  auto tok_start = [&](int sq) -> long { return p.cu_seqlens ? (long)p.cu_seqlens[sq] : (long)sq * p.T; };
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((tok_start(mid) >> 6) + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  long tok0;
  int len;
  if (!seq_extent_d(p, lo, tok0, len)) return false;
  const long c = slot - ((tok0 >> 6) + lo);
  if (c < 0 || 64 * c >= len) return false;
  tb = tok0 + 64 * c;
  nv = (int)min(64L, (long)len - 64 * c);
  return true;
}

template <typename E, int DK>
__global__ __launch_bounds__(256, 1) void dplrk_prep_kernel(DplrKeyParams p) {
  constexpr int SE = DK + 8;  // element pitch of the staged inputs (rows 16-byte aligned)
  constexpr int SG = DK + 4;
  __shared__ __align__(16) E As[KC * SE];
  __shared__ __align__(16) E Bs[KC * SE];
  __shared__ __align__(16) E Ks[KC * SE];
  __shared__ __align__(16) E Qs[KC * SE];
  __shared__ __align__(16) float Gs[KC * SG];
  __shared__ float Ab[KC * SC];  // A_ab
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H;
  const long slot = blockIdx.x / H;
  const int h = blockIdx.x % H;
  long tb;
  int nv;
  if (!slot_chunk_d(p, slot, tb, nv)) return;
  const size_t sh = (size_t)slot * H + h;
  for (int i = tid; i < KC * DK; i += 256) {
    const int r = i / DK, d = i % DK;
    const size_t o = ((size_t)(tb + r) * H + h) * DK + d;
    const bool in = r < nv;
    As[r * SE + d] = in ? ((const E *)p.a)[o] : to_e<E>(0.f);
    Bs[r * SE + d] = in ? ((const E *)p.b)[o] : to_e<E>(0.f);
    Ks[r * SE + d] = in ? ((const E *)p.k)[o] : to_e<E>(0.f);
    Qs[r * SE + d] = in ? ((const E *)p.q)[o] : to_e<E>(0.f);
    Gs[r * SG + d] = in ? p.log_alpha[o] : 0.f;
  }
  for (int i = tid; i < KC * SC; i += 256) Ab[i] = 0.f;
  __syncthreads();
  if (tid < DK) {
    float g = 0.f;
    for (int r = 0; r < KC; ++r) {
      g += Gs[r * SG + tid];
      Gs[r * SG + tid] = g;
    }
    p.gam[sh * DK + tid] = __expf(g);
  }
  __syncthreads();
  auto gp = [&](int j, int c) { return j > 0 ? Gs[(j - 1) * SG + c] : 0.f; };
  for (int i = tid; i < KC * DK; i += 256) {
    const int r = i / DK, d = i % DK;
    const float g = Gs[r * SG + d], gC = Gs[(KC - 1) * SG + d], et = __expf(gC - g);
    p.at[(sh * KC + r) * DK + d] = to_f(As[r * SE + d]) * __expf(gp(r, d));
    p.qg[(sh * KC + r) * DK + d] = to_f(Qs[r * SE + d]) * __expf(g);
    p.bhT[(sh * DK + d) * KC + r] = to_f(Bs[r * SE + d]) * et;
    p.khT[(sh * DK + d) * KC + r] = to_f(Ks[r * SE + d]) * et;
  }
  // the Gram matrices: 16 tiles of each (upper ones zero), ten lower ones computed
  float *const outs[4] = {nullptr, p.aak + sh * KC * KC, p.pqb + sh * KC * KC, p.pqk + sh * KC * KC};
  for (int t = wave; t < 64; t += 4) {
    const int w = t >> 4, tt = t & 15, a = tt >> 2, b = tt & 3;  // matrix w, tile (a, b)
    const int m = 16 * a + 7;
    const bool strict = w < 2;  // A_ab, A_ak: i < j; P_qb, P_qk: i <= r
    const E *X = w < 2 ? As : Qs;
    const E *Y = (w & 1) ? Ks : Bs;
    f32x4 acc = zero4();
    if (b <= a)
      acc = dprod<DK>(
          [&](int k0) {
            f32x8 f;
            const int r = 16 * a + lm;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
              const int c = k0 + 8 * lg + ii;
              const float x = strict ? gp(r, c) : Gs[r * SG + c];
              f[ii] = to_f(X[r * SE + c]) * __expf(x - Gs[m * SG + c]);
            }
            return f;
          },
          [&](int k0) {
            f32x8 f;
            const int i = 16 * b + lm;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
              const int c = k0 + 8 * lg + ii;
              f[ii] = to_f(Y[i * SE + c]) * __expf(Gs[m * SG + c] - Gs[i * SG + c]);
            }
            return f;
          });
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * a + 4 * lg + j, i = 16 * b + lm;
      const float v = (strict ? i < r : i <= r) ? acc[j] : 0.f;
      if (w == 0)
        Ab[r * SC + i] = v;
      else
        outs[w][r * KC + i] = v;
    }
  }
  __syncthreads();
  if (tid < KC) {
    // (I - A_ab)^-1, column c per thread: T[r][c] = [r == c] + sum_{i<r} A_ab[r][i] T[i][c]
    const int c = tid;
    float x[KC];
#pragma unroll
    for (int r = 0; r < KC; ++r) {
      float acc = r == c ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc += Ab[r * SC + i] * x[i];
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < KC; ++r) p.tm[(sh * KC + r) * KC + c] = x[r];
  }
}

template <typename E, int DK>
__global__ __launch_bounds__(256, 1) void dplrk_state_kernel(DplrKeyParams p) {
  __shared__ __align__(16) float Ms[DK * SV];
  __shared__ __align__(16) float Vs[KC * SV];
  __shared__ __align__(16) float Rs[KC * SV];
  __shared__ __align__(16) float Us[KC * SV];
  __shared__ float gsh[DK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H, dv = p.dv, nb = dv / KBV;
  const int jb = blockIdx.x % nb, pair = blockIdx.x / nb;
  const int n = pair / H, h = pair % H, col0 = jb * KBV;
  long tok0;
  int len;
  if (!seq_extent_d(p, n, tok0, len)) return;  // malformed offsets: leave untouched
  const int nchunks = (len + KC - 1) / KC;
  const long slot0 = (tok0 >> 6) + n;
  const size_t sbase = ((size_t)n * H + h) * DK * dv + col0;
  for (int i = tid; i < DK * KBV; i += 256) {
    const int d = i / KBV, j = i % KBV;
    Ms[d * SV + j] = p.init_state ? p.init_state[sbase + (size_t)d * dv + j] : 0.f;
  }
  auto colB = [&](const float *X, int n0) {
    return [=](int k0) {
      f32x8 f;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) f[ii] = X[(k0 + 8 * lg + ii) * SV + n0 + lm];
      return f;
    };
  };
  for (int c = 0; c < nchunks; ++c) {
    const size_t sh = (size_t)(slot0 + c) * H + h;
    const int nv = min(KC, len - c * KC);
    const size_t tbase = (size_t)tok0 + (size_t)c * KC;
    for (int i = tid; i < KC * KBV; i += 256) {
      const int r = i / KBV, j = i % KBV;
      Vs[r * SV + j] = r < nv ? to_f(((const E *)p.v)[((tbase + r) * H + h) * dv + col0 + j]) : 0.f;
    }
    if (tid < DK) gsh[tid] = p.gam[sh * DK + tid];
    __syncthreads();
    const float *at = p.at + sh * KC * DK, *qg = p.qg + sh * KC * DK;
    const float *tm = p.tm + sh * KC * KC, *aak = p.aak + sh * KC * KC, *pqb = p.pqb + sh * KC * KC,
                *pqk = p.pqk + sh * KC * KC;
    // R = (A e^{Gp}) M0 + A_ak V
    for (int t = wave; t < 8; t += 4) {
      const int m0 = 16 * (t >> 1), n0 = 16 * (t & 1);
      const f32x4 r1 = dprod<DK>([&](int k0) { return ld8(at + (m0 + lm) * DK + k0 + 8 * lg); }, colB(Ms, n0));
      const f32x4 r2 = dprod<KC>([&](int k0) { return ld8(aak + (m0 + lm) * KC + k0 + 8 * lg); }, colB(Vs, n0),
                                 0, m0 + 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) Rs[(m0 + 4 * lg + j) * SV + n0 + lm] = r1[j] + r2[j];
    }
    __syncthreads();
    // U = (I - A_ab)^-1 R
    for (int t = wave; t < 8; t += 4) {
      const int m0 = 16 * (t >> 1), n0 = 16 * (t & 1);
      const f32x4 u = dprod<KC>([&](int k0) { return ld8(tm + (m0 + lm) * KC + k0 + 8 * lg); }, colB(Rs, n0), 0,
                                m0 + 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) Us[(m0 + 4 * lg + j) * SV + n0 + lm] = u[j];
    }
    __syncthreads();
    // O = (Q e^G) M0 + P_qb U + P_qk V
    for (int t = wave; t < 8; t += 4) {
      const int m0 = 16 * (t >> 1), n0 = 16 * (t & 1);
      const f32x4 o1 = dprod<DK>([&](int k0) { return ld8(qg + (m0 + lm) * DK + k0 + 8 * lg); }, colB(Ms, n0));
      const f32x4 o2 = dprod<KC>([&](int k0) { return ld8(pqb + (m0 + lm) * KC + k0 + 8 * lg); }, colB(Us, n0), 0,
                                 m0 + 16);
      const f32x4 o3 = dprod<KC>([&](int k0) { return ld8(pqk + (m0 + lm) * KC + k0 + 8 * lg); }, colB(Vs, n0), 0,
                                 m0 + 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = m0 + 4 * lg + j;
        if (r < nv && p.o) ((E *)p.o)[((tbase + r) * H + h) * dv + col0 + n0 + lm] = to_e<E>(o1[j] + o2[j] + o3[j]);
      }
    }
    __syncthreads();  // every read of M0 is done
    // M = diag(e^{G_C}) M0 + (B e^{G_C - G})^T U + (K e^{G_C - G})^T V
    for (int t = wave; t < (DK / 16) * 2; t += 4) {
      const int m0 = 16 * (t >> 1), n0 = 16 * (t & 1);
      const f32x4 a1 =
          dprod<KC>([&](int k0) { return ld8(p.bhT + (sh * DK + m0 + lm) * KC + k0 + 8 * lg); }, colB(Us, n0));
      const f32x4 a2 =
          dprod<KC>([&](int k0) { return ld8(p.khT + (sh * DK + m0 + lm) * KC + k0 + 8 * lg); }, colB(Vs, n0));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = m0 + 4 * lg + j;
        Ms[d * SV + n0 + lm] = gsh[d] * Ms[d * SV + n0 + lm] + a1[j] + a2[j];
      }
    }
    __syncthreads();
  }
  if (p.final_state)
    for (int i = tid; i < DK * KBV; i += 256) {
      const int d = i / KBV, j = i % KBV;
      p.final_state[sbase + (size_t)d * dv + j] = Ms[d * SV + j];
    }
}

template <typename E, int DK>
hipError_t launch_dk(const DplrKeyParams &p, hipStream_t stream) {
  const unsigned items = (unsigned)(p.slots * p.H), serial = (unsigned)(p.N * p.H * (p.dv / KBV));
  if (serial == 0) return hipSuccess;
  if (items) hipLaunchKernelGGL((dplrk_prep_kernel<E, DK>), dim3(items), dim3(256), 0, stream, p);
  hipLaunchKernelGGL((dplrk_state_kernel<E, DK>), dim3(serial), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dplr_key(const DplrKeyParams &p, int dtype, int dk, hipStream_t stream) {
  if (dtype == 1) {
    if (dk == 128) return launch_dk<bf16, 128>(p, stream);
    if (dk == 64) return launch_dk<bf16, 64>(p, stream);
  } else {
    if (dk == 64) return launch_dk<float, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

// gdn_bwd_key.hip -- gradients of the chunked forward with one decay per key channel
// (the channel-wise gate of "Decoding Hybrid Linear Attention Architectures", sec. 3
// item 6, and with the additive write gated linear attention's gate, item 4).
//
// Reverse mode through the chunk equations of sec. 5 with the per-channel decay inside
// the contractions.  Per chunk, with G[r][c] the chunk-local prefix of log alpha of key
// channel c, Gamma[r][i][c] = e^{G[r][c] - G[i][c]} (i <= r),
//   A[r][i] = beta_r sum_c K[r][c] K[i][c] Gamma[r][i][c] (i < r),  T = (I + A)^-1,
//   P[r][i] = sum_c Q[r][c] K[i][c] Gamma[r][i][c] (i <= r),
//   Kt = K e^G, Qt = Q e^G, Kh = K e^{G_C - G}, gam = e^{G_C} (per channel),
//   X' = V - Kt M0, Delta = T diag(beta) X' (the additive write: Delta = V),
//   O = Qt M0 + P Delta,  M_C = diag(gam) M0 + Kh^T Delta.
// Given dO and dM (the gradient of M_C):
//   dDelta = P^T dO + Kh dM,  Y = T^T dDelta,  dV = diag(beta) Y,
//   dM0 = Qt^T dO + diag(gam) dM - Kt^T diag(beta) Y,
//   dP = incl(dO Delta^T), dT = dDelta (diag(beta) X')^T, dA = -strict(T^T dT T^T),
//   dQt = dO M0^T, dKt = -diag(beta) Y M0^T, dKh = Delta dM^T, dgam_c = <M0[c], dM[c]>;
// with Z = sum_i dA[r][i] K[i] Gamma[r][i], Zc = sum_r beta_r dA[r][i] K[r] Gamma[r][i],
// Pr = sum_i dP[r][i] K[i] Gamma[r][i], Pc = sum_r dP[r][i] Q[r] Gamma[r][i] (per channel):
//   dq = Pr + e^G dQt,  dk = beta Z + Zc + Pc + e^G dKt + e^{G_C - G} dKh,
//   dbeta = rowsum(Y * X') + rowsum(K * Z),
//   dG = beta K Z - K Zc + Q Pr - K Pc + Kt dKt + Qt dQt - Kh dKh,
//   dG_C = colsum(Kh * dKh) + gam dgam,  dlog alpha[t] = sum_{r >= t} dG[r] + dG_C.
// Every pairwise factor is split at row m = 16a + 7 of a 16-row block a: e^{G[r] - G[m]}
// on one side, e^{G[m] - G[i]} on the other, so that no factor exceeds the decay
// accumulated over eight tokens (the forward's reading of the decay range).
//
// Four launches, everything in between in the caller's workspace (fp32):
//  1. bwdk_prep_kernel, one workgroup per (chunk, head), fully parallel: Kt, Kh (row-major),
//     Kt^T, Qt^T, Kh^T (channel-major), gam, T and T^T (delta write), P^T;
//  2. bwdk_fwd_kernel, one workgroup per (sequence, head, 32 value columns), chunks in
//     order: the chunk-entering states;
//  3. bwdk_rev_kernel, one workgroup per (sequence, head, value block of 64, 32 or 16
//     columns, the widest that fills the chip), chunks in reverse: the chunk-end state
//     gradient dM and dDelta of every chunk, dV, and the initial-state gradient (also the
//     scalar gates' reverse pass, in its SCAL form);
//  4. bwdk_chunk_kernel, one workgroup per (chunk, head), fully parallel: everything
//     else (dq, dk, dbeta, dlog alpha).
// Products run on the bf16 matrix cores with every fp32 operand split into hi + lo bf16
// terms (three MFMAs per 32-deep step, about 2^-17 relative error per product); sums
// are in fp32 and in a fixed order (deterministic, no atomics).
#include "gdn_common.h"
#include "gdn_kernels.h"
#include "gdn_tile.h"
#include "gdn_bwd_slices.h"

namespace gdn {

namespace {

constexpr int KC = 64;        // chunk length
constexpr int KBV = 32;       // value columns per workgroup of the serial passes
constexpr int SV = KBV + 4;   // fp32 pitch of 32-column tiles (rows 16-byte aligned)
constexpr int SC = KC + 1;    // fp32 pitch of 64-column tiles

template <typename E> __device__ __forceinline__ f32x8 ldrow8(const E *p);
template <> __device__ __forceinline__ f32x8 ldrow8<float>(const float *p) { return ld8(p); }
template <> __device__ __forceinline__ f32x8 ldrow8<bf16>(const bf16 *p) { return widen8(ld8(p)); }

__device__ __forceinline__ f32x8 zero8() {
  f32x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = 0.f;
  return z;
}

// One 16x16 tile of C = A B over k in [0, K): fa(k0) and fb(k0) give this lane's fp32
// fragments (A: its row, B: its column, at k = k0 + 8 lg .. + 7).  32-deep steps
// outside [kbeg, kend) are skipped (known zeros; wave-uniform bounds).
template <int K, class FA, class FB>
__device__ __forceinline__ f32x4 kprod(FA fa, FB fb, int kbeg = 0, int kend = K) {
  f32x4 acc = zero4();
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32)
    if (k0 + 32 > kbeg && k0 < kend) acc = mm(split8(fa(k0)), split8(fb(k0)), acc);
  return acc;
}

__device__ __forceinline__ bool seq_extent_k(const BwdKeyParams &p, int n, long &tok0, int &len) {
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

// The chunk that owns a slot: its first token and valid rows (false: no chunk owns it)
__device__ __forceinline__ bool slot_chunk(const BwdKeyParams &p, long slot, long &tb, int &nv) {
  auto tok_start = [&](int sq) -> long { return p.cu_seqlens ? (long)p.cu_seqlens[sq] : (long)sq * p.T; };
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((tok_start(mid) >> 6) + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  long tok0;
  int len;
  if (!seq_extent_k(p, lo, tok0, len)) return false;
  const long c = slot - ((tok0 >> 6) + lo);
  if (c < 0 || 64 * c >= len) return false;
  tb = tok0 + 64 * c;
  nv = (int)min(64L, (long)len - 64 * c);
  return true;
}

constexpr int PNT = 512;  // threads of the preparation (eight waves)

// ---------------------------------------------------------------- 1. operands per chunk
template <typename E, int DK, bool ADD>
__global__ __launch_bounds__(PNT, 1) void bwdk_prep_kernel(BwdKeyParams p) {
  constexpr int SG = DK + 4;
  __shared__ __align__(16) float Ks[KC * SG];
  __shared__ __align__(16) float Qs[KC * SG];
  __shared__ __align__(16) float Gs[KC * SG];
  __shared__ float As[KC * SC];
  __shared__ float Ps[KC * SC];
  __shared__ float Ts[KC * SC];
  __shared__ float ys[3 * 16 * 17];
  __shared__ float bsh[KC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H;
  const long slot = blockIdx.x / H;
  const int h = blockIdx.x % H;
  long tb;
  int nv;
  if (!slot_chunk(p, slot, tb, nv)) return;
  const size_t sh = (size_t)slot * H + h;
  {  // 16-byte loads, all in flight before the LDS stores (rows past the end are zero)
    constexpr int VE = 16 / (int)sizeof(E), PR = DK / VE, NI = KC * PR / PNT;  // k, q
    constexpr int PG = DK / 4, NG = KC * PG / PNT;                             // log alpha
    typedef E EV __attribute__((ext_vector_type(16 / sizeof(E))));
    u32x4 xk[NI], xq[NI], y[NG];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int pc = tid + PNT * u, r = pc / PR, g = pc % PR;
      const size_t o = ((size_t)(tb + r) * H + h) * DK + g * VE;
      xk[u] = r < nv ? *(const u32x4 *)((const E *)p.k + o) : (u32x4){0u, 0u, 0u, 0u};
      xq[u] = r < nv ? *(const u32x4 *)((const E *)p.q + o) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int pc = tid + PNT * u, r = pc / PG, g = pc % PG;
      y[u] = r < nv ? *(const u32x4 *)(p.log_alpha + ((size_t)(tb + r) * H + h) * DK + 4 * g)
                    : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int pc = tid + PNT * u, r = pc / PR, g = pc % PR;
      const EV ek = __builtin_bit_cast(EV, xk[u]), eq = __builtin_bit_cast(EV, xq[u]);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        Ks[r * SG + g * VE + e] = to_f(ek[e]);
        Qs[r * SG + g * VE + e] = to_f(eq[e]);
      }
    }
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int pc = tid + PNT * u, r = pc / PG, g = pc % PG;
      *(u32x4 *)(Gs + r * SG + 4 * g) = y[u];
    }
  }
  if (tid < KC) bsh[tid] = (!ADD && tid < nv) ? p.beta[(size_t)(tb + tid) * H + h] : 0.f;
  for (int i = tid; i < KC * SC; i += PNT) As[i] = Ps[i] = 0.f;
  __syncthreads();
  {  // per-channel inclusive prefix: PNT / DK parts of rows per channel, then the offsets
    constexpr int NP = PNT / DK, RP = KC / NP;
    const int d = tid % DK, q = tid / DK;
    float g = 0.f;
    for (int r = q * RP; r < (q + 1) * RP; ++r) {
      g += Gs[r * SG + d];
      Gs[r * SG + d] = g;
    }
    Ts[q * DK + d] = g;  // part totals (Ts is free until T is formed)
    __syncthreads();
    float off = 0.f;
    for (int u = 0; u < q; ++u) off += Ts[u * DK + d];
    if (q > 0)
      for (int r = q * RP; r < (q + 1) * RP; ++r) Gs[r * SG + d] += off;
  }
  __syncthreads();
  // row-major Kt, Kh: 8 consecutive channels per thread (two 16-byte stores each)
  for (int i = 8 * tid; i < KC * DK; i += 8 * PNT) {
    const int r = i / DK, d = i % DK;
    const f32x8 gv = ld8(Gs + r * SG + d), gc = ld8(Gs + (KC - 1) * SG + d), kk = ld8(Ks + r * SG + d);
    f32x4 kt0, kt1, kh0, kh1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float g = gv[e], gC = gc[e], kv = kk[e];
      const float a = kv * __expf(g), b = kv * __expf(gC - g);
      if (e < 4) kt0[e] = a, kh0[e] = b;
      else kt1[e - 4] = a, kh1[e - 4] = b;
    }
    if (!ADD) {
      *(f32x4 *)(p.kt + sh * KC * DK + i) = kt0;
      *(f32x4 *)(p.kt + sh * KC * DK + i + 4) = kt1;
    }
    *(f32x4 *)(p.kh + sh * KC * DK + i) = kh0;
    *(f32x4 *)(p.kh + sh * KC * DK + i + 4) = kh1;
  }
  // channel-major Kt^T, Kh^T, Qt^T: 8 consecutive rows per thread
  for (int i = 8 * tid; i < DK * KC; i += 8 * PNT) {
    const int d = i / KC, r = i % KC;
    const float gC = Gs[(KC - 1) * SG + d];
    f32x4 a0, a1, b0, b1, c0, c1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float g = Gs[(r + e) * SG + d], kv = Ks[(r + e) * SG + d], eg = __expf(g);
      const float a = kv * eg, b = kv * __expf(gC - g), c = Qs[(r + e) * SG + d] * eg;
      if (e < 4) a0[e] = a, b0[e] = b, c0[e] = c;
      else a1[e - 4] = a, b1[e - 4] = b, c1[e - 4] = c;
    }
    if (!ADD) {
      *(f32x4 *)(p.ktT + sh * DK * KC + i) = a0;
      *(f32x4 *)(p.ktT + sh * DK * KC + i + 4) = a1;
    }
    if (!p.states_ready) {  // read only by the chunk-state kernel (bwdk_fwd_kernel)
      *(f32x4 *)(p.khT + sh * DK * KC + i) = b0;
      *(f32x4 *)(p.khT + sh * DK * KC + i + 4) = b1;
    }
    *(f32x4 *)(p.qtT + sh * DK * KC + i) = c0;
    *(f32x4 *)(p.qtT + sh * DK * KC + i + 4) = c1;
  }
  if (tid < DK) p.gam[sh * DK + tid] = __expf(Gs[(KC - 1) * SG + tid]);
  // the ten lower 16x16 tiles of P (and of A): row operand x[r] e^{G[r] - G[m]}, column
  // operand K[i] e^{G[m] - G[i]}, m = 16a + 7 of the row block a
  for (int t = wave; t < (ADD ? 10 : 20); t += PNT / 64) {
    const int tt = t % 10, a = tt < 1 ? 0 : tt < 3 ? 1 : tt < 6 ? 2 : 3;
    const int b = tt - a * (a + 1) / 2, m = 16 * a + 7;
    const float *X = t < 10 ? Qs : Ks;
    const f32x4 acc = kprod<DK>(
        [&](int k0) {  // row r of x e^{G[r] - G[m]} (16-byte reads)
          const int r = 16 * a + lm, c0 = k0 + 8 * lg;
          const f32x8 xv = ld8(X + r * SG + c0), gr = ld8(Gs + r * SG + c0), gm = ld8(Gs + m * SG + c0);
          f32x8 f;
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) f[ii] = xv[ii] * __expf(gr[ii] - gm[ii]);
          return f;
        },
        [&](int k0) {  // row i of K e^{G[m] - G[i]}
          const int i = 16 * b + lm, c0 = k0 + 8 * lg;
          const f32x8 kv = ld8(Ks + i * SG + c0), gi = ld8(Gs + i * SG + c0), gm = ld8(Gs + m * SG + c0);
          f32x8 f;
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) f[ii] = kv[ii] * __expf(gm[ii] - gi[ii]);
          return f;
        });
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * a + 4 * lg + j, i = 16 * b + lm;
      if (t < 10)
        Ps[r * SC + i] = i <= r ? acc[j] : 0.f;
      else
        As[r * SC + i] = i < r ? bsh[r] * acc[j] : 0.f;
    }
  }
  __syncthreads();
  if constexpr (!ADD) {
    tri_inv64<1>(As, SC, Ts, SC, ys);  // T = (I + A)^-1
    for (int i = tid; i < KC * KC; i += PNT) {
      const int r = i / KC, c = i % KC;
      p.tm[sh * KC * KC + i] = Ts[r * SC + c];
      p.tmT[sh * KC * KC + i] = Ts[c * SC + r];
    }
  }
  for (int i = tid; i < KC * KC; i += PNT) {
    const int r = i / KC, c = i % KC;
    p.pmT[sh * KC * KC + i] = Ps[c * SC + r];
  }
}

// ---------------------------------------------------------------- 2. chunk-entering states
template <typename E, int DK, bool ADD>
__global__ __launch_bounds__(256, 1) void bwdk_fwd_kernel(BwdKeyParams p) {
  __shared__ __align__(16) float Ms[DK * SV];
  __shared__ __align__(16) float Xs[KC * SV];
  __shared__ __align__(16) float Ds[KC * SV];
  __shared__ __align__(16) float Vs[KC * SV];
  __shared__ float bsh[KC], gsh[DK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H, dv = p.dv, nb = dv / KBV;
  int pair, jb;
  xcd_pair_block(blockIdx.x, p.N * p.H, nb, pair, jb);
  const int n = pair / H, h = pair % H, col0 = jb * KBV;
  long tok0;
  int len;
  if (!seq_extent_k(p, n, tok0, len)) return;
  const int nchunks = (len + KC - 1) / KC;
  const long slot0 = (tok0 >> 6) + n;
  const size_t sbase = ((size_t)n * H + h) * DK * dv + col0;
  for (int i = tid; i < DK * KBV; i += 256) {
    const int d = i / KBV, j = i % KBV;
    Ms[d * SV + j] = p.init_state ? p.init_state[sbase + (size_t)d * dv + j] : 0.f;
  }
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const size_t sh = (size_t)(slot0 + c) * H + h;
    const int nv = min(KC, len - c * KC);
    const size_t tbase = (size_t)tok0 + (size_t)c * KC;
    for (int i = tid; i < DK * KBV; i += 256) {
      const int d = i / KBV, j = i % KBV;
      p.states[(sh * DK + d) * dv + col0 + j] = Ms[d * SV + j];
    }
    for (int i = tid; i < KC * KBV; i += 256) {
      const int r = i / KBV, j = i % KBV;
      Vs[r * SV + j] = r < nv ? to_f(((const E *)p.v)[((tbase + r) * H + h) * dv + col0 + j]) : 0.f;
    }
    if (tid < KC) bsh[tid] = (!ADD && tid < nv) ? p.beta[(tbase + tid) * H + h] : 0.f;
    if (tid < DK) gsh[tid] = p.gam[sh * DK + tid];
    __syncthreads();
    if constexpr (!ADD) {
      // X' = V - Kt M  (eight 16x16 tiles, two per wave)
      for (int t = wave; t < 8; t += 4) {
        const int m0 = 16 * (t >> 1), n0 = 16 * (t & 1);
        const f32x4 acc = kprod<DK>([&](int k0) { return ld8(p.kt + (sh * KC + m0 + lm) * DK + k0 + 8 * lg); },
                                    [&](int k0) {
                                      f32x8 f;
#pragma unroll
                                      for (int ii = 0; ii < 8; ++ii) f[ii] = Ms[(k0 + 8 * lg + ii) * SV + n0 + lm];
                                      return f;
                                    });
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = m0 + 4 * lg + j;
          Xs[r * SV + n0 + lm] = Vs[r * SV + n0 + lm] - acc[j];
        }
      }
      __syncthreads();
      // Delta = T diag(beta) X'  (T lower triangular)
      for (int t = wave; t < 8; t += 4) {
        const int m0 = 16 * (t >> 1), n0 = 16 * (t & 1);
        const f32x4 acc = kprod<KC>([&](int k0) { return ld8(p.tm + (sh * KC + m0 + lm) * KC + k0 + 8 * lg); },
                                    [&](int k0) {
                                      f32x8 f;
#pragma unroll
                                      for (int ii = 0; ii < 8; ++ii) {
                                        const int k = k0 + 8 * lg + ii;
                                        f[ii] = bsh[k] * Xs[k * SV + n0 + lm];
                                      }
                                      return f;
                                    },
                                    0, m0 + 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) Ds[(m0 + 4 * lg + j) * SV + n0 + lm] = acc[j];
      }
      __syncthreads();
    }
    const float *D = ADD ? Vs : Ds;
    // M = diag(gam) M + Kh^T Delta
    for (int t = wave; t < (DK / 16) * 2; t += 4) {
      const int m0 = 16 * (t >> 1), n0 = 16 * (t & 1);
      const f32x4 acc = kprod<KC>([&](int k0) { return ld8(p.khT + (sh * DK + m0 + lm) * KC + k0 + 8 * lg); },
                                  [&](int k0) {
                                    f32x8 f;
#pragma unroll
                                    for (int ii = 0; ii < 8; ++ii) f[ii] = D[(k0 + 8 * lg + ii) * SV + n0 + lm];
                                    return f;
                                  });
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = m0 + 4 * lg + j;
        Ms[d * SV + n0 + lm] = gsh[d] * Ms[d * SV + n0 + lm] + acc[j];
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- 3. reverse state pass
// The gradient dM of the chunk-end state stays in the matrix-core accumulators of the
// four waves (d_k / 4 key rows each, VB value columns) for the whole sequence.  Per
// chunk (in reverse): dDelta = P^T dO + Kh dM, Y = T^T dDelta, dV = diag(beta) Y,
// dM <- diag(gam) dM + Qt^T dO - Kt^T diag(beta) Y.  The B operands (dM, dO, dDelta,
// -diag(beta) Y) are staged once per chunk in LDS, transposed and split into hi and lo
// bf16 halves, so that every fragment is two 16-byte reads; the A operands are read
// from the workspace one phase ahead of their products.
// SCAL (no gate or a scalar gate): K, Q^T and K^T are the inputs themselves (exact in
// bf16) and the row factors move to the other side: dDelta = P^T dO + diag(e^{g_C - g})
// (K dM), and e^g scales the staged B operands of the dM update (e^g dO, -e^g beta Y).
template <typename E, int DK, bool ADD, int VB, bool SCAL>
__global__ __launch_bounds__(256, 1) void bwdk_rev_kernel(BwdKeyParams p) {
  constexpr int PM = DK + 8, PV = KC + 8;  // bf16 pitches of the transposed operands
  constexpr int NCT = VB / 16, RB = DK / 64, SK = DK / 32;
  constexpr bool VX = std::is_same<E, bf16>::value;  // dO exact in bf16: no lo half
  typedef decltype(in8((const E *)nullptr)) KF;      // an input fragment (exact or split)
  __shared__ __align__(16) bf16 dGh[SCAL ? VB * PV : 8];  // e^g dO (SCAL)
  __shared__ __align__(16) bf16 dGl[SCAL ? VB * PV : 8];
  __shared__ float egs[KC], ets[KC];                      // e^g, e^{g_C - g} (SCAL)
  __shared__ __align__(16) bf16 dMh[VB * PM];
  __shared__ __align__(16) bf16 dMl[VB * PM];
  __shared__ __align__(16) bf16 dOh[VB * PV];
  __shared__ __align__(16) bf16 dOl[VB * PV];
  __shared__ __align__(16) bf16 dDh[VB * PV];
  __shared__ __align__(16) bf16 dDl[VB * PV];
  __shared__ __align__(16) bf16 bYh[VB * PV];
  __shared__ __align__(16) bf16 bYl[VB * PV];
  __shared__ float bsh[KC], gsh[DK];
  // Staged A operands (the additive write with the per-key-channel gate at 16 value
  // columns): the next chunk's P^T, Kh and Qt^T are fetched into registers at the top of
  // a chunk, a whole chunk ahead of their use, and written to LDS at the top of the next;
  // the fragments are then read from LDS.  Fetched one phase ahead instead (the other
  // path), their latency is exposed between the short products of a 16-column block
  // (3.37 -> 3.20 ms for the whole backward of B=2, T=16384, H=16, d=128).  With the
  // delta write the same staging measured no faster: there the 128 KB of operands per
  // chunk and workgroup bound the pass, not their latency.  Each operand is rows of
  // 16-byte pieces with piece c of row r stored at c ^ (r & 15), so a fragment read by
  // 16 lanes of 16 rows touches 16 bank groups.
  constexpr int O_TM = KC * KC / 4, O_KH = O_TM + (ADD ? 0 : KC * KC / 4), O_QT = O_KH + KC * DK / 4;
  constexpr int O_KT = O_QT + DK * KC / 4, N_PC = O_KT + (ADD ? 0 : DK * KC / 4);  // piece offsets
  constexpr int BASE_LDS = (2 * (SCAL ? VB * PV : 8) + 2 * VB * PM + 6 * VB * PV) * 2 + (3 * KC + DK) * 4 + 256;
  constexpr bool STG = !SCAL && ADD && VB == 16;
  static_assert(!STG || BASE_LDS + 16 * N_PC <= 160 * 1024, "LDS budget of the staged operands");
  static_assert(N_PC % 256 == 0 && O_KH % 256 == 0 && O_QT % 256 == 0 && O_KT % 256 == 0, "whole steps per operand");
  __shared__ __align__(16) float stg[STG ? 4 * N_PC : 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H, dv = p.dv, nb = dv / VB;
  int pair, jb;
  xcd_pair_block(blockIdx.x, p.N * p.H, nb, pair, jb);
  const int n = pair / H, h = pair % H, col0 = jb * VB;
  long tok0;
  int len;
  if (!seq_extent_k(p, n, tok0, len)) return;
  const int nchunks = (len + KC - 1) / KC;
  const long slot0 = (tok0 >> 6) + n;
  const size_t sbase = ((size_t)n * H + h) * DK * dv + col0;
  // dM: wave w holds key rows 16 (RB w + rb) + 4 lg + j, value columns 16 ct + lm
  f32x4 dM[RB][NCT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 16 * (RB * wave + rb) + 4 * lg + j;
        dM[rb][ct][j] = p.dfinal ? p.dfinal[sbase + (size_t)d * dv + 16 * ct + lm] : 0.f;
      }
  auto put_t = [&](bf16 *Xh, bf16 *Xl, int pitch, int r0, int ct, const f32x4 &v) {
    bf16x4 hv, lv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hv[j] = (bf16)v[j];
      lv[j] = (bf16)(v[j] - (float)hv[j]);
    }
    const int o = (16 * ct + lm) * pitch + r0 + 4 * lg;
    *(bf16x4 *)(Xh + o) = hv;
    *(bf16x4 *)(Xl + o) = lv;
  };
  auto bfrag = [&](const bf16 *Xh, const bf16 *Xl, int pitch, int ct, int k0) {
    const int o = (16 * ct + lm) * pitch + k0 + 8 * lg;
    return Split{ld8(Xh + o), ld8(Xl + o)};
  };
  auto ofrag = [&](int ct, int k0) {
    if constexpr (VX) {
      return ld8(dOh + (16 * ct + lm) * PV + k0 + 8 * lg);
    } else {
      return bfrag(dOh, dOl, PV, ct, k0);
    }
  };
  typedef decltype(ofrag(0, 0)) OF;
  const int r0 = 16 * wave + lm;  // this lane's A row of the 64-row products
  const int s0 = wave >> 1;       // P^T and T^T rows of block w vanish below column 16 w
  // A fragments (fp32 rows of the workspace, split when used; SCAL: the inputs), loaded
  // one phase ahead
  f32x8 f_pm[2], f_kh[SCAL ? 1 : SK], f_tm[2], f_qt[SCAL ? 1 : RB][2], f_kt[SCAL ? 1 : RB][2];
  KF k_r[SCAL ? SK : 1], q_t[SCAL ? RB : 1][2], k_t[SCAL ? RB : 1][2];
  auto load_1 = [&](int cc) {
    const size_t sh = (size_t)(slot0 + cc) * H + h;
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s >= s0) f_pm[s] = ld8(p.pmT + (sh * KC + r0) * KC + 32 * s + 8 * lg);
    if constexpr (SCAL) {  // K row r0 of the chunk (rows past the end re-read the last row:
                           // their e^{g_C - g} is 0)
      const int nvc = min(KC, len - cc * KC);
      const size_t t = (size_t)tok0 + (size_t)cc * KC + min(r0, nvc - 1);
#pragma unroll
      for (int s = 0; s < SK; ++s) k_r[s] = in8((const E *)p.k + (t * H + h) * DK + 32 * s + 8 * lg);
    } else {
#pragma unroll
      for (int s = 0; s < SK; ++s) f_kh[s] = ld8(p.kh + (sh * KC + r0) * DK + 32 * s + 8 * lg);
    }
  };
  auto load_2 = [&](size_t sh) {
    if constexpr (!ADD)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s >= s0) f_tm[s] = ld8(p.tmT + (sh * KC + r0) * KC + 32 * s + 8 * lg);
  };
  auto load_3 = [&](size_t sh) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int d = 16 * (RB * wave + rb) + lm;
        const size_t o = (sh * DK + d) * KC + 32 * s + 8 * lg;
        if constexpr (SCAL) {
          q_t[rb][s] = in8((const E *)p.qT + o);
          if (!ADD) k_t[rb][s] = in8((const E *)p.kT + o);
        } else {
          f_qt[rb][s] = ld8(p.qtT + o);
          if (!ADD) f_kt[rb][s] = ld8(p.ktT + o);
        }
      }
  };
  // the staged path: step u of a thread covers pieces 256 u .. 256 u + 255 of the
  // concatenated operands (each operand holds whole steps), the thread's piece is
  // 256 u + tid; kh rows hold DK / 4 pieces, the others 16
  constexpr int NPC = STG ? N_PC / 256 : 1;
  u32x4 pre[NPC];
  auto stg_fetch = [&](int cc) {
    const size_t sh = (size_t)(slot0 + cc) * H + h;
#pragma unroll
    for (int u = 0; u < NPC; ++u) {
      const int i = 256 * u, o = i < O_TM ? 0 : i < O_KH ? O_TM : i < O_QT ? O_KH : i < O_KT ? O_QT : O_KT;
      const float *src = i < O_TM   ? p.pmT + sh * KC * KC
                         : i < O_KH ? p.tmT + sh * KC * KC
                         : i < O_QT ? p.kh + sh * KC * DK
                         : i < O_KT ? p.qtT + sh * DK * KC
                                    : p.ktT + sh * DK * KC;
      pre[u] = *(const u32x4 *)(src + 4 * (i - o + tid));
    }
  };
  auto stg_put = [&]() {
#pragma unroll
    for (int u = 0; u < NPC; ++u) {
      const int i = 256 * u, o = i < O_TM ? 0 : i < O_KH ? O_TM : i < O_QT ? O_KH : i < O_KT ? O_QT : O_KT;
      const int rp = (i >= O_KH && i < O_QT) ? DK / 4 : 16, q = i - o + tid, r = q / rp, c = q % rp;
      *(u32x4 *)(stg + 4 * (o + r * rp + (c ^ (r & 15)))) = pre[u];
    }
  };
  // the 8 floats at columns col .. col + 7 (col a multiple of 8) of row r of the staged
  // operand at piece offset o with rp pieces per row
  auto sfr = [&](int o, int rp, int r, int col) {
    const int c = col >> 2, x = r & 15;
    const f32x4 a = *(const f32x4 *)(stg + 4 * (o + r * rp + (c ^ x)));
    const f32x4 b = *(const f32x4 *)(stg + 4 * (o + r * rp + ((c + 1) ^ x)));
    return (f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  };
  // the A fragments, from LDS (staged) or from the registers loaded a phase ahead
  auto A_pm = [&](int s) { return STG ? sfr(0, 16, r0, 32 * s + 8 * lg) : f_pm[s]; };
  auto A_kh = [&](int s) { return STG ? sfr(O_KH, DK / 4, r0, 32 * s + 8 * lg) : f_kh[SCAL ? 0 : s]; };
  auto A_tm = [&](int s) { return STG ? sfr(O_TM, 16, r0, 32 * s + 8 * lg) : f_tm[s]; };
  auto A_qt = [&](int rb, int s) {
    return STG ? sfr(O_QT, 16, 16 * (RB * wave + rb) + lm, 32 * s + 8 * lg) : f_qt[SCAL ? 0 : rb][s];
  };
  auto A_kt = [&](int rb, int s) {
    return STG ? sfr(O_KT, 16, 16 * (RB * wave + rb) + lm, 32 * s + 8 * lg) : f_kt[SCAL ? 0 : rb][s];
  };
  // dO of a chunk, beta and e^{g_C} (no branch around a load: rows past the end read
  // the last row and are zeroed when staged)
  // 16-byte pieces of a chunk's dO slice: NPR per row, PPT per thread (a thread-count
  // guard when there are fewer pieces than threads, uniform over each wave)
  constexpr int VE = 16 / (int)sizeof(E), NPR = VB / VE, NPO = KC * NPR, PPT = (NPO + 255) / 256;
  u32x4 oraw[PPT];
  float onext[SCAL ? PPT : 1];  // SCAL: e^g of each staged dO piece's row
  float bnext = 0.f, gnext = 0.f, enext = 0.f, tnext = 0.f;
  auto load_o = [&](int cc) {
    const int nvc = min(KC, len - cc * KC);
    const size_t tbc = (size_t)tok0 + (size_t)cc * KC, shc = (size_t)(slot0 + cc) * H + h;
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int pc = tid + 256 * u, r = min(pc / NPR, nvc - 1), g = pc % NPR;
      if (pc < NPO) {
        oraw[u] = *(const u32x4 *)((const E *)p.dout + ((tbc + r) * H + h) * dv + col0 + VE * g);
        if constexpr (SCAL) onext[u] = p.egr[shc * KC + r];
      }
    }
    if (!ADD) bnext = p.beta[(tbc + min(tid % KC, nvc - 1)) * H + h];
    gnext = p.gam[shc * DK + tid % DK];
    if constexpr (SCAL) {
      enext = p.egr[shc * KC + tid % KC];
      tnext = p.etr[shc * KC + tid % KC];
    }
  };
  if (nchunks > 0) {
    if constexpr (STG) stg_fetch(nchunks - 1);
    else load_1(nchunks - 1);
    load_o(nchunks - 1);
  }
  for (int c = nchunks - 1; c >= 0; --c) {
    const size_t sh = (size_t)(slot0 + c) * H + h;
    const int nv = min(KC, len - c * KC);
    const size_t tbase = (size_t)tok0 + (size_t)c * KC;
    if constexpr (STG) stg_put();  // every read of the last chunk's operands is done
    // the chunk-end gradient: to the workspace and, split, to LDS
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 16 * (RB * wave + rb) + 4 * lg + j;
          p.dmc[(sh * DK + d) * dv + col0 + 16 * ct + lm] = dM[rb][ct][j];
        }
        put_t(dMh, dMl, PM, 16 * (RB * wave + rb), ct, dM[rb][ct]);
      }
    {
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int pc = tid + 256 * u, r = pc / NPR, g = pc % NPR;
        if (pc >= NPO) break;
        const bool in = r < nv;
        typedef E EV __attribute__((ext_vector_type(16 / sizeof(E))));
        const EV ev = __builtin_bit_cast(EV, oraw[u]);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const float x = in ? to_f(ev[e]) : 0.f;
          const int col = VE * g + e;
          const bf16 hv = (bf16)x;
          dOh[col * PV + r] = hv;
          if constexpr (!VX) dOl[col * PV + r] = (bf16)(x - (float)hv);
          if constexpr (SCAL) {
            const float xg = x * onext[u];
            const bf16 hg = (bf16)xg;
            dGh[col * PV + r] = hg;
            dGl[col * PV + r] = (bf16)(xg - (float)hg);
          }
        }
      }
      if (tid < KC) bsh[tid] = (!ADD && tid < nv) ? bnext : 0.f;
      if (tid < DK) gsh[tid] = gnext;
      if (SCAL && tid < KC) {
        egs[tid] = enext;
        ets[tid] = tnext;
      }
    }
    if (STG && c > 0) {  // the next chunk's operands, in flight for a whole chunk
      stg_fetch(c - 1);
      load_o(c - 1);
    }
    __syncthreads();
    if constexpr (!STG) load_2(sh);
    OF fo[NCT][2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int s = 0; s < 2; ++s) fo[ct][s] = ofrag(ct, 32 * s);
    // dDelta = P^T dO + Kh dM
    {
      f32x4 D[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        D[ct] = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s)
          if (s >= s0) D[ct] = mm(split8(A_pm(s)), fo[ct][s], D[ct]);
        if constexpr (SCAL) {
          f32x4 D2 = zero4();
#pragma unroll
          for (int s = 0; s < SK; ++s) D2 = mm(k_r[s], bfrag(dMh, dMl, PM, ct, 32 * s), D2);
#pragma unroll
          for (int j = 0; j < 4; ++j) D[ct][j] += ets[16 * wave + 4 * lg + j] * D2[j];
        } else {
#pragma unroll
          for (int s = 0; s < SK; ++s) D[ct] = mm(split8(A_kh(s)), bfrag(dMh, dMl, PM, ct, 32 * s), D[ct]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * wave + 4 * lg + j;
          p.dd[(sh * KC + r) * dv + col0 + 16 * ct + lm] = D[ct][j];
          if (ADD && r < nv) ((E *)p.dv_out)[((tbase + r) * H + h) * dv + col0 + 16 * ct + lm] = to_e<E>(D[ct][j]);
        }
        if constexpr (!ADD) put_t(dDh, dDl, PV, 16 * wave, ct, D[ct]);
      }
    }
    __syncthreads();
    if constexpr (!STG) load_3(sh);
    if constexpr (!ADD) {
      // Y = T^T dDelta;  dV = diag(beta) Y;  -diag(beta) Y into LDS for the dM update
      f32x4 Y[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        Y[ct] = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s)
          if (s >= s0) Y[ct] = mm(split8(A_tm(s)), bfrag(dDh, dDl, PV, ct, 32 * s), Y[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 nb4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * wave + 4 * lg + j;
          const float by = bsh[r] * Y[ct][j];
          nb4[j] = SCAL ? -by * egs[r] : -by;
          if (r < nv) ((E *)p.dv_out)[((tbase + r) * H + h) * dv + col0 + 16 * ct + lm] = to_e<E>(by);
        }
        put_t(bYh, bYl, PV, 16 * wave, ct, nb4);
      }
      __syncthreads();
    }
    if (!STG && c > 0) {
      load_1(c - 1);
      load_o(c - 1);
    }
    // dM <- diag(gam) dM + Qt^T dO - Kt^T diag(beta) Y
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int d0 = 16 * (RB * wave + rb);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dM[rb][ct][j] *= gsh[d0 + 4 * lg + j];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if constexpr (SCAL) {
            dM[rb][ct] = mm(q_t[rb][s], bfrag(dGh, dGl, PV, ct, 32 * s), dM[rb][ct]);
            if constexpr (!ADD) dM[rb][ct] = mm(k_t[rb][s], bfrag(bYh, bYl, PV, ct, 32 * s), dM[rb][ct]);
          } else {
            dM[rb][ct] = mm(split8(A_qt(rb, s)), fo[ct][s], dM[rb][ct]);
            if constexpr (!ADD) dM[rb][ct] = mm(split8(A_kt(rb, s)), bfrag(bYh, bYl, PV, ct, 32 * s), dM[rb][ct]);
          }
        }
      }
    }
    __syncthreads();  // every read of this chunk's dO, dM and -diag(beta) Y is done
  }
  if (p.dinit)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 16 * (RB * wave + rb) + 4 * lg + j;
          p.dinit[sbase + (size_t)d * dv + 16 * ct + lm] = dM[rb][ct][j];
        }
}

// ---------------------------------------------------------------- 4. per-chunk gradients
template <typename E, int DK, bool ADD>
__global__ __launch_bounds__(512, 1) void bwdk_chunk_kernel(BwdKeyParams p) {
  constexpr int SG = DK + 4;
  constexpr int NCT = DK / 32;  // 16-column channel tiles per wave
  // One region, two lives: the value slices (slice_sums); then G (then dG), T, dT (then
  // dA), dP and a last part holding W, then K and Q of the chunk (the I/O dtype, rows of
  // DK + 2 elements, so that a column read is free of bank conflicts)
  constexpr int PK = DK + 2;
  constexpr int LAST = 2 * KC * PK * (int)sizeof(E) > KC * SC * 4 ? 2 * KC * PK * (int)sizeof(E) : KC * SC * 4;
  constexpr int B_BYTES = (KC * SG + 3 * KC * SC) * 4 + LAST, A_BYTES = SliceLds<E, DK, ADD>::BYTES;
  __shared__ __align__(16) char U[A_BYTES > B_BYTES ? A_BYTES : B_BYTES];
  __shared__ float bsh[KC], gcl[DK], rb[2][KC], gcp[4][DK], dbys[KC], dbp[2][KC], dgmc[DK];
  float *const Gs = (float *)U, *const Tl = Gs + KC * SG, *const dTl = Tl + KC * SC, *const dPl = dTl + KC * SC;
  float *const Wl = dPl + KC * SC;
  E *const Kst = (E *)Wl, *const Qst = (E *)Wl + KC * PK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H, dv = p.dv;
  const long slot = blockIdx.x / H;
  const int h = blockIdx.x % H;
  long tb;
  int nv;
  if (!slot_chunk(p, slot, tb, nv)) return;
  const size_t sh = (size_t)slot * H + h;
  const E *kin = (const E *)p.k, *qin = (const E *)p.q;
  // K and Q from the last part (rows past the end zero)
  auto K_ = [&](int r, int c) { return to_f(Kst[r * PK + c]); };
  auto Q_ = [&](int r, int c) { return to_f(Qst[r * PK + c]); };
  if (tid < KC) bsh[tid] = (!ADD && tid < nv) ? p.beta[(size_t)(tb + tid) * H + h] : 0.f;
  __syncthreads();

  // ---- the sums over the value columns (dP, dT, dQt, dKt, dKh, the dbeta rows and
  // <M0[c], dM[c]>)
  SliceSums<DK> S;
  {
    SliceIn in;
    in.st = p.states + sh * DK * dv;
    in.dmc = p.dmc + sh * DK * dv;
    in.dd = p.dd + sh * KC * dv;
    in.tm = p.tm + sh * KC * KC;
    in.tmT = p.tmT + sh * KC * KC;
    in.kt = p.kt + sh * KC * DK;
    in.v = p.v;
    in.dout = p.dout;
    in.tb = (size_t)tb;
    in.nv = nv;
    in.H = H;
    in.h = h;
    in.dv = dv;
    slice_sums<E, DK, ADD, true>(in, U, (const E *)nullptr, nullptr, bsh, S);
  }
  const int wa = wave & 3, wc = wave >> 2;
  f32x4 *const aP = S.aP, *const aT = S.aT, *const aQ = S.aQ, *const aK = S.aK, *const aH = S.aH;
  // G per channel and T into the region
  for (int i = tid; i < KC * DK; i += 512) {
    const int r = i / DK, d = i % DK;
    Gs[r * SG + d] = r < nv ? p.log_alpha[((size_t)(tb + r) * H + h) * DK + d] : 0.f;
  }
  if (!ADD)
    for (int i = tid; i < KC * KC; i += 512) Tl[(i / KC) * SC + i % KC] = p.tm[sh * KC * KC + i];
  if constexpr (!ADD) {  // dbeta rows: the lanes' columns, then the two column blocks
    f32x4 dby = S.dby;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) dby[j] += __shfl_xor(dby[j], off);
    if (lm == 0)
#pragma unroll
      for (int j = 0; j < 4; ++j) dbp[wave & 1][16 * (wave >> 1) + 4 * lg + j] = dby[j];
  }
#pragma unroll
  for (int q = 0; q < SliceSums<DK>::NM; ++q) {  // <M0[d], dM[d]>: eight threads per key row
    float x = S.dgm[q];
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    if ((tid & 7) == 0) dgmc[(tid + 512 * q) >> 3] = x;
  }
  __syncthreads();
  if (tid < DK) {
    float g = 0.f;
    for (int r = 0; r < KC; ++r) {
      g += Gs[r * SG + tid];
      Gs[r * SG + tid] = g;
    }
    gcl[tid] = g;
  }
  // ---- dP (inclusive lower) and dT into LDS; dA = -strict(T^T dT T^T)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = wave + 8 * u, m0 = 16 * (t >> 2), n0 = 16 * (t & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = m0 + 4 * lg + j, i = n0 + lm;
      dPl[r * SC + i] = i <= r ? aP[u][j] : 0.f;
      if (!ADD) dTl[r * SC + i] = aT[u][j];
    }
  }
  if (!ADD && tid < KC) dbys[tid] = dbp[0][tid] + dbp[1][tid];
  __syncthreads();
  if constexpr (!ADD) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // W = dT T^T
      const int t = wave + 8 * u, m0 = 16 * (t >> 2), n0 = 16 * (t & 3);
      const f32x4 w = kprod<KC>(
          [&](int k0) {
            f32x8 f;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) f[ii] = dTl[(m0 + lm) * SC + k0 + 8 * lg + ii];
            return f;
          },
          [&](int k0) {
            f32x8 f;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) f[ii] = Tl[(n0 + lm) * SC + k0 + 8 * lg + ii];
            return f;
          },
          0, n0 + 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) Wl[(m0 + 4 * lg + j) * SC + n0 + lm] = w[j];
    }
    __syncthreads();
    f32x4 da[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // dA = -T^T W
      const int t = wave + 8 * u, m0 = 16 * (t >> 2), n0 = 16 * (t & 3);
      da[u] = kprod<KC>(
          [&](int k0) {
            f32x8 f;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) f[ii] = Tl[(k0 + 8 * lg + ii) * SC + m0 + lm];
            return f;
          },
          [&](int k0) {
            f32x8 f;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) f[ii] = Wl[(k0 + 8 * lg + ii) * SC + n0 + lm];
            return f;
          },
          m0, KC);
    }
    __syncthreads();  // every read of dT is done
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = wave + 8 * u, m0 = 16 * (t >> 2), n0 = 16 * (t & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = m0 + 4 * lg + j, i = n0 + lm;
        dTl[r * SC + i] = i < r ? -da[u][j] : 0.f;
      }
    }
    __syncthreads();
  }

  {  // K and Q of the chunk into the staging region (W and the slices are dead)
    constexpr int VE = 16 / (int)sizeof(E), PR = DK / VE, NI = (KC * PR + 511) / 512;
    typedef E EV __attribute__((ext_vector_type(16 / sizeof(E))));
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int pc = tid + 512 * u, r = pc / PR, g = pc % PR;
      if (pc >= KC * PR) break;
      const size_t o = ((size_t)(tb + r) * H + h) * DK + g * VE;
      const u32x4 xk = r < nv ? *(const u32x4 *)(kin + o) : (u32x4){0u, 0u, 0u, 0u};
      const u32x4 xq = r < nv ? *(const u32x4 *)(qin + o) : (u32x4){0u, 0u, 0u, 0u};
      const EV ek = __builtin_bit_cast(EV, xk), eq = __builtin_bit_cast(EV, xq);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        Kst[r * PK + g * VE + e] = ek[e];
        Qst[r * PK + g * VE + e] = eq[e];
      }
    }
    __syncthreads();
  }
  // ---- per-channel terms, tiles (row block wa, channel blocks wc + 2u)
  const int a = wa, mref = 16 * a + 7;
  float rbs[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4 dgt[NCT];
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int c = 16 * (wc + 2 * u) + lm;
    const float gm = Gs[mref * SG + c];
    // rows i of the column operand K[i] e^{G[m] - G[i]}, i < 16 (a + 1)
    auto kcol = [&](int k0) {
      f32x8 f;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const int i = k0 + 8 * lg + ii;
        f[ii] = i < 16 * (a + 1) ? K_(i, c) * __expf(gm - Gs[i * SG + c]) : 0.f;
      }
      return f;
    };
    // Pr and Z share their column operand, Pc and Zc their row factors: each is formed
    // once per 32-deep step
    f32x4 Pr = zero4(), Z = zero4(), Pc = zero4(), Zc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < KC; k0 += 32) {
      if (k0 < 16 * (a + 1)) {  // columns i < 16 (a + 1)
        const Split bk = split8(kcol(k0));
        f32x8 fp;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) fp[ii] = dPl[(16 * a + lm) * SC + k0 + 8 * lg + ii];
        Pr = mm(split8(fp), bk, Pr);
        if constexpr (!ADD) {
          f32x8 ft;
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) ft[ii] = dTl[(16 * a + lm) * SC + k0 + 8 * lg + ii];
          Z = mm(split8(ft), bk, Z);
        }
      }
      if (k0 + 32 > 16 * a) {  // rows r >= 16 a
        f32x8 fq, fk, fp;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int r = k0 + 8 * lg + ii;
          const float e = r >= 16 * a ? __expf(Gs[r * SG + c] - gm) : 0.f;
          fq[ii] = Q_(r, c) * e;
          fk[ii] = K_(r, c) * e;
          fp[ii] = dPl[r * SC + 16 * a + lm];
        }
        Pc = mm(split8(fp), split8(fq), Pc);
        if constexpr (!ADD) {
          f32x8 ft;
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) {
            const int r = k0 + 8 * lg + ii;
            ft[ii] = bsh[r] * dTl[r * SC + 16 * a + lm];
          }
          Zc = mm(split8(ft), split8(fk), Zc);
        }
      }
    }
    float gcs = 0.f;
    const float gC = gcl[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * a + 4 * lg + j;
      const float g = Gs[r * SG + c];
      const float eg = __expf(g), et = __expf(gC - g), fr = __expf(g - gm), fc = __expf(gm - g);
      const float kv = K_(r, c), qv = Q_(r, c), br = bsh[r];
      const float z = Z[j] * fr, pr = Pr[j] * fr, zc = Zc[j] * fc, pc = Pc[j] * fc;
      const float dq = pr + eg * aQ[u][j];
      const float dk = br * z + zc + pc + eg * aK[u][j] + et * aH[u][j];
      dgt[u][j] = br * kv * z - kv * zc + qv * pr - kv * pc + kv * eg * aK[u][j] + qv * eg * aQ[u][j] -
                  kv * et * aH[u][j];
      rbs[j] += kv * z;
      gcs += kv * et * aH[u][j];
      if (r < nv) {
        const size_t o = ((size_t)(tb + r) * H + h) * DK + c;
        ((E *)p.dq)[o] = to_e<E>(dq);
        ((E *)p.dk)[o] = to_e<E>(dk);
      }
    }
    gcs += __shfl_xor(gcs, 16);
    gcs += __shfl_xor(gcs, 32);
    if (lg == 0) gcp[a][c] = gcs;
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1)
#pragma unroll
    for (int j = 0; j < 4; ++j) rbs[j] += __shfl_xor(rbs[j], off);
  __syncthreads();  // every read of G is done
#pragma unroll
  for (int u = 0; u < NCT; ++u) {
    const int c = 16 * (wc + 2 * u) + lm;
#pragma unroll
    for (int j = 0; j < 4; ++j) Gs[(16 * a + 4 * lg + j) * SG + c] = dgt[u][j];
  }
  if (lm == 0)
#pragma unroll
    for (int j = 0; j < 4; ++j) rb[wc][16 * a + 4 * lg + j] = rbs[j];
  __syncthreads();
  if (tid < DK) {  // d log alpha: reverse prefix of dG plus dG_C, per channel
    const int c = tid;
    const float dgc = ((gcp[0][c] + gcp[1][c]) + (gcp[2][c] + gcp[3][c])) + __expf(gcl[c]) * dgmc[c];
    float acc = 0.f;
    for (int r = KC - 1; r >= 0; --r) {
      acc += Gs[r * SG + c];
      if (r < nv) p.dlog_alpha[((size_t)(tb + r) * H + h) * DK + c] = acc + dgc;
    }
  }
  if (!ADD && tid < nv) p.dbeta[(size_t)(tb + tid) * H + h] = dbys[tid] + (rb[0][tid] + rb[1][tid]);
}

// The reverse pass takes the widest value block (64, 32 or 16 columns) that still gives
// one workgroup per compute unit: a wider block reads the A operands once for more
// columns, a narrower one puts more of the chip to work on few long sequences
template <typename E, int DK, bool ADD, bool SCAL = false>
void launch_rev(const BwdKeyParams &p, hipStream_t stream) {
  const long pairs = (long)p.N * p.H;
  if (pairs * (p.dv / 64) >= 256)
    hipLaunchKernelGGL((bwdk_rev_kernel<E, DK, ADD, 64, SCAL>), dim3((unsigned)(pairs * (p.dv / 64))), dim3(256), 0,
                       stream, p);
  else if (pairs * (p.dv / 32) >= 256)
    hipLaunchKernelGGL((bwdk_rev_kernel<E, DK, ADD, 32, SCAL>), dim3((unsigned)(pairs * (p.dv / 32))), dim3(256), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((bwdk_rev_kernel<E, DK, ADD, 16, SCAL>), dim3((unsigned)(pairs * (p.dv / 16))), dim3(256), 0,
                       stream, p);
}

template <typename E, int DK>
hipError_t launch_k(const BwdKeyParams &p, bool add, hipStream_t stream) {
  const unsigned items = (unsigned)(p.slots * p.H), serial = (unsigned)(p.N * p.H * (p.dv / KBV));
  if (items == 0 || serial == 0) return hipSuccess;
  if (add) {
    hipLaunchKernelGGL((bwdk_prep_kernel<E, DK, true>), dim3(items), dim3(PNT), 0, stream, p);
    if (!p.states_ready)
      hipLaunchKernelGGL((bwdk_fwd_kernel<E, DK, true>), dim3(serial), dim3(256), 0, stream, p);
    launch_rev<E, DK, true>(p, stream);
    hipLaunchKernelGGL((bwdk_chunk_kernel<E, DK, true>), dim3(items), dim3(512), 0, stream, p);
  } else {
    hipLaunchKernelGGL((bwdk_prep_kernel<E, DK, false>), dim3(items), dim3(PNT), 0, stream, p);
    if (!p.states_ready)
      hipLaunchKernelGGL((bwdk_fwd_kernel<E, DK, false>), dim3(serial), dim3(256), 0, stream, p);
    launch_rev<E, DK, false>(p, stream);
    hipLaunchKernelGGL((bwdk_chunk_kernel<E, DK, false>), dim3(items), dim3(512), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwdk_rev(const BwdKeyParams &p, int dtype, int dk, bool add, hipStream_t stream) {
  // (the scalar-gate path's reverse pass: the SCAL operands, bf16 with d_k 64 or 128 or
  // fp32 with d_k 64)
  if (p.N * p.H * (p.dv / KBV) == 0) return hipSuccess;
  if (dtype == 1 && dk == 128) add ? launch_rev<bf16, 128, true, true>(p, stream) : launch_rev<bf16, 128, false, true>(p, stream);
  else if (dtype == 1 && dk == 64) add ? launch_rev<bf16, 64, true, true>(p, stream) : launch_rev<bf16, 64, false, true>(p, stream);
  else if (dtype == 0 && dk == 64) add ? launch_rev<float, 64, true, true>(p, stream) : launch_rev<float, 64, false, true>(p, stream);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_key(const BwdKeyParams &p, int dtype, int dk, bool add, hipStream_t stream) {
  if (dtype == 1) {
    if (dk == 128) return launch_k<bf16, 128>(p, add, stream);
    if (dk == 64) return launch_k<bf16, 64>(p, add, stream);
  } else {
    if (dk == 128) return launch_k<float, 128>(p, add, stream);
    if (dk == 64) return launch_k<float, 64>(p, add, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

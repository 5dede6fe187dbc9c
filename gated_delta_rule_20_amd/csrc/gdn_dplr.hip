// gdn_dplr.hip -- chunked forward of the diagonal-plus-low-rank transition.
//
// "Decoding Hybrid Linear Attention Architectures", sec. 3 item 5: the state transition
// Diag(alpha_t) + a_t b_t^T with an additive write, S_t = S_{t-1}(Diag(alpha_t) + a_t b_t^T)
// + v_t k_t^T, here with one decay per (token, head) or none.  In storage orientation
// (M = S^T) one token is u = a^T M_{t-1}, M_t = alpha M_{t-1} + b u + k v^T, o = M_t^T q.
// Within a chunk entering with M0 (G the inclusive prefix of log alpha, G_{-1} = 0) the
// rows u_j solve a unit lower-triangular system, the UT form of the delta rule:
//   (I - A_ab) U = diag(e^{G_{j-1}}) A M0 + A_ak V,
//   A_ab[j,i] = (a_j . b_i) e^{G_{j-1} - G_i},  A_ak[j,i] = (a_j . k_i) e^{G_{j-1} - G_i}  (i < j)
//   O   = diag(e^G) Q M0 + P_qb U + P_qk V,
//   P_qb[r,j] = (q_r . b_j) e^{G_r - G_j},  P_qk[r,j] = (q_r . k_j) e^{G_r - G_j}  (j <= r)
//   M_C = e^{G_C} M0 + (diag(e^{G_C - G}) B)^T U + (diag(e^{G_C - G}) K)^T V.
//
// One workgroup (4 waves; 8 for bf16) per (sequence, head, 32 value columns) walks its sequence;
// the state block (d_k x 32, fp32) stays in LDS.  T = (I - A_ab)^-1 by forward
// substitution of the 16x16 diagonal blocks and block substitution of the rest.  Two
// kernels: fp32 I/O (d_k = 64) on the fp32 matrix cores with operands gathered from
// LDS (dplr_fwd_kernel), and bf16 I/O on the bf16 matrix cores (dplr_bf16_kernel).
#include <type_traits>

#include "gdn_common.h"
#include "gdn_kernels.h"
#include "gdn_tile.h"

namespace gdn {

namespace {

constexpr int DC = 64;    // chunk length
constexpr int DNT = 256;  // threads per workgroup (fp32 kernel)
constexpr int DNB = 512;  // threads per workgroup (bf16 kernel): two waves per SIMD
constexpr int NWB = DNB / 64;
constexpr int DVB = 32;   // value columns per workgroup
constexpr int DSV = DVB + 1, DST = DC + 1;

template <typename E, int DK, int GATE>
__global__ __launch_bounds__(DNT, 1) void dplr_fwd_kernel(DplrParams p) {
  constexpr int SKE = DK + 8;
  constexpr int VE = 16 / (int)sizeof(E);
  constexpr int RK = DC * (DK / VE) / DNT;  // 16-byte pieces of a [64][DK] operand per thread
  __shared__ __align__(16) E Ql[DC * SKE];
  __shared__ __align__(16) E Kl[DC * SKE];
  __shared__ __align__(16) E Al[DC * SKE];
  __shared__ __align__(16) E Bl[DC * SKE];
  __shared__ float X1[DC * DST], Tb[DC * DST];
  __shared__ float Ml[DK * DSV], Vb[DC * DSV], Rb[DC * DSV], Ub[DC * DSV];
  __shared__ float gs[DC], eg[DC], egp[DC], et[DC], misc[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H, dv = p.dv, nb = dv / DVB;
  int pair, jb;
  xcd_pair_block(blockIdx.x, p.N * p.H, nb, pair, jb);
  const int n = pair / H, h = pair % H, col0 = jb * DVB;
  long tok0;
  int len;
  if (p.cu_seqlens) {
    const int s0 = p.cu_seqlens[n], s1 = p.cu_seqlens[n + 1];
    if (s0 < 0 || s1 < s0 || s1 > p.T) return;  // malformed offsets: leave untouched
    tok0 = s0;
    len = s1 - s0;
  } else {
    tok0 = (long)n * p.T;
    len = p.T;
  }
  const int nchunks = (len + DC - 1) / DC;
  const size_t sstate = ((size_t)n * H + h) * DK * dv + col0;
  auto Q_ = [&](int r, int d) { return to_f(Ql[r * SKE + d]); };
  auto K_ = [&](int r, int d) { return to_f(Kl[r * SKE + d]); };
  auto A_ = [&](int r, int d) { return to_f(Al[r * SKE + d]); };
  auto B_ = [&](int r, int d) { return to_f(Bl[r * SKE + d]); };

  for (int i = tid; i < DK * DVB; i += DNT) {
    const int d = i / DVB, j = i % DVB;
    Ml[d * DSV + j] = p.init_state ? p.init_state[sstate + (size_t)d * dv + j] : 0.f;
  }
  for (int i = tid; i < DC * DST; i += DNT) Tb[i] = X1[i] = 0.f;  // upper blocks stay zero

  for (int c = 0; c < nchunks; ++c) {
    const int nv = min(DC, len - c * DC);
    const size_t tb = (size_t)tok0 + (size_t)c * DC;
    __syncthreads();  // the previous chunk is done with every buffer
    // ---- inputs (rows past the sequence end are zero): 16-byte loads
#pragma unroll
    for (int u = 0; u < RK; ++u) {
      const int pc = tid + DNT * u, r = pc / (DK / VE), g = pc % (DK / VE);
      u32x4 qv = {0u, 0u, 0u, 0u}, kv = qv, av = qv, bv = qv;
      if (r < nv) {
        const size_t o = ((tb + r) * H + h) * DK + g * VE;
        qv = *(const u32x4 *)((const E *)p.q + o);
        kv = *(const u32x4 *)((const E *)p.k + o);
        av = *(const u32x4 *)((const E *)p.a + o);
        bv = *(const u32x4 *)((const E *)p.b + o);
      }
      *(u32x4 *)(Ql + r * SKE + g * VE) = qv;
      *(u32x4 *)(Kl + r * SKE + g * VE) = kv;
      *(u32x4 *)(Al + r * SKE + g * VE) = av;
      *(u32x4 *)(Bl + r * SKE + g * VE) = bv;
    }
    for (int i = tid; i < DC * DVB; i += DNT) {
      const int r = i / DVB, j = i % DVB;
      Vb[r * DSV + j] = r < nv ? to_f(((const E *)p.v)[((tb + r) * H + h) * dv + col0 + j]) : 0.f;
    }
    if (tid < DC) gs[tid] = (GATE == GATE_HEAD && tid < nv) ? p.log_alpha[(tb + tid) * p.la_stride + h] : 0.f;
    __syncthreads();
    if (wave == 0) {  // decay prefix: e^G, e^{G_{j-1}}, e^{G_C - G}, e^{G_C}
      float g = gs[lane];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(g, off);
        if (lane >= off) g += y;
      }
      const float gC = __shfl(g, 63), gp = __shfl_up(g, 1);
      gs[lane] = g;
      eg[lane] = __expf(g);
      egp[lane] = lane == 0 ? 1.f : __expf(gp);
      et[lane] = __expf(gC - g);
      if (lane == 0) misc[0] = __expf(gC);
    }
    __syncthreads();
    auto e_out = [&](int r, int j) {  // e^{G_r - G_j}, j <= r
      return j <= r ? (GATE == GATE_HEAD ? __expf(gs[r] - gs[j]) : 1.f) : 0.f;
    };
    auto e_in = [&](int j, int i) {  // e^{G_{j-1} - G_i}, i < j
      return i < j ? (GATE == GATE_HEAD ? __expf((j > 0 ? gs[j - 1] : 0.f) - gs[i]) : 1.f) : 0.f;
    };
    // ---- P_qk into X1; O = e^G Q M0 (two tiles of the 64 x 32 output per wave, kept in registers)
    f32x4 Oacc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int t = wave + 4 * q, m0 = (t >> 1) * 16, n0 = (t & 1) * 16;
      const f32x4 v = tile<DK>(m0, n0, lg, lm, Q_, [&](int d, int j) { return Ml[d * DSV + j]; });
#pragma unroll
      for (int u = 0; u < 4; ++u) Oacc[q][u] = eg[m0 + 4 * lg + u] * v[u];
    }
    // X1 = lower(rowf colf^T * fac): the 10 lower 16x16 tiles, 3/3/2/2 per wave (the
    // upper ones were zeroed once and are never written)
    auto gram = [&](auto rowf, auto colf, auto fac) {
      for (int t = wave; t < 10; t += 4) {
        const int mb = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
        const int m0 = 16 * mb, n0 = 16 * (t - mb * (mb + 1) / 2);
        const f32x4 v = tile<DK>(m0, n0, lg, lm, rowf, [&](int d, int i) { return colf(i, d); });
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = m0 + 4 * lg + u, i = n0 + lm;
          X1[r * DST + i] = v[u] * fac(r, i);
        }
      }
    };
    gram(Q_, K_, e_out);
    __syncthreads();
    // ---- O += P_qk V
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int t = wave + 4 * q, m0 = (t >> 1) * 16, n0 = (t & 1) * 16;
      Oacc[q] += tile<DC>(m0, n0, lg, lm, [&](int r, int i) { return X1[r * DST + i]; },
                          [&](int i, int j) { return Vb[i * DSV + j]; });
    }
    __syncthreads();
    // ---- A_ab into X1, then T = (I - A_ab)^-1 into Tb
    gram(A_, B_, e_in);
    __syncthreads();
    if (wave == 0) {  // diagonal blocks: lane (lg, lm) solves column lm of block lg
      const int o = 16 * lg;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = r == lm ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) acc += X1[(o + r) * DST + o + i] * x[i];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Tb[(o + r) * DST + o + lm] = x[r];
    }
    __syncthreads();
    if (wave < 3) {  // off-diagonal blocks, block column b = wave: T[a][b] = T[a][a] sum_k A[a][k] T[k][b]
      const int b = wave;
      float *ys = Rb + wave * (16 * 17);  // scratch (R is formed afterwards)
      for (int a = b + 1; a < 4; ++a) {
        const f32x4 y = tile<DC>(16 * a, 16 * b, lg, lm,
                                 [&](int r, int k) { return (k >= 16 * b && k < 16 * a) ? X1[r * DST + k] : 0.f; },
                                 [&](int k, int col) { return Tb[k * DST + col]; });
#pragma unroll
        for (int u = 0; u < 4; ++u) ys[(4 * lg + u) * 17 + lm] = y[u];
        const f32x4 z = tile<32>(16 * a, 16 * b, lg, lm,
                                 [&](int r, int k) { return k < 16 ? Tb[r * DST + 16 * a + k] : 0.f; },
                                 [&](int k, int col) { return k < 16 ? ys[k * 17 + col - 16 * b] : 0.f; });
#pragma unroll
        for (int u = 0; u < 4; ++u) Tb[(16 * a + 4 * lg + u) * DST + 16 * b + lm] = z[u];
      }
    }
    __syncthreads();
    // ---- A_ak into X1; R = diag(e^{G_{j-1}}) A M0 + A_ak V into Rb
    gram(A_, K_, e_in);
    __syncthreads();
    mfma_mm<DC, DVB, DK, 4>(wave, lane, A_, [&](int d, int j) { return Ml[d * DSV + j]; }, [&](int r, int j, f32x4 v) {
      const f32x4 w = tile<DC>(r - 4 * lg, j - lm, lg, lm, [&](int rr, int i) { return X1[rr * DST + i]; },
                               [&](int i, int jj) { return Vb[i * DSV + jj]; });
#pragma unroll
      for (int u = 0; u < 4; ++u) Rb[(r + u) * DSV + j] = egp[r + u] * v[u] + w[u];
    });
    __syncthreads();
    // ---- U = T R
    mfma_mm<DC, DVB, DC, 4>(wave, lane, [&](int r, int i) { return Tb[r * DST + i]; },
                            [&](int i, int j) { return Rb[i * DSV + j]; }, [&](int r, int j, f32x4 v) {
#pragma unroll
                              for (int u = 0; u < 4; ++u) Ub[(r + u) * DSV + j] = v[u];
                            });
    __syncthreads();
    // ---- P_qb into X1; O += P_qb U
    gram(Q_, B_, e_out);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int t = wave + 4 * q, m0 = (t >> 1) * 16, n0 = (t & 1) * 16;
      Oacc[q] += tile<DC>(m0, n0, lg, lm, [&](int r, int i) { return X1[r * DST + i]; },
                          [&](int i, int j) { return Ub[i * DSV + j]; });
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = m0 + 4 * lg + u;
        if (r < nv) ((E *)p.o)[((tb + r) * H + h) * dv + col0 + n0 + lm] = to_e<E>(Oacc[q][u]);
      }
    }
    // ---- M <- e^{G_C} M + (e^{G_C - G} B)^T U + (e^{G_C - G} K)^T V   (DK x 32)
    {
      constexpr int TPW = (DK / 16) * 2 / 4;  // tiles per wave
      f32x4 nm[TPW];
      const float gam = misc[0];
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int t = wave + 4 * q, m0 = (t >> 1) * 16, n0 = (t & 1) * 16;
        const f32x4 t1 = tile<DC>(m0, n0, lg, lm, [&](int d, int r) { return et[r] * B_(r, d); },
                                  [&](int r, int j) { return Ub[r * DSV + j]; });
        const f32x4 t2 = tile<DC>(m0, n0, lg, lm, [&](int d, int r) { return et[r] * K_(r, d); },
                                  [&](int r, int j) { return Vb[r * DSV + j]; });
#pragma unroll
        for (int u = 0; u < 4; ++u) nm[q][u] = gam * Ml[(m0 + 4 * lg + u) * DSV + n0 + lm] + t1[u] + t2[u];
      }
      __syncthreads();  // every read of the old state is done
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int t = wave + 4 * q, m0 = (t >> 1) * 16, n0 = (t & 1) * 16;
#pragma unroll
        for (int u = 0; u < 4; ++u) Ml[(m0 + 4 * lg + u) * DSV + n0 + lm] = nm[q][u];
      }
    }
  }
  __syncthreads();
  if (p.final_state)
    for (int i = tid; i < DK * DVB; i += DNT) {
      const int d = i / DVB, j = i % DVB;
      p.final_state[sstate + (size_t)d * dv + j] = Ml[d * DSV + j];
    }
}

// bf16 I/O: every product on the bf16 matrix cores (16x16x32).  The inputs q, k, a, b,
// v are bf16 already, so the four Gram products Q K^T, A B^T, A K^T, Q B^T are exact
// bf16 MFMAs; a product with an fp32 operand (the state, T, R, U, the decayed Gram
// tiles) takes that operand as a hi + lo pair of bf16 terms (Split), which keeps it to
// about 2^-17 relative.  M, R, U and V are kept transposed ([value column][k]) so that
// every fragment is one or two 16-byte LDS reads; K^T and B^T fragments of the state
// update come from the transposing LDS read.  The next chunk's inputs are loaded into
// registers while the current one computes.
template <int DK, int GATE>
__global__ __launch_bounds__(DNB, 1) void dplr_bf16_kernel(DplrParams p) {
  constexpr int SKE = DK + 8;  // bf16 row pitch of Q, K, A, B
  constexpr int SX = DC + 4;   // fp32 row pitch of the 64 x 64 tiles
  constexpr int SM = DK + 4;   // fp32 row pitch of M^T
  constexpr int SVT = DC + 8;  // bf16 row pitch of V^T
  constexpr int SR = DC + 4;   // fp32 row pitch of R^T and U^T
  constexpr int RK = DC * DK / 8 / DNB;  // 16-byte pieces of a [64][DK] operand per thread
  constexpr int OQ = 8 / NWB;             // 64 x 32 output tiles per wave
  __shared__ __align__(16) bf16 Ql[DC * SKE];
  __shared__ __align__(16) bf16 Kl[DC * SKE];
  __shared__ __align__(16) bf16 Al[DC * SKE];
  __shared__ __align__(16) bf16 Bl[DC * SKE];
  __shared__ __align__(16) bf16 Vt[DVB * SVT];
  __shared__ __align__(16) float X1[DC * SX];
  __shared__ __align__(16) float X2[DC * SX];
  __shared__ __align__(16) float Tb[DC * SX];
  __shared__ __align__(16) float Mt[DVB * SM];
  __shared__ __align__(16) float Rt[DVB * SR];
  __shared__ __align__(16) float Ut[DVB * SR];
  __shared__ __align__(16) float gs[DC], eg[DC], egp[DC], et[DC];
  __shared__ float misc[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H, dv = p.dv, nb = dv / DVB;
  int pair, jb;
  xcd_pair_block(blockIdx.x, p.N * p.H, nb, pair, jb);
  const int n = pair / H, h = pair % H, col0 = jb * DVB;
  long tok0;
  int len;
  if (p.cu_seqlens) {
    const int s0 = p.cu_seqlens[n], s1 = p.cu_seqlens[n + 1];
    if (s0 < 0 || s1 < s0 || s1 > p.T) return;  // malformed offsets: leave untouched
    tok0 = s0;
    len = s1 - s0;
  } else {
    tok0 = (long)n * p.T;
    len = p.T;
  }
  const int nchunks = (len + DC - 1) / DC;
  const size_t sstate = ((size_t)n * H + h) * DK * dv + col0;

  // fragment loaders: rows of a bf16 operand (exact), rows of an fp32 one (split)
  auto rowb = [&](const bf16 *X, int pitch, int row) {
    const bf16 *base = X + row * pitch + 8 * lg;
    return [=](int k0) { return ld8(base + k0); };
  };
  auto rowf = [&](const float *X, int pitch, int row) {
    const float *base = X + row * pitch + 8 * lg;
    return [=](int k0) { return split8(ld8(base + k0)); };
  };

  for (int i = tid; i < DK * DVB; i += DNB) {
    const int d = i / DVB, j = i % DVB;
    Mt[j * SM + d] = p.init_state ? p.init_state[sstate + (size_t)d * dv + j] : 0.f;
  }
  for (int i = tid; i < DC * SX; i += DNB) Tb[i] = X1[i] = X2[i] = 0.f;  // upper blocks stay zero

  // ---- a chunk's inputs: 16-byte loads into registers one chunk ahead (rows past the
  // sequence end re-read its last row and are zeroed when staged)
  u32x4 pq[RK], pk[RK], pa[RK], pb[RK], pv;
  float pl = 0.f;
  auto fetch = [&](int cc) {
    const int last = min(DC, len - cc * DC) - 1;
    const size_t tbc = (size_t)tok0 + (size_t)cc * DC;
#pragma unroll
    for (int u = 0; u < RK; ++u) {
      const int pc = tid + DNB * u, r = min(pc / (DK / 8), last), g = pc % (DK / 8);
      const size_t o = ((tbc + r) * H + h) * DK + g * 8;
      pq[u] = *(const u32x4 *)((const bf16 *)p.q + o);
      pk[u] = *(const u32x4 *)((const bf16 *)p.k + o);
      pa[u] = *(const u32x4 *)((const bf16 *)p.a + o);
      pb[u] = *(const u32x4 *)((const bf16 *)p.b + o);
    }
    if (tid < DC * DVB / 8) {  // V: one 16-byte piece per thread of the first 256
      const int r = min(tid / 4, last), g = tid % 4;
      pv = *(const u32x4 *)((const bf16 *)p.v + ((tbc + r) * H + h) * dv + col0 + 8 * g);
    }
    if (GATE == GATE_HEAD && tid < DC) pl = p.log_alpha[(tbc + min(tid, last)) * p.la_stride + h];
  };
  if (nchunks > 0) fetch(0);

  for (int c = 0; c < nchunks; ++c) {
    const int nv = min(DC, len - c * DC);
    const size_t tb = (size_t)tok0 + (size_t)c * DC;
    __syncthreads();  // the previous chunk is done with every buffer
    // ---- stage the inputs; wave 0 forms the decay prefix from its registers
#pragma unroll
    for (int u = 0; u < RK; ++u) {
      opaque(pq[u]);
      opaque(pk[u]);
      opaque(pa[u]);
      opaque(pb[u]);
      const int pc = tid + DNB * u, r = pc / (DK / 8), g = pc % (DK / 8);
      if (r >= nv) pq[u] = pk[u] = pa[u] = pb[u] = (u32x4){0u, 0u, 0u, 0u};
      *(u32x4 *)(Ql + r * SKE + g * 8) = pq[u];
      *(u32x4 *)(Kl + r * SKE + g * 8) = pk[u];
      *(u32x4 *)(Al + r * SKE + g * 8) = pa[u];
      *(u32x4 *)(Bl + r * SKE + g * 8) = pb[u];
    }
    if (tid < DC * DVB / 8) {
      opaque(pv);
      const int r = tid / 4, g = tid % 4;
      const bf16x8 v8 = __builtin_bit_cast(bf16x8, pv);
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(8 * g + e) * SVT + r] = r < nv ? v8[e] : (bf16)0.f;
    }
    if (wave == 0) {  // e^G, e^{G_{j-1}}, e^{G_C - G}, e^{G_C}
      opaque(pl);
      float g = lane < nv ? pl : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(g, off);
        if (lane >= off) g += y;
      }
      const float gC = __shfl(g, 63), gp = __shfl_up(g, 1);
      gs[lane] = g;
      eg[lane] = __expf(g);
      egp[lane] = lane == 0 ? 1.f : __expf(gp);
      et[lane] = __expf(gC - g);
      if (lane == 0) misc[0] = __expf(gC);
    }
    if (c + 1 < nchunks) fetch(c + 1);  // in flight during this chunk's compute
    __syncthreads();
    auto e_out = [&](int r, int j) {  // e^{G_r - G_j}, j <= r
      return j <= r ? (GATE == GATE_HEAD ? __expf(gs[r] - gs[j]) : 1.f) : 0.f;
    };
    auto e_in = [&](int j, int i) {  // e^{G_{j-1} - G_i}, i < j
      return i < j ? (GATE == GATE_HEAD ? __expf((j > 0 ? gs[j - 1] : 0.f) - gs[i]) : 1.f) : 0.f;
    };
    // X = lower(R C^T * fac): the 10 lower 16x16 tiles over waves w0 .. w0 + nw - 1 (the
    // upper ones were zeroed once and are never written)
    auto gram = [&](const bf16 *R, const bf16 *Cm, auto fac, float *X, int w0, int nw) {
      for (int t = wave - w0; t < 10; t += nw) {
        const int mb = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
        const int m0 = 16 * mb, n0 = 16 * (t - mb * (mb + 1) / 2);
        const f32x4 v = tile_frag<DK>(rowb(R, SKE, m0 + lm), rowb(Cm, SKE, n0 + lm));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = m0 + 4 * lg + u, i = n0 + lm;
          X[r * SX + i] = v[u] * fac(r, i);
        }
      }
    };
    // output tiles of a 64 x 32 product: two per wave
    auto otile = [&](int q, int &m0, int &n0) {
      const int t = wave + NWB * q;
      m0 = (t >> 1) * 16;
      n0 = (t & 1) * 16;
    };
    auto kend = [](int m0) { return m0 < 32 ? 32 : 64; };  // last nonzero column of a lower row block
    // ---- O = diag(e^G) Q M0 in registers; P_qk into X1
    f32x4 Oacc[OQ];
#pragma unroll
    for (int q = 0; q < OQ; ++q) {
      int m0, n0;
      otile(q, m0, n0);
      const f32x4 v = tile_frag<DK>(rowb(Ql, SKE, m0 + lm), rowf(Mt, SM, n0 + lm));
#pragma unroll
      for (int u = 0; u < 4; ++u) Oacc[q][u] = eg[m0 + 4 * lg + u] * v[u];
    }
    gram(Ql, Kl, e_out, X1, 0, NWB);
    __syncthreads();
    // ---- O += P_qk V; A_ab into X2
#pragma unroll
    for (int q = 0; q < OQ; ++q) {
      int m0, n0;
      otile(q, m0, n0);
      Oacc[q] += tile_frag<DC>(rowf(X1, SX, m0 + lm), rowb(Vt, SVT, n0 + lm), kend(m0));
    }
    gram(Al, Bl, e_in, X2, 0, NWB);
    __syncthreads();
    // ---- T = (I - A_ab)^-1 into Tb (waves 0-2) while the other waves form A_ak (into X1)
    // and then R = diag(e^{G_{j-1}}) A M0 + A_ak V (into R^T)
    if (wave == 0) {  // diagonal blocks: lane (lg, lm) solves column lm of block lg
      const int o = 16 * lg;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float *arow = X2 + (o + r) * SX + o;
        float acc = r == lm ? 1.f : 0.f;
#pragma unroll
        for (int i4 = 0; i4 < (r + 3) / 4; ++i4) {
          const f32x4 a4 = *(const f32x4 *)(arow + 4 * i4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * i4 + e < r) acc += a4[e] * x[4 * i4 + e];
        }
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Tb[(o + r) * SX + o + lm] = x[r];
    } else {
      gram(Al, Kl, e_in, X1, 1, NWB - 1);
    }
    __syncthreads();
    if (wave < 3) {  // off-diagonal blocks, block column b = wave: T[a][b] = T[a][a] sum_k A[a][k] T[k][b]
      const int b = wave;
      float *ys = Ut + wave * (16 * 20);  // scratch (U is formed afterwards): y^T, row pitch 20
      for (int a = b + 1; a < 4; ++a) {
        f32x4 y = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DC; k0 += 32) {
          if (k0 + 32 <= 16 * b || k0 >= 16 * a) continue;  // wave-uniform
          const int kk = k0 + 8 * lg;                        // this lane's 8 k-slots
          const bool in = kk >= 16 * b && kk < 16 * a;
          f32x8 af = ld8(X2 + (16 * a + lm) * SX + kk), bfv;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (!in) af[i] = 0.f;
            bfv[i] = Tb[(kk + i) * SX + 16 * b + lm];
          }
          y = mm(split8(af), split8(bfv), y);
        }
        *(f32x4 *)(ys + lm * 20 + 4 * lg) = y;
        __builtin_amdgcn_wave_barrier();
        f32x8 tf = ld8(Tb + (16 * a + lm) * SX + 16 * a + 8 * (lg & 1));
        f32x8 yf = ld8(ys + lm * 20 + 8 * (lg & 1));
        if (lg >= 2) tf = yf = (f32x8){0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const f32x4 z = mm(split8(tf), split8(yf), zero4());
#pragma unroll
        for (int u = 0; u < 4; ++u) Tb[(16 * a + 4 * lg + u) * SX + 16 * b + lm] = z[u];
        __builtin_amdgcn_wave_barrier();
      }
    } else {
      for (int t = wave - 3; t < 8; t += NWB - 3) {  // the 8 tiles of R over waves 3 ..
        const int m0 = (t >> 1) * 16, n0 = (t & 1) * 16;
        const f32x4 v = tile_frag<DK>(rowb(Al, SKE, m0 + lm), rowf(Mt, SM, n0 + lm));
        const f32x4 w = tile_frag<DC>(rowf(X1, SX, m0 + lm), rowb(Vt, SVT, n0 + lm), kend(m0));
        f32x4 res;
#pragma unroll
        for (int u = 0; u < 4; ++u) res[u] = egp[m0 + 4 * lg + u] * v[u] + w[u];
        *(f32x4 *)(Rt + (n0 + lm) * SR + m0 + 4 * lg) = res;
      }
    }
    __syncthreads();
    // ---- U = T R into U^T; P_qb into X1
#pragma unroll
    for (int q = 0; q < OQ; ++q) {
      int m0, n0;
      otile(q, m0, n0);
      const f32x4 v = tile_frag<DC>(rowf(Tb, SX, m0 + lm), rowf(Rt, SR, n0 + lm), kend(m0));
      *(f32x4 *)(Ut + (n0 + lm) * SR + m0 + 4 * lg) = v;
    }
    gram(Ql, Bl, e_out, X1, 0, NWB);
    __syncthreads();
    // ---- O += P_qb U; store O
#pragma unroll
    for (int q = 0; q < OQ; ++q) {
      int m0, n0;
      otile(q, m0, n0);
      Oacc[q] += tile_frag<DC>(rowf(X1, SX, m0 + lm), rowf(Ut, SR, n0 + lm), kend(m0));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = m0 + 4 * lg + u;
        if (r < nv) ((bf16 *)p.o)[((tb + r) * H + h) * dv + col0 + n0 + lm] = (bf16)Oacc[q][u];
      }
    }
    // ---- M <- e^{G_C} M + B^T diag(e^{G_C - G}) U + K^T diag(e^{G_C - G}) V   (DK x 32)
    {
      constexpr int TPW = (DK / 16) * 2 / NWB;  // tiles per wave
      f32x4 nm[TPW];
      const float gam = misc[0];
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int t = wave + NWB * q, m0 = (t >> 1) * 16, n0 = (t & 1) * 16;
        const float *urow = Ut + (n0 + lm) * SR + 8 * lg;
        const bf16 *vrow = Vt + (n0 + lm) * SVT + 8 * lg;
        const f32x4 t1 = tile_frag<DC>([&](int k0) { return col_frag(Bl, SKE, k0, m0, lg, lm); },
                                       [&](int k0) {
                                         const f32x8 e8 = ld8(et + k0 + 8 * lg);
                                         return split8(ld8(urow + k0) * e8);
                                       });
        const f32x4 t2 = tile_frag<DC>([&](int k0) { return col_frag(Kl, SKE, k0, m0, lg, lm); },
                                       [&](int k0) {
                                         const f32x8 e8 = ld8(et + k0 + 8 * lg);
                                         return split8(widen8(ld8(vrow + k0)) * e8);
                                       });
        const f32x4 mo = *(const f32x4 *)(Mt + (n0 + lm) * SM + m0 + 4 * lg);
        nm[q] = gam * mo + t1 + t2;
      }
      __syncthreads();  // every read of the old state is done
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const int t = wave + NWB * q, m0 = (t >> 1) * 16, n0 = (t & 1) * 16;
        *(f32x4 *)(Mt + (n0 + lm) * SM + m0 + 4 * lg) = nm[q];
      }
    }
  }
  __syncthreads();
  if (p.final_state)
    for (int i = tid; i < DK * DVB; i += DNB) {
      const int d = i / DVB, j = i % DVB;
      p.final_state[sstate + (size_t)d * dv + j] = Mt[j * SM + d];
    }
}

// One token per stream, the state updated in place (the constant-cost decode step of
// "Decoding Hybrid Linear Attention Architectures", sec. 6, for this transition).  With
// the state M (rows d, columns j) read once:
//   u_j = sum_d a_d M[d][j],  s_j = sum_d q_d alpha_d M[d][j]
//   M'  = Diag(alpha) M + b u^T + k v^T,   o_j = s_j + (q . b) u_j + (q . k) v_j
// One workgroup per (stream, head); each thread keeps RP rows x 4 columns of M in
// registers, the two column reductions go through LDS.
template <typename E, int DK, int DV, int GATE>
__global__ __launch_bounds__(256) void dplr_step_kernel(DplrStepParams p) {
  constexpr int CQ = DV / 4;    // column quads
  constexpr int RG = 256 / CQ;  // row groups
  constexpr int RP = DK / RG;   // rows per thread
  static_assert(RP >= 1 && RG * RP == DK, "step geometry");
  __shared__ float qs[DK], as_[DK], bs_[DK], ks[DK], al[DK];
  __shared__ f32x4 red_u[RG][CQ], red_s[RG][CQ];
  __shared__ float dots[2];

  const int pair = blockIdx.x;  // stream * H + head
  const int tid = threadIdx.x, cq = tid % CQ, rg = tid / CQ;
  const size_t rowk = (size_t)pair * DK;
  if (tid < DK) {
    qs[tid] = to_f(((const E *)p.q)[rowk + tid]);
    as_[tid] = to_f(((const E *)p.a)[rowk + tid]);
    bs_[tid] = to_f(((const E *)p.b)[rowk + tid]);
    ks[tid] = to_f(((const E *)p.k)[rowk + tid]);
    float a = 1.f;
    if (GATE == GATE_HEAD) a = __expf(p.log_alpha[(size_t)(pair / p.H) * p.la_stride + pair % p.H]);
    if (GATE == GATE_KEY) a = __expf(p.log_alpha[rowk + tid]);
    al[tid] = a;
  }
  float *st = p.state + (size_t)pair * DK * DV;
  f32x4 m[RP];
#pragma unroll
  for (int u = 0; u < RP; ++u) m[u] = *(const f32x4 *)(st + (size_t)(rg * RP + u) * DV + 4 * cq);
  const E *vp = (const E *)p.v + (size_t)pair * DV + 4 * cq;  // needed only after the reductions
  f32x4 vv;
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = to_f(vp[e]);
  __syncthreads();

  f32x4 uu = zero4(), ss = zero4();
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    const int row = rg * RP + u;
    uu += m[u] * as_[row];
    ss += m[u] * (qs[row] * al[row]);
  }
  red_u[rg][cq] = uu;
  red_s[rg][cq] = ss;
  if (tid < 64) {  // q . b and q . k
    float db = 0.f, dk = 0.f;
    for (int i = tid; i < DK; i += 64) {
      db += qs[i] * bs_[i];
      dk += qs[i] * ks[i];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      db += __shfl_xor(db, off);
      dk += __shfl_xor(dk, off);
    }
    if (tid == 0) {
      dots[0] = db;
      dots[1] = dk;
    }
  }
  __syncthreads();

  f32x4 U = zero4(), S = zero4();
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    U += red_u[g][cq];
    S += red_s[g][cq];
  }
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    const int row = rg * RP + u;
    *(f32x4 *)(st + (size_t)row * DV + 4 * cq) = m[u] * al[row] + U * bs_[row] + vv * ks[row];
  }
  if (rg == 0) {
    E *o = (E *)p.o + (size_t)pair * DV + 4 * cq;
    const float qb = dots[0], qk = dots[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = to_e<E>(S[e] + qb * U[e] + qk * vv[e]);
  }
}

// Serving decode of this transition: L tokens per stream against a pool of states.  The
// stream's state is read once from slot src[n], carried through its L tokens in
// registers (the step above, token by token), and stored after token t into slot
// dst[n, t] when that slot is in [0, P).  A stream whose src slot is outside [0, P) is
// padding: nothing is read or written for it.
template <typename E, int DK, int DV, int GATE>
__global__ __launch_bounds__(256) void dplr_decode_kernel(DplrDecodeParams p) {
  constexpr int CQ = DV / 4;
  constexpr int RG = 256 / CQ;
  constexpr int RP = DK / RG;
  static_assert(RP >= 1 && RG * RP == DK, "decode geometry");
  __shared__ float qs[2][DK], as_[2][DK], bs_[2][DK], ks[2][DK], al[2][DK];
  __shared__ f32x4 red_u[RG][CQ], red_s[RG][CQ];
  __shared__ float dots[2][2];

  const int pair = blockIdx.x, n = pair / p.H, h = pair % p.H;
  const int src = p.src[n];
  if (src < 0 || src >= p.P) return;  // padding stream
  const int tid = threadIdx.x, cq = tid % CQ, rg = tid / CQ;
  const size_t slot = (size_t)p.H * DK * DV, head = (size_t)h * DK * DV;
  f32x4 m[RP];
  {
    const float *st = p.pool + (size_t)src * slot + head;
#pragma unroll
    for (int u = 0; u < RP; ++u) m[u] = *(const f32x4 *)(st + (size_t)(rg * RP + u) * DV + 4 * cq);
  }
  for (int t = 0; t < p.L; ++t) {
    const int b = t & 1;  // the token vectors alternate between two buffers
    const size_t tok = (size_t)n * p.L + t, rowk = (tok * p.H + h) * DK;
    if (tid < DK) {
      qs[b][tid] = to_f(((const E *)p.q)[rowk + tid]);
      as_[b][tid] = to_f(((const E *)p.a)[rowk + tid]);
      bs_[b][tid] = to_f(((const E *)p.b)[rowk + tid]);
      ks[b][tid] = to_f(((const E *)p.k)[rowk + tid]);
      float a = 1.f;
      if (GATE == GATE_HEAD) a = __expf(p.log_alpha[tok * p.la_stride + h]);
      if (GATE == GATE_KEY) a = __expf(p.log_alpha[rowk + tid]);
      al[b][tid] = a;
    }
    const E *vp = (const E *)p.v + (tok * p.H + h) * DV + 4 * cq;
    f32x4 vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = to_f(vp[e]);
    __syncthreads();
    f32x4 uu = zero4(), ss = zero4();
#pragma unroll
    for (int u = 0; u < RP; ++u) {
      const int row = rg * RP + u;
      uu += m[u] * as_[b][row];
      ss += m[u] * (qs[b][row] * al[b][row]);
    }
    red_u[rg][cq] = uu;
    red_s[rg][cq] = ss;
    if (tid < 64) {
      float db = 0.f, dk = 0.f;
      for (int i = tid; i < DK; i += 64) {
        db += qs[b][i] * bs_[b][i];
        dk += qs[b][i] * ks[b][i];
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        db += __shfl_xor(db, off);
        dk += __shfl_xor(dk, off);
      }
      if (tid == 0) {
        dots[b][0] = db;
        dots[b][1] = dk;
      }
    }
    __syncthreads();
    f32x4 U = zero4(), S = zero4();
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      U += red_u[g][cq];
      S += red_s[g][cq];
    }
#pragma unroll
    for (int u = 0; u < RP; ++u) {
      const int row = rg * RP + u;
      m[u] = m[u] * al[b][row] + U * bs_[b][row] + vv * ks[b][row];
    }
    if (rg == 0) {
      E *o = (E *)p.o + (tok * p.H + h) * DV + 4 * cq;
      const float qb = dots[b][0], qk = dots[b][1];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = to_e<E>(S[e] + qb * U[e] + qk * vv[e]);
    }
    const int dst = p.dst[tok];
    if (dst >= 0 && dst < p.P) {
      float *sd = p.pool + (size_t)dst * slot + head;
#pragma unroll
      for (int u = 0; u < RP; ++u) *(f32x4 *)(sd + (size_t)(rg * RP + u) * DV + 4 * cq) = m[u];
    }
    // red_u / red_s are rewritten by the next token only after its first barrier, which
    // every thread reaches after reading them here
  }
}

template <typename E, int DK, int DV>
hipError_t launch_dd(const DplrDecodeParams &p, int gate, hipStream_t stream) {
  const dim3 grid(p.N * p.H), block(256);
  if (gate == GATE_NONE)
    hipLaunchKernelGGL((dplr_decode_kernel<E, DK, DV, GATE_NONE>), grid, block, 0, stream, p);
  else if (gate == GATE_HEAD)
    hipLaunchKernelGGL((dplr_decode_kernel<E, DK, DV, GATE_HEAD>), grid, block, 0, stream, p);
  else if (gate == GATE_KEY)
    hipLaunchKernelGGL((dplr_decode_kernel<E, DK, DV, GATE_KEY>), grid, block, 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
template <typename E>
hipError_t launch_dd_e(const DplrDecodeParams &p, int dk, int dv, int gate, hipStream_t stream) {
  if (dk == 64 && dv == 64) return launch_dd<E, 64, 64>(p, gate, stream);
  if (dk == 64 && dv == 128) return launch_dd<E, 64, 128>(p, gate, stream);
  if (dk == 128 && dv == 64) return launch_dd<E, 128, 64>(p, gate, stream);
  if (dk == 128 && dv == 128) return launch_dd<E, 128, 128>(p, gate, stream);
  return hipErrorInvalidValue;
}

template <typename E, int DK, int DV>
hipError_t launch_ds(const DplrStepParams &p, int gate, hipStream_t stream) {
  const dim3 grid(p.N * p.H), block(256);
  if (gate == GATE_NONE)
    hipLaunchKernelGGL((dplr_step_kernel<E, DK, DV, GATE_NONE>), grid, block, 0, stream, p);
  else if (gate == GATE_HEAD)
    hipLaunchKernelGGL((dplr_step_kernel<E, DK, DV, GATE_HEAD>), grid, block, 0, stream, p);
  else if (gate == GATE_KEY)
    hipLaunchKernelGGL((dplr_step_kernel<E, DK, DV, GATE_KEY>), grid, block, 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
template <typename E>
hipError_t launch_ds_e(const DplrStepParams &p, int dk, int dv, int gate, hipStream_t stream) {
  if (dk == 64 && dv == 64) return launch_ds<E, 64, 64>(p, gate, stream);
  if (dk == 64 && dv == 128) return launch_ds<E, 64, 128>(p, gate, stream);
  if (dk == 128 && dv == 64) return launch_ds<E, 128, 64>(p, gate, stream);
  if (dk == 128 && dv == 128) return launch_ds<E, 128, 128>(p, gate, stream);
  return hipErrorInvalidValue;
}

template <typename E, int DK>
hipError_t launch_dp(const DplrParams &p, int gate, hipStream_t stream) {
  const int blocks = p.N * p.H * (p.dv / DVB);
  if (blocks == 0) return hipSuccess;
  if (gate != GATE_HEAD && gate != GATE_NONE) return hipErrorInvalidValue;
  if constexpr (std::is_same<E, bf16>::value) {
    if (gate == GATE_HEAD)
      hipLaunchKernelGGL((dplr_bf16_kernel<DK, GATE_HEAD>), dim3(blocks), dim3(DNB), 0, stream, p);
    else
      hipLaunchKernelGGL((dplr_bf16_kernel<DK, GATE_NONE>), dim3(blocks), dim3(DNB), 0, stream, p);
  } else {
    if (gate == GATE_HEAD)
      hipLaunchKernelGGL((dplr_fwd_kernel<E, DK, GATE_HEAD>), dim3(blocks), dim3(DNT), 0, stream, p);
    else
      hipLaunchKernelGGL((dplr_fwd_kernel<E, DK, GATE_NONE>), dim3(blocks), dim3(DNT), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dplr_decode(const DplrDecodeParams &p, int dtype, int dk, int dv, int gate, hipStream_t stream) {
  if (p.N == 0) return hipSuccess;
  return dtype == 1 ? launch_dd_e<bf16>(p, dk, dv, gate, stream) : launch_dd_e<float>(p, dk, dv, gate, stream);
}

hipError_t launch_dplr_step(const DplrStepParams &p, int dtype, int dk, int dv, int gate, hipStream_t stream) {
  if (p.N == 0) return hipSuccess;
  return dtype == 1 ? launch_ds_e<bf16>(p, dk, dv, gate, stream) : launch_ds_e<float>(p, dk, dv, gate, stream);
}

hipError_t launch_dplr(const DplrParams &p, int dtype, int dk, int gate, hipStream_t stream) {
  if (dtype == 1) {
    if (dk == 128) return launch_dp<bf16, 128>(p, gate, stream);
    if (dk == 64) return launch_dp<bf16, 64>(p, gate, stream);
  } else {
    if (dk == 64) return launch_dp<float, 64>(p, gate, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

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
// Two launches:
//  1. dplrk_prep_kernel, one workgroup per (chunk, head), fully parallel: the Gram
//     tiles, T = (I - A_ab)^-1 (blocked: substitution of the diagonal blocks, block
//     substitution of the rest on the matrix cores), and every state-independent
//     operand of the chunk into the caller's workspace, each already split into a hi
//     and a lo bf16 half (row-major, so that a matrix-core A fragment is two 16-byte
//     loads and needs no arithmetic): T, A_ak, P_qb, P_qk (64 x 64), A e^{Gp} and
//     Q e^G (64 x d_k), (B e^{G_C - G})^T and (K e^{G_C - G})^T (d_k x 64); e^{G_C} in fp32.
//  2. dplrk_state_kernel, one workgroup per (sequence, head, 64 or 32 value columns: 64
//     when that still gives one workgroup per compute unit), chunks in order.  The fp32 state block stays in the matrix-core accumulators of its four
//     waves (d_k / 4 key rows each) for the whole sequence; its split bf16 copy, V, R
//     and U sit transposed in LDS so that every B fragment is two 16-byte reads.
// Products run on the bf16 matrix cores with every fp32 operand a hi + lo pair (about
// 2^-17 relative error per product); bf16 inputs (v) are taken exactly; accumulation
// in fp32.
#include "gdn_common.h"
#include "gdn_kernels.h"
#include "gdn_tile.h"

namespace gdn {

namespace {

constexpr int KC = 64;
constexpr int KBV = 32;     // value columns per workgroup of the state pass
constexpr int SC = KC + 1;  // fp32 pitch of 64-column tiles in LDS
constexpr int PV = KC + 8;  // bf16 pitch of the transposed 64-row operands (V, R, U)

// One 16x16 tile over k in [0, K) from fragment loaders (steps from k0 = kend on are
// known zeros of a triangular operand and skipped; kend wave-uniform).
template <int K, class FA, class FB>
__device__ __forceinline__ f32x4 dprod(FA fa, FB fb, int kend = K) {
  f32x4 acc = zero4();
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32)
    if (k0 < kend) acc = mm(fa(k0), fb(k0), acc);
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

// The hi half of slot-head sh's copy of a (rows x cols) split matrix; its lo half
// follows at + rows * cols.
__device__ __forceinline__ bf16 *split_hi(bf16 *base, size_t sh, int rows, int cols) {
  return base + sh * 2 * (size_t)rows * cols;
}

// eight consecutive input elements as fp32 (one 16-byte read for bf16)
__device__ __forceinline__ f32x8 rowf8(const bf16 *x) { return widen8(ld8(x)); }
__device__ __forceinline__ f32x8 rowf8(const float *x) { return ld8(x); }
__device__ __forceinline__ f32x8 zero8() {
  f32x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = 0.f;
  return z;
}

constexpr int PNT = 512;  // threads of the preparation (eight waves)

template <typename E, int DK>
__global__ __launch_bounds__(PNT, 1) void dplrk_prep_kernel(DplrKeyParams p) {
  constexpr int SE = DK + 8;  // element pitch of the staged inputs (rows 16-byte aligned)
  constexpr int SG = DK + 4;
  constexpr int NP = PNT / DK, RP = KC / NP;  // prefix: parts per channel, rows per part
  __shared__ __align__(16) E As[KC * SE];
  __shared__ __align__(16) E Bs[KC * SE];
  __shared__ __align__(16) E Ks[KC * SE];
  __shared__ __align__(16) E Qs[KC * SE];
  __shared__ __align__(16) float Gs[KC * SG];
  __shared__ float Ab[KC * SC];  // A_ab
  __shared__ float Tb[KC * SC];  // T
  __shared__ float ys[3 * 16 * 17];
  __shared__ float tot[NP][DK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H;
  const long slot = blockIdx.x / H;
  const int h = blockIdx.x % H;
  long tb;
  int nv;
  if (!slot_chunk_d(p, slot, tb, nv)) return;
  const size_t sh = (size_t)slot * H + h;
  {  // 16-byte loads, all in flight before the LDS stores (rows past the end are zero)
    constexpr int VE = 16 / (int)sizeof(E), PR = DK / VE, NI = KC * PR / PNT;  // inputs
    constexpr int PG = DK / 4, NG = KC * PG / PNT;                             // log alpha
    const E *src[4] = {(const E *)p.a, (const E *)p.b, (const E *)p.k, (const E *)p.q};
    E *dst[4] = {As, Bs, Ks, Qs};
    u32x4 x[4][NI], y[NG];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int pc = tid + PNT * u, r = pc / PR, g = pc % PR;
      const size_t o = ((size_t)(tb + r) * H + h) * DK + g * VE;
#pragma unroll
      for (int a = 0; a < 4; ++a) x[a][u] = r < nv ? *(const u32x4 *)(src[a] + o) : (u32x4){0u, 0u, 0u, 0u};
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
#pragma unroll
      for (int a = 0; a < 4; ++a) *(u32x4 *)(dst[a] + r * SE + g * VE) = x[a][u];
    }
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int pc = tid + PNT * u, r = pc / PG, g = pc % PG;
      *(u32x4 *)(Gs + r * SG + 4 * g) = y[u];
    }
  }
  __syncthreads();
  {  // per-channel inclusive prefix: NP parts of RP rows per channel, then the offsets
    const int d = tid % DK, q = tid / DK;
    float g = 0.f;
    for (int r = q * RP; r < (q + 1) * RP; ++r) {
      g += Gs[r * SG + d];
      Gs[r * SG + d] = g;
    }
    tot[q][d] = g;
    __syncthreads();
    float off = 0.f;
    for (int u = 0; u < q; ++u) off += tot[u][d];
    if (q > 0)
      for (int r = q * RP; r < (q + 1) * RP; ++r) Gs[r * SG + d] += off;
  }
  __syncthreads();
  if (tid < DK) p.gam[sh * DK + tid] = __expf(Gs[(KC - 1) * SG + tid]);
  {  // A e^{Gp} and Q e^G (row-major), the write weights (channel-major), split; each
     // thread forms 8 consecutive elements and stores each half with one 16-byte store
    bf16 *ath = split_hi(p.at, sh, KC, DK), *qgh = split_hi(p.qg, sh, KC, DK);
    for (int i = 8 * tid; i < KC * DK; i += 8 * PNT) {
      const int r = i / DK, d = i % DK;
      const f32x8 av = rowf8(As + r * SE + d), qv = rowf8(Qs + r * SE + d), gr = ld8(Gs + r * SG + d);
      const f32x8 gq = r > 0 ? ld8(Gs + (r - 1) * SG + d) : zero8();
      f32x8 fa, fq;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        fa[e] = av[e] * __expf(gq[e]);
        fq[e] = qv[e] * __expf(gr[e]);
      }
      const Split sa = split8(fa), sq = split8(fq);
      *(bf16x8 *)(ath + i) = sa.hi;
      *(bf16x8 *)(ath + KC * DK + i) = sa.lo;
      *(bf16x8 *)(qgh + i) = sq.hi;
      *(bf16x8 *)(qgh + KC * DK + i) = sq.lo;
    }
    bf16 *bhh = split_hi(p.bhT, sh, DK, KC), *khh = split_hi(p.khT, sh, DK, KC);
    for (int i = 8 * tid; i < DK * KC; i += 8 * PNT) {
      const int d = i / KC, r = i % KC;
      const float gC = Gs[(KC - 1) * SG + d];
      f32x8 fb, fk;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float et = __expf(gC - Gs[(r + e) * SG + d]);
        fb[e] = to_f(Bs[(r + e) * SE + d]) * et;
        fk[e] = to_f(Ks[(r + e) * SE + d]) * et;
      }
      const Split sb = split8(fb), sk = split8(fk);
      *(bf16x8 *)(bhh + i) = sb.hi;
      *(bf16x8 *)(bhh + DK * KC + i) = sb.lo;
      *(bf16x8 *)(khh + i) = sk.hi;
      *(bf16x8 *)(khh + DK * KC + i) = sk.lo;
    }
  }
  // the Gram matrices: the ten lower 16x16 tiles of each (the upper ones are zero)
  bf16 *outs[4] = {nullptr, split_hi(p.aak, sh, KC, KC), split_hi(p.pqb, sh, KC, KC), split_hi(p.pqk, sh, KC, KC)};
  for (int t = wave; t < 64; t += PNT / 64) {
    const int w = t >> 4, tt = t & 15, a = tt >> 2, b = tt & 3;  // matrix w, tile (a, b)
    const int m = 16 * a + 7;
    const bool strict = w < 2;  // A_ab, A_ak: i < j; P_qb, P_qk: i <= r
    const E *X = w < 2 ? As : Qs;
    const E *Y = (w & 1) ? Ks : Bs;
    f32x4 acc = zero4();
    if (b <= a)
      acc = dprod<DK>(
          [&](int k0) {  // row r of X e^{G[r] - G[m]} (A rows: e^{G[r-1] - G[m]}), vector reads
            const int r = 16 * a + lm, c0 = k0 + 8 * lg;
            const int rg = strict ? r - 1 : r;
            const f32x8 xv = rowf8(X + r * SE + c0), gm = ld8(Gs + m * SG + c0);
            const f32x8 gx = rg >= 0 ? ld8(Gs + rg * SG + c0) : zero8();
            f32x8 f;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) f[ii] = xv[ii] * __expf(gx[ii] - gm[ii]);
            return split8(f);
          },
          [&](int k0) {  // row i of Y e^{G[m] - G[i]}
            const int i = 16 * b + lm, c0 = k0 + 8 * lg;
            const f32x8 yv = rowf8(Y + i * SE + c0), gm = ld8(Gs + m * SG + c0), gi = ld8(Gs + i * SG + c0);
            f32x8 f;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) f[ii] = yv[ii] * __expf(gm[ii] - gi[ii]);
            return split8(f);
          });
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * a + 4 * lg + j, i = 16 * b + lm;
      const float v = (strict ? i < r : i <= r) ? acc[j] : 0.f;
      if (w == 0)
        Ab[r * SC + i] = v;
      else
        store_split(outs[w], outs[w] + KC * KC, r * KC + i, v);
    }
  }
  __syncthreads();
  tri_inv64<-1>(Ab, SC, Tb, SC, ys);  // T = (I - A_ab)^-1
  bf16 *tmh = split_hi(p.tm, sh, KC, KC);
  for (int i = 8 * tid; i < KC * KC; i += 8 * PNT) {
    f32x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = Tb[(i / KC) * SC + i % KC + e];
    const Split st = split8(f);
    *(bf16x8 *)(tmh + i) = st.hi;
    *(bf16x8 *)(tmh + KC * KC + i) = st.lo;
  }
}

template <typename E, int DK, int NCT>
__global__ __launch_bounds__(256, 1) void dplrk_state_kernel(DplrKeyParams p) {
  constexpr int BV = 16 * NCT;  // value columns of this workgroup
  constexpr int PM = DK + 8;    // bf16 pitch of the transposed state (one row per value column)
  constexpr int SK = DK / 32;   // 32-deep steps over the key channels
  __shared__ __align__(16) bf16 MTh[BV * PM];
  __shared__ __align__(16) bf16 MTl[BV * PM];
  __shared__ __align__(16) bf16 VTh[BV * PV];
  __shared__ __align__(16) bf16 VTl[BV * PV];
  __shared__ __align__(16) bf16 RTh[BV * PV];
  __shared__ __align__(16) bf16 RTl[BV * PV];
  __shared__ __align__(16) bf16 UTh[BV * PV];
  __shared__ __align__(16) bf16 UTl[BV * PV];
  __shared__ float gsh[DK];
  constexpr bool VX = std::is_same<E, bf16>::value;  // v exact in bf16: no lo half needed
  constexpr int RB = DK / 64;                         // 16-row state blocks per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H, dv = p.dv, nb = dv / BV;
  int pair, jb;
  xcd_pair_block(blockIdx.x, p.N * p.H, nb, pair, jb);
  const int n = pair / H, h = pair % H, col0 = jb * BV;
  long tok0;
  int len;
  if (!seq_extent_d(p, n, tok0, len)) return;  // malformed offsets: leave untouched
  const int nchunks = (len + KC - 1) / KC;
  const long slot0 = (tok0 >> 6) + n;
  const size_t sbase = ((size_t)n * H + h) * DK * dv + col0;
  // the state: wave w holds key rows 16 (RB w + rb) + 4 lg + j, value columns 16 ct + lm
  f32x4 Mc[RB][NCT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 16 * (RB * wave + rb) + 4 * lg + j;
        Mc[rb][ct][j] = p.init_state ? p.init_state[sbase + (size_t)d * dv + 16 * ct + lm] : 0.f;
      }
  // a C tile (rows r0 + 4 lg + j, column 16 ct + lm) into a transposed split LDS matrix
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
  auto put_state = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) put_t(MTh, MTl, PM, 16 * (RB * wave + rb), ct, Mc[rb][ct]);
  };
  put_state();
  // B fragment (column 16 ct + lm, k = k0 + 8 lg ..) of a transposed split LDS matrix
  auto bfrag = [&](const bf16 *Xh, const bf16 *Xl, int pitch, int ct, int k0) {
    const int o = (16 * ct + lm) * pitch + k0 + 8 * lg;
    return Split{ld8(Xh + o), ld8(Xl + o)};
  };
  auto vfrag = [&](int ct, int k0) {
    if constexpr (VX) {
      return ld8(VTh + (16 * ct + lm) * PV + k0 + 8 * lg);
    } else {
      return bfrag(VTh, VTl, PV, ct, k0);
    }
  };
  const int r0 = 16 * wave + lm;    // this lane's A row of the 64-row products
  const int kend = 16 * wave + 16;  // triangular 64 x 64 operands: columns below kend
  const int ks = (kend + 31) / 32;  // ... their 32-deep steps
  // A fragments of a split matrix (rows x cols) in the workspace, row `row`: the loads
  // of each phase are issued one phase ahead and consumed from registers
  auto ldrow = [&](const bf16 *Xh, int rows, int cols, int row, int k0) {
    const bf16 *x = Xh + (size_t)row * cols + k0 + 8 * lg;
    return Split{ld8(x), ld8(x + (size_t)rows * cols)};
  };
  Split f_at[SK], f_aak[2], f_tm[2], f_qg[SK], f_pqb[2], f_pqk[2], f_bh[RB][2], f_kh[RB][2];
  auto load_r = [&](size_t sh) {
    const bf16 *ath = split_hi(p.at, sh, KC, DK), *aakh = split_hi(p.aak, sh, KC, KC);
#pragma unroll
    for (int s = 0; s < SK; ++s) f_at[s] = ldrow(ath, KC, DK, r0, 32 * s);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < ks) f_aak[s] = ldrow(aakh, KC, KC, r0, 32 * s);
  };
  auto load_u = [&](size_t sh) {
    const bf16 *tmh = split_hi(p.tm, sh, KC, KC);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < ks) f_tm[s] = ldrow(tmh, KC, KC, r0, 32 * s);
  };
  auto load_o = [&](size_t sh) {
    const bf16 *qgh = split_hi(p.qg, sh, KC, DK), *pqbh = split_hi(p.pqb, sh, KC, KC);
    const bf16 *pqkh = split_hi(p.pqk, sh, KC, KC);
#pragma unroll
    for (int s = 0; s < SK; ++s) f_qg[s] = ldrow(qgh, KC, DK, r0, 32 * s);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < ks) {
        f_pqb[s] = ldrow(pqbh, KC, KC, r0, 32 * s);
        f_pqk[s] = ldrow(pqkh, KC, KC, r0, 32 * s);
      }
  };
  auto load_m = [&](size_t sh) {
    const bf16 *bhh = split_hi(p.bhT, sh, DK, KC), *khh = split_hi(p.khT, sh, DK, KC);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int d = 16 * (RB * wave + rb) + lm;
        f_bh[rb][s] = ldrow(bhh, DK, KC, d, 32 * s);
        f_kh[rb][s] = ldrow(khh, DK, KC, d, 32 * s);
      }
  };
  // V of a chunk and its e^{G_C}, loaded one chunk ahead with no branch around a load
  // (rows past the end read the last row and are zeroed when staged): thread = (token,
  // a quarter of the columns); every thread reads the e^{G_C} of channel tid % DK
  constexpr int VC = BV / 4, VL = VC * (int)sizeof(E) / 16;  // columns, 16-byte loads
  u32x4 vraw[VL];
  float gnext = 0.f;
  auto load_v = [&](size_t tbase, int nvc, size_t shn) {
    const int r = min(tid >> 2, nvc - 1), g = tid & 3;
    const E *src = (const E *)p.v + ((tbase + r) * H + h) * dv + col0 + VC * g;
#pragma unroll
    for (int u = 0; u < VL; ++u) vraw[u] = *(const u32x4 *)(src + u * (16 / (int)sizeof(E)));
    gnext = p.gam[shn * DK + tid % DK];
  };
  if (nchunks > 0) {
    load_r((size_t)slot0 * H + h);
    load_v((size_t)tok0, min(KC, len), (size_t)slot0 * H + h);
  }
  typedef decltype(vfrag(0, 0)) VF;
  for (int c = 0; c < nchunks; ++c) {
    const size_t sh = (size_t)(slot0 + c) * H + h;
    const int nv = min(KC, len - c * KC);
    const size_t tbase = (size_t)tok0 + (size_t)c * KC;
    {
      const int r = tid >> 2, g = tid & 3;
      const bool in = r < nv;
#pragma unroll
      for (int u = 0; u < VL; ++u) {
        typedef E EV __attribute__((ext_vector_type(16 / sizeof(E))));
        const EV ev = __builtin_bit_cast(EV, vraw[u]);
#pragma unroll
        for (int e = 0; e < 16 / (int)sizeof(E); ++e) {
          const float x = in ? to_f(ev[e]) : 0.f;
          const int col = VC * g + u * (16 / (int)sizeof(E)) + e;
          const bf16 hv = (bf16)x;
          VTh[col * PV + r] = hv;
          if constexpr (!VX) VTl[col * PV + r] = (bf16)(x - (float)hv);
        }
      }
      if (tid < DK) gsh[tid] = gnext;
    }
    __syncthreads();
    load_u(sh);
    // this chunk's B fragments of M0 and V (read once, used by R, O and the update)
    Split bm[NCT][SK];
    VF bv[NCT][2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int s = 0; s < SK; ++s) bm[ct][s] = bfrag(MTh, MTl, PM, ct, 32 * s);
#pragma unroll
      for (int s = 0; s < 2; ++s) bv[ct][s] = vfrag(ct, 32 * s);
    }
    // R = (A e^{Gp}) M0 + A_ak V
    {
      f32x4 R[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        R[ct] = zero4();
#pragma unroll
        for (int s = 0; s < SK; ++s) R[ct] = mm(f_at[s], bm[ct][s], R[ct]);
#pragma unroll
        for (int s = 0; s < 2; ++s)
          if (s < ks) R[ct] = mm(f_aak[s], bv[ct][s], R[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) put_t(RTh, RTl, PV, 16 * wave, ct, R[ct]);
    }
    __syncthreads();
    load_o(sh);
    // U = (I - A_ab)^-1 R
    {
      Split br[NCT][2];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int s = 0; s < 2; ++s) br[ct][s] = bfrag(RTh, RTl, PV, ct, 32 * s);
      f32x4 U[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        U[ct] = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s)
          if (s < ks) U[ct] = mm(f_tm[s], br[ct][s], U[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) put_t(UTh, UTl, PV, 16 * wave, ct, U[ct]);
    }
    __syncthreads();
    load_m(sh);
    if (c + 1 < nchunks) load_v(tbase + KC, min(KC, len - (c + 1) * KC), sh + H);
    Split bu[NCT][2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int s = 0; s < 2; ++s) bu[ct][s] = bfrag(UTh, UTl, PV, ct, 32 * s);
    // O = (Q e^G) M0 + P_qb U + P_qk V
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 O = zero4();
#pragma unroll
      for (int s = 0; s < SK; ++s) O = mm(f_qg[s], bm[ct][s], O);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s < ks) O = mm(f_pqk[s], bv[ct][s], mm(f_pqb[s], bu[ct][s], O));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * wave + 4 * lg + j;
        if (r < nv && p.o) ((E *)p.o)[((tbase + r) * H + h) * dv + col0 + 16 * ct + lm] = to_e<E>(O[j]);
      }
    }
    if (c + 1 < nchunks) load_r(sh + H);
    // M = diag(e^{G_C}) M0 + (B e^{G_C - G})^T U + (K e^{G_C - G})^T V
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int d0 = 16 * (RB * wave + rb);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int j = 0; j < 4; ++j) Mc[rb][ct][j] *= gsh[d0 + 4 * lg + j];
#pragma unroll
        for (int s = 0; s < 2; ++s) Mc[rb][ct] = mm(f_kh[rb][s], bv[ct][s], mm(f_bh[rb][s], bu[ct][s], Mc[rb][ct]));
      }
    }
    __syncthreads();  // every read of M0, V and gam is done
    put_state();
  }
  if (p.final_state)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 16 * (RB * wave + rb) + 4 * lg + j;
          p.final_state[sbase + (size_t)d * dv + 16 * ct + lm] = Mc[rb][ct][j];
        }
}

template <typename E, int DK>
hipError_t launch_dk(const DplrKeyParams &p, hipStream_t stream) {
  const unsigned items = (unsigned)(p.slots * p.H), serial = (unsigned)(p.N * p.H * (p.dv / KBV));
  if (serial == 0) return hipSuccess;
  if (items) hipLaunchKernelGGL((dplrk_prep_kernel<E, DK>), dim3(items), dim3(PNT), 0, stream, p);
  // 64 value columns per workgroup when that still gives one per compute unit (the A
  // operands are then read once for twice the columns; the full-size per-channel test
  // takes this path), else 32
  if ((long)p.N * p.H * (p.dv / 64) >= 256)
    hipLaunchKernelGGL((dplrk_state_kernel<E, DK, 4>), dim3(serial / 2), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((dplrk_state_kernel<E, DK, KBV / 16>), dim3(serial), dim3(256), 0, stream, p);
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

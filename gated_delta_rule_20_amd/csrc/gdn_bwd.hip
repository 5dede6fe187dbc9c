// gdn_bwd.hip -- gradients of the chunked (gated) delta rule.
//
// Reverse mode through the chunk equations of the forward ("Decoding Hybrid Linear
// Attention Architectures", sec. 5; the WY / UT form of "Linear Attention Variants",
// DeltaNet section), for the delta write and the additive write, with no gate, one
// decay per (token, head) or one constant decay per head.
// Per chunk, with G the chunk-local decay prefix, Gamma[r,i] = e^{G_r - G_i} (i <= r),
// Kt = e^G K, Qt = e^G Q, Kh = e^{G_C - G} K, gam = e^{G_C},
// A = strict(diag(beta)(K K^T * Gamma)), T = (I + A)^-1, P = incl(Q K^T * Gamma),
// X = diag(beta)(V - Kt M0), Delta = T X, O = Qt M0 + P Delta,
// M_C = gam M0 + Kh^T Delta; given dO and dM (the gradient of M_C):
//   dDelta = P^T dO + Kh dM,   Y = T^T dDelta,   dV = diag(beta) Y
//   dM0    = Qt^T dO + gam dM - Kt^T diag(beta) Y            (carried to the chunk before)
//   dT = dDelta X^T,  dA = -strict(T^T dT T^T),  dP = incl(dO Delta^T)
//   dQt = dO M0^T,  dKt = -diag(beta) Y M0^T,  dKh = Delta dM^T,  dbeta_r += Y_r . (V - Kt M0)_r
// then A, P, Gamma, Kt, Qt, Kh and gam give dq, dk, dbeta and dG, and d log alpha_t is
// the sum of dG_r over r >= t in the chunk plus dG_C.
//
// Four launches:
//  1. a forward that stores every chunk's entering state M0 instead of o: the
//     pipelined kernel's STATES variant for bf16 with d_k = 128, the fused kernel
//     otherwise;
//  2. bwd_prep_kernel, one workgroup per (chunk, head), fully parallel: P and T of every
//     chunk (the parts of the chunk that depend on neither state nor value columns);
//  3. bwd_state_kernel, one workgroup per (sequence, head, 32 value columns), walks the
//     chunks in reverse carrying dM: it writes dV and the entering-state gradient, and
//     per value block the partial sums of dP, dT, dQ, dK, dG, dbeta and dG_C (the terms
//     that sum over value columns);
//  4. bwd_chunk_kernel, one workgroup per (chunk, head), fully parallel: it sums the
//     partials in a fixed order (deterministic), forms dA and the Gram / Gamma terms
//     and writes dq, dk, dbeta and d log alpha.
// All arithmetic is fp32 or its equivalent (inputs in bf16 or fp32).  With bf16 I/O the
// products run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16): an operand whose
// values are bf16 inputs (q, k, dO) is taken exactly, any other is split into a hi + lo
// pair of bf16 terms (about 2^-17 relative error per product).  With fp32 I/O they run
// on v_mfma_f32_16x16x4f32 with operands gathered from LDS.  The rest runs on the
// vector units.
#include "gdn_common.h"
#include "gdn_kernels.h"
#include "gdn_tile.h"

namespace gdn {

namespace {

constexpr int BC = 64;    // chunk length
constexpr int BNT = 1024;  // threads per workgroup of the per-chunk kernel (four waves per SIMD)
constexpr int BNW = BNT / 64;
// threads per workgroup of the reverse-state kernel: the additive write's variant runs
// two waves per SIMD; the delta write's needs more registers than that leaves (256 per
// wave) and runs one
template <bool ADD> constexpr int state_threads() { return ADD ? 512 : 256; }
constexpr int BVB = 32;   // value columns per workgroup of the reverse-state kernel
constexpr int SV = BVB + 4, ST = BC + 1;  // fp32 row strides (padded; SV rows 16-byte aligned)

// floats of one partial record (per chunk slot, head and value block); dP, dT (64 x 64)
// and dQ, dK (64 x d_k) are stored transposed, [column][row], so that a lane's four
// rows of a matrix-core tile are one 16-byte store and one 16-byte load
template <int DK> struct Part {
  static constexpr int DP = 0, DT = BC * BC, DQ = 2 * BC * BC, DKO = DQ + BC * DK, DG = DKO + BC * DK,
                       DB = DG + BC, GC = DB + BC, SIZE = GC + BC;
};

// sequence extent of stream n (false: malformed offsets)
__device__ __forceinline__ bool seq_extent(const BwdParams &p, int n, long &tok0, int &len) {
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

// the chunk of a slot: (first token, valid rows), or false when no chunk owns it
__device__ __forceinline__ bool slot_chunk(const BwdParams &p, long slot, size_t &tb, int &nv) {
  auto tok_start = [&](int sq) -> long { return p.cu_seqlens ? (long)p.cu_seqlens[sq] : (long)sq * p.T; };
  int lo = 0, hi = p.N - 1;  // the last n with floor(tok0_n / 64) + n <= slot
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((tok_start(mid) >> 6) + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  long tok0;
  int len;
  if (!seq_extent(p, lo, tok0, len)) return false;
  const long c = slot - ((tok0 >> 6) + lo);
  if (c < 0 || 64 * c >= len) return false;
  nv = (int)min(64L, (long)len - 64 * c);
  tb = (size_t)tok0 + (size_t)c * BC;
  return true;
}

// One workgroup per (chunk slot, head), fully parallel: P = incl(Q K^T * Gamma) and, for
// the delta write, T = (I + A)^-1 with A = strict(diag(beta) K K^T * Gamma), both fp32
// row-major into the workspace (the blocks above the diagonal zero).  The Gram tiles
// take the bf16 inputs exactly; T is the blocked inverse (tri_inv64).
template <typename E, int DK, int GATE, bool ADD>
__global__ __launch_bounds__(256, 2) void bwd_prep_kernel(BwdParams p) {
  constexpr int SKE = DK + 8;
  __shared__ __align__(16) E Kl[BC * SKE];
  __shared__ __align__(16) E Ql[BC * SKE];
  __shared__ float Al[BC * ST], Tl[BC * ST];
  __shared__ float ys[3 * 16 * 17];
  __shared__ float bs[BC], gs[BC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H;
  const long slot = blockIdx.x / H;
  const int h = blockIdx.x % H;
  size_t tb;
  int nv;
  if (!slot_chunk(p, slot, tb, nv)) return;
  auto K_ = [&](int r, int d) { return to_f(Kl[r * SKE + d]); };
  auto Q_ = [&](int r, int d) { return to_f(Ql[r * SKE + d]); };
  {  // K, Q: 16-byte loads, all in flight before the LDS stores (rows past the end zero)
    constexpr int VE = 16 / (int)sizeof(E), RK = BC * (DK / VE) / 256;
    u32x4 kv[RK], qv[RK];
#pragma unroll
    for (int u = 0; u < RK; ++u) {
      const int pc = tid + 256 * u, r = pc / (DK / VE), g = pc % (DK / VE);
      const size_t o = ((tb + r) * H + h) * DK + g * VE;
      kv[u] = r < nv ? *(const u32x4 *)((const E *)p.k + o) : (u32x4){0u, 0u, 0u, 0u};
      qv[u] = r < nv ? *(const u32x4 *)((const E *)p.q + o) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < RK; ++u) {
      const int pc = tid + 256 * u, r = pc / (DK / VE), g = pc % (DK / VE);
      *(u32x4 *)(Kl + r * SKE + g * VE) = kv[u];
      *(u32x4 *)(Ql + r * SKE + g * VE) = qv[u];
    }
  }
  if (tid < BC) {
    const bool ok = tid < nv;
    bs[tid] = (!ADD && ok) ? p.beta[(tb + tid) * H + h] : 0.f;
    gs[tid] = (GATE == GATE_HEAD && ok) ? p.log_alpha[(tb + tid) * p.la_stride + h] : 0.f;
  }
  __syncthreads();
  if (wave == 0) {
    float g = gs[lane];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(g, off);
      if (lane >= off) g += y;
    }
    gs[lane] = g;
  }
  __syncthreads();
  float *pm = p.pmat + ((size_t)slot * H + h) * BC * BC;
  for (int t = wave; t < 16; t += 4) {
    const int m0 = (t >> 2) * 16, n0 = (t & 3) * 16;
    f32x4 av = zero4(), pv = zero4();
    if (n0 <= m0) {
      if constexpr (std::is_same<E, bf16>::value) {  // bf16 rows read whole
        const E *kr = Kl + (m0 + lm) * SKE + 8 * lg, *qr = Ql + (m0 + lm) * SKE + 8 * lg;
        const E *kc = Kl + (n0 + lm) * SKE + 8 * lg;
        if (!ADD) av = tile_frag<DK>([&](int k0) { return ld8(kr + k0); }, [&](int k0) { return ld8(kc + k0); });
        pv = tile_frag<DK>([&](int k0) { return ld8(qr + k0); }, [&](int k0) { return ld8(kc + k0); });
      } else {
        if (!ADD) av = tile_g<E, DK, true, true>(m0, n0, lg, lm, K_, [&](int d, int i) { return K_(i, d); });
        pv = tile_g<E, DK, true, true>(m0, n0, lg, lm, Q_, [&](int d, int i) { return K_(i, d); });
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = m0 + 4 * lg + u, i = n0 + lm;
      const float gam = i <= r ? (GATE == GATE_HEAD ? __expf(gs[r] - gs[i]) : 1.f) : 0.f;
      if (!ADD) Al[r * ST + i] = i < r ? bs[r] * av[u] * gam : 0.f;
      pm[r * BC + i] = pv[u] * gam;
    }
  }
  if constexpr (!ADD) {
    __syncthreads();
    tri_inv64<1>(Al, ST, Tl, ST, ys);
    float *tm = p.tmat + ((size_t)slot * H + h) * BC * BC;
    for (int i4 = 4 * tid; i4 < BC * BC; i4 += 4 * 256) {
      const int r = i4 / BC, i = i4 % BC;
      *(f32x4 *)(tm + i4) = (f32x4){Tl[r * ST + i], Tl[r * ST + i + 1], Tl[r * ST + i + 2], Tl[r * ST + i + 3]};
    }
  }
}

template <typename E, int DK, int GATE, bool ADD>
__global__ __launch_bounds__(state_threads<ADD>(), 1) void bwd_state_kernel(BwdParams p) {
  constexpr int SNT = state_threads<ADD>(), NWS = SNT / 64;
  constexpr int NH = NWS / 4;  // column parts of the dQ / dK phase
  constexpr int SKE = DK + 8;
  constexpr int VE = 16 / (int)sizeof(E);        // elements per 16-byte piece
  constexpr int RK = BC * (DK / VE) / SNT;       // K / Q pieces per thread
  constexpr int NPV = BC * (BVB / VE);           // V / dO pieces
  constexpr int RV = (NPV + SNT - 1) / SNT;      // ... per thread (the first NPV threads)
  constexpr int RM = DK * (BVB / 4) / SNT;       // entering-state pieces per thread
  constexpr int RT = BC * BC / 4 / SNT;          // T / P pieces per thread
  typedef E EV __attribute__((ext_vector_type(VE)));
  typedef Part<DK> PT;
  __shared__ __align__(16) E Kl[BC * SKE];
  __shared__ __align__(16) E Ql[BC * SKE];
  __shared__ __align__(16) float Vb[BC * SV];
  __shared__ __align__(16) float dOb[BC * SV];
  __shared__ __align__(16) float M0[DK * SV];
  __shared__ __align__(16) float dM[DK * SV];
  __shared__ __align__(16) float Tl[BC * ST];
  __shared__ __align__(16) float Pl[BC * ST];
  __shared__ __align__(16) float Tb[BC * ST];
  __shared__ __align__(16) float Xl[BC * SV];
  __shared__ __align__(16) float dDl[BC * SV];
  __shared__ float bs[BC], gs[BC], eg[BC], et[BC], wsum[NWS], misc[4];
  __shared__ float rsum[NH][3][BC];  // row sums of the dQ / dK products, per column part
  // delta write: V is dead once X is formed; additive write: Delta = V and Y = dDelta
  float *const Yl = ADD ? dDl : Vb;
  float *const Dl = ADD ? Vb : Tl;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = p.H, dv = p.dv, nb = dv / BVB;
  int pair, jb;
  xcd_pair_block(blockIdx.x, p.N * p.H, nb, pair, jb);
  const int n = pair / H, h = pair % H, col0 = jb * BVB;
  long tok0;
  int len;
  if (!seq_extent(p, n, tok0, len)) return;
  const int nchunks = (len + BC - 1) / BC;
  const long slot0 = (tok0 >> 6) + n;
  const size_t sstate = ((size_t)n * H + h) * DK * dv + col0;
  auto K_ = [&](int r, int d) { return to_f(Kl[r * SKE + d]); };
  auto Q_ = [&](int r, int d) { return to_f(Ql[r * SKE + d]); };

  for (int i = tid; i < DK * BVB; i += SNT) {
    const int d = i / BVB, j = i % BVB;
    dM[d * SV + j] = p.dfinal ? p.dfinal[sstate + (size_t)d * dv + j] : 0.f;
  }

  // ---- a chunk's inputs: 16-byte loads into registers one chunk ahead (rows past the
  // sequence end re-read its last row and are zeroed when staged)
  u32x4 pk[RK], pq[RK], pv[RV], pd[RV];
  f32x4 pm[RM], pt[RT], pp[RT];
  float pb = 0.f, pl = 0.f;
  auto fetch = [&](int cc) {
    const int last = min(BC, len - cc * BC) - 1;
    const size_t tbc = (size_t)tok0 + (size_t)cc * BC;
    const size_t tp = (((size_t)slot0 + cc) * H + h) * BC * BC;  // T and P of the chunk
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      if (!ADD) pt[u] = *(const f32x4 *)(p.tmat + tp + 4 * (tid + SNT * u));
      pp[u] = *(const f32x4 *)(p.pmat + tp + 4 * (tid + SNT * u));
    }
#pragma unroll
    for (int u = 0; u < RK; ++u) {
      const int pc = tid + SNT * u, r = min(pc / (DK / VE), last), g = pc % (DK / VE);
      const size_t o = ((tbc + r) * H + h) * DK + g * VE;
      pk[u] = *(const u32x4 *)((const E *)p.k + o);
      pq[u] = *(const u32x4 *)((const E *)p.q + o);
    }
#pragma unroll
    for (int u = 0; u < RV; ++u) {
      const int pc = tid + SNT * u, r = min(pc / (BVB / VE), last), g = pc % (BVB / VE);
      if (pc >= NPV) break;
      const size_t o = ((tbc + r) * H + h) * dv + col0 + g * VE;
      pv[u] = *(const u32x4 *)((const E *)p.v + o);
      pd[u] = *(const u32x4 *)((const E *)p.dout + o);
    }
#pragma unroll
    for (int u = 0; u < RM; ++u) {
      const int pc = tid + SNT * u, d = pc / (BVB / 4), g = pc % (BVB / 4);
      pm[u] = *(const f32x4 *)(p.states + ((((size_t)slot0 + cc) * H + h) * DK + d) * dv + col0 + 4 * g);
    }
    if (tid < BC) {
      const size_t t = tbc + min(tid, last);
      pb = ADD ? 0.f : p.beta[t * H + h];
      pl = GATE == GATE_HEAD ? p.log_alpha[t * p.la_stride + h] : 0.f;
    }
  };
  auto stage = [&](int nvc) {
#pragma unroll
    for (int u = 0; u < RK; ++u) {
      opaque(pk[u]);
      opaque(pq[u]);
      const int pc = tid + SNT * u, r = pc / (DK / VE), g = pc % (DK / VE);
      if (r >= nvc) pk[u] = pq[u] = (u32x4){0u, 0u, 0u, 0u};
      *(u32x4 *)(Kl + r * SKE + g * VE) = pk[u];
      *(u32x4 *)(Ql + r * SKE + g * VE) = pq[u];
    }
#pragma unroll
    for (int u = 0; u < RV; ++u) {
      const int pc = tid + SNT * u, r = pc / (BVB / VE), g = pc % (BVB / VE);
      if (pc >= NPV) break;
      opaque(pv[u]);
      opaque(pd[u]);
      const EV ev = __builtin_bit_cast(EV, pv[u]), ed = __builtin_bit_cast(EV, pd[u]);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        Vb[r * SV + g * VE + e] = r < nvc ? to_f(ev[e]) : 0.f;
        dOb[r * SV + g * VE + e] = r < nvc ? to_f(ed[e]) : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < RM; ++u) {
      opaque(pm[u]);
      const int pc = tid + SNT * u, d = pc / (BVB / 4), g = pc % (BVB / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) M0[d * SV + 4 * g + e] = pm[u][e];
    }
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int i4 = 4 * (tid + SNT * u), r = i4 / BC, i = i4 % BC;
      if (!ADD) opaque(pt[u]);
      opaque(pp[u]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!ADD) Tb[r * ST + i + e] = pt[u][e];
        Pl[r * ST + i + e] = pp[u][e];
      }
    }
    if (tid < BC) {
      opaque(pb);
      opaque(pl);
      bs[tid] = tid < nvc ? pb : 0.f;
      gs[tid] = tid < nvc ? pl : 0.f;
    }
  };
  if (nchunks > 0) fetch(nchunks - 1);

  for (int c = nchunks - 1; c >= 0; --c) {
    const int nv = min(BC, len - c * BC);
    const size_t tb = (size_t)tok0 + (size_t)c * BC;  // token of row 0
    const size_t slot = (size_t)(slot0 + c);
    __syncthreads();  // the previous chunk is done with every buffer
    stage(nv);
    if (c > 0) fetch(c - 1);  // in flight during this chunk's compute
    __syncthreads();
    if (wave == 0) {  // decay prefix
      float g = gs[lane];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(g, off);
        if (lane >= off) g += y;
      }
      const float gC = __shfl(g, 63);
      gs[lane] = g;
      eg[lane] = __expf(g);
      et[lane] = __expf(gC - g);
      if (lane == 0) misc[0] = __expf(gC);
    }
    __syncthreads();
    // ---- V - Kt M0 into Xl (64 x 32; the delta write only)
    if constexpr (!ADD)
      mm_g<E, BC, BVB, DK, NWS, true, false>(wave, lane, K_, [&](int d, int j) { return M0[d * SV + j]; },
                                             [&](int r, int j, f32x4 v) {
#pragma unroll
                                               for (int u = 0; u < 4; ++u)
                                                 Xl[(r + u) * SV + j] = Vb[(r + u) * SV + j] - eg[r + u] * v[u];
                                             });
    __syncthreads();
    // ---- Delta = T diag(beta) (V - Kt M0) (the additive write: Delta = V, already in Vb);
    // dDelta = P^T dO + diag(e^{G_C - G}) K dM  (8 tiles each)
    {
      const int lg = lane >> 4, lm = lane & 15;
      for (int t = wave; t < 8; t += NWS) {
        const int m0 = (t >> 1) * 16, n0 = (t & 1) * 16;
        f32x4 dd = zero4();
        if (!ADD)
          dd = tile_g<E, BC, false, false>(m0, n0, lg, lm, [&](int r, int i) { return Tb[r * ST + i]; },
                                           [&](int i, int j) { return bs[i] * Xl[i * SV + j]; }, 0, m0 + 16);
        const f32x4 d1 = tile_g<E, BC, false, true>(m0, n0, lg, lm, [&](int r, int i) { return Pl[i * ST + r]; },
                                                    [&](int i, int j) { return dOb[i * SV + j]; }, m0);
        const f32x4 d2 =
            tile_g<E, DK, true, false>(m0, n0, lg, lm, K_, [&](int d, int j) { return dM[d * SV + j]; });
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = m0 + 4 * lg + u, j = n0 + lm;
          if (!ADD) Dl[r * SV + j] = dd[u];
          dDl[r * SV + j] = d1[u] + et[r] * d2[u];
        }
      }
    }
    __syncthreads();
    // ---- Y = T^T dDelta (the additive write: Y = dDelta, already in dDl)
    if constexpr (!ADD)
      mm_g<E, BC, BVB, BC, NWS, false, false>(wave, lane, [&](int r, int i) { return Tb[i * ST + r]; },
                              [&](int i, int j) { return dDl[i * SV + j]; }, [&](int r, int j, f32x4 v) {
#pragma unroll
                                for (int u = 0; u < 4; ++u) Yl[(r + u) * SV + j] = v[u];
                              });
    __syncthreads();
    // ---- dV (complete for this value block)
    for (int i = tid; i < BC * BVB; i += SNT) {
      const int r = i / BVB, j = i % BVB;
      if (r < nv) ((E *)p.dv_out)[((tb + r) * H + h) * dv + col0 + j] = to_e<E>(ADD ? Yl[r * SV + j] : bs[r] * Yl[r * SV + j]);
    }
    float *pr = p.part + ((slot * H + h) * nb + jb) * (size_t)PT::SIZE;
    // ---- dP = incl(dO Delta^T), dT = dDelta (diag(beta) X)^T  (partial over value columns;
    // no dT for the additive write)
    if constexpr (std::is_same<E, bf16>::value) {
      // these contract over the 32 value columns: every fragment is a row piece
      const int lg = lane >> 4, lm = lane & 15;
      for (int t = wave; t < 16; t += NWS) {
        const int m0 = (t >> 2) * 16, n0 = (t & 3) * 16, i = n0 + lm;
        f32x4 vp = zero4();
        if (n0 <= m0)
          vp = tile_frag<BVB>([&](int k0) { return to_bf8(ld8(dOb + (m0 + lm) * SV + 8 * lg + k0)); },
                              [&](int k0) { return split8(ld8(Dl + i * SV + 8 * lg + k0)); });
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (i > m0 + 4 * lg + u) vp[u] = 0.f;
        *(f32x4 *)(pr + PT::DP + i * BC + m0 + 4 * lg) = vp;
        if (!ADD) {
          const float bi = bs[i];
          const f32x4 vt = tile_frag<BVB>([&](int k0) { return split8(ld8(dDl + (m0 + lm) * SV + 8 * lg + k0)); },
                                          [&](int k0) { return split8(ld8(Xl + i * SV + 8 * lg + k0) * bi); });
          *(f32x4 *)(pr + PT::DT + i * BC + m0 + 4 * lg) = vt;
        }
      }
    } else {
      mm_g<E, BC, BC, BVB, NWS, true, false>(wave, lane, [&](int r, int j) { return dOb[r * SV + j]; },
                              [&](int j, int i) { return Dl[i * SV + j]; }, [&](int r, int i, f32x4 v) {
#pragma unroll
                                for (int u = 0; u < 4; ++u) pr[PT::DP + i * BC + r + u] = i <= r + u ? v[u] : 0.f;
                              });
      if constexpr (!ADD)
        mm_g<E, BC, BC, BVB, NWS, false, false>(wave, lane, [&](int r, int j) { return dDl[r * SV + j]; },
                                [&](int j, int i) { return bs[i] * Xl[i * SV + j]; }, [&](int r, int i, f32x4 v) {
#pragma unroll
                                  for (int u = 0; u < 4; ++u) pr[PT::DT + i * BC + r + u] = v[u];
                                });
    }
    // ---- dQ = e^G dO M0^T, dK = -e^G beta Y M0^T + e^{G_C - G} Delta dM^T, and the rows of
    // dG: e^G (dO M0^T).Q - e^G beta (Y M0^T).K - e^{G_C - G} (Delta dM^T).K.  A wave takes
    // one 16-row block and one of NH parts of the DK columns; the row sums of the parts
    // meet in LDS.
    {
      const int lg = lane >> 4, lm = lane & 15;
      const int m0 = 16 * (wave & 3), half = wave >> 2;
      float gq[4] = {0.f, 0.f, 0.f, 0.f}, gk[4] = {0.f, 0.f, 0.f, 0.f}, gz[4] = {0.f, 0.f, 0.f, 0.f};
      // this wave's rows of dO, Y and Delta as A fragments (the contraction is over the
      // 32 value columns: one 32-deep step)
      [[maybe_unused]] bf16x8 fdo;
      [[maybe_unused]] Split fy, fd;
      if constexpr (std::is_same<E, bf16>::value) {
        fdo = to_bf8(ld8(dOb + (m0 + lm) * SV + 8 * lg));
        fy = split8(ld8(Yl + (m0 + lm) * SV + 8 * lg));
        fd = split8(ld8(Dl + (m0 + lm) * SV + 8 * lg));
      }
      for (int n0 = half * (DK / NH); n0 < (half + 1) * (DK / NH); n0 += 16) {
        f32x4 w, uu, z;
        if constexpr (std::is_same<E, bf16>::value) {
          const Split fm = split8(ld8(M0 + (n0 + lm) * SV + 8 * lg));
          const Split fdm = split8(ld8(dM + (n0 + lm) * SV + 8 * lg));
          w = mm(fdo, fm, zero4());
          uu = ADD ? zero4() : mm(fy, fm, zero4());
          z = mm(fd, fdm, zero4());
        } else {
          w = tile<BVB>(m0, n0, lg, lm, [&](int r, int j) { return dOb[r * SV + j]; },
                        [&](int j, int d) { return M0[d * SV + j]; });
          uu = zero4();
          if (!ADD)
            uu = tile<BVB>(m0, n0, lg, lm, [&](int r, int j) { return Yl[r * SV + j]; },
                           [&](int j, int d) { return M0[d * SV + j]; });
          z = tile<BVB>(m0, n0, lg, lm, [&](int r, int j) { return Dl[r * SV + j]; },
                        [&](int j, int d) { return dM[d * SV + j]; });
        }
        const int d = n0 + lm;
        f32x4 sq, sk;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = m0 + 4 * lg + u;
          const float qv = Q_(r, d), kv = K_(r, d);
          sq[u] = eg[r] * w[u];
          sk[u] = -eg[r] * bs[r] * uu[u] + et[r] * z[u];
          gq[u] += w[u] * qv;
          gk[u] += uu[u] * kv;
          gz[u] += z[u] * kv;
        }
        *(f32x4 *)(pr + PT::DQ + d * BC + m0 + 4 * lg) = sq;
        *(f32x4 *)(pr + PT::DKO + d * BC + m0 + 4 * lg) = sk;
      }
      // a row's columns are spread over the 16 lanes lm of its lane group
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          gq[u] += __shfl_xor(gq[u], off);
          gk[u] += __shfl_xor(gk[u], off);
          gz[u] += __shfl_xor(gz[u], off);
        }
      if (lm == 0)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = m0 + 4 * lg + u;
          rsum[half][0][r] = gq[u];
          rsum[half][1][r] = gk[u];
          rsum[half][2][r] = gz[u];
        }
    }
    // ---- dM <- gam dM + Qt^T dO - Kt^T diag(beta) Y (no last term for the additive write)
    // (DK x 32: DK / 8 tiles), into registers: written after the next barrier
    const int lgm = lane >> 4, lmm = lane & 15;
    constexpr int TILES = (DK / 16) * 2;
    f32x4 nm[TILES / NWS];
    {
      const float gam = misc[0];
#pragma unroll
      for (int q = 0; q < TILES / NWS; ++q) {
        const int t = wave + NWS * q, m0 = (t >> 1) * 16, n0 = (t & 1) * 16;
        const f32x4 n1 = tile_g<E, BC, false, true>(m0, n0, lgm, lmm, [&](int d, int r) { return eg[r] * Q_(r, d); },
                                  [&](int r, int j) { return dOb[r * SV + j]; });
        f32x4 n2 = zero4();
        if (!ADD)
          n2 = tile_g<E, BC, false, false>(m0, n0, lgm, lmm, [&](int d, int r) { return eg[r] * bs[r] * K_(r, d); },
                                           [&](int r, int j) { return Yl[r * SV + j]; });
#pragma unroll
        for (int u = 0; u < 4; ++u) nm[q][u] = gam * dM[(m0 + 4 * lgm + u) * SV + n0 + lmm] + n1[u] - n2[u];
      }
    }
    // ---- dbeta rows: Y . (V - Kt M0);  dG_C: the e^{G_C - G} terms plus gam <M0, dM>
    float part_m = 0.f;
    for (int i = tid; i < DK * BVB; i += SNT) part_m += M0[(i / BVB) * SV + i % BVB] * dM[(i / BVB) * SV + i % BVB];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part_m += __shfl_xor(part_m, off);
    if (lane == 0) wsum[wave] = part_m;
    if (!ADD && tid < BC) {
      float sb = 0.f;
      for (int j = 0; j < BVB; ++j) sb += Yl[tid * SV + j] * Xl[tid * SV + j];
      pr[PT::DB + tid] = sb;
    }
    __syncthreads();  // every read of the old dM is done; the row sums are in LDS
    if (wave == 0) {  // lane = row: the dG rows, and dG_C (their e^{G_C - G} terms plus gam <M0, dM>)
      const int r = lane;
      float gq = 0.f, gk = 0.f, gz = 0.f;
#pragma unroll
      for (int c = 0; c < NH; ++c) {
        gq += rsum[c][0][r];
        gk += rsum[c][1][r];
        gz += rsum[c][2][r];
      }
      pr[PT::DG + r] = eg[r] * gq - eg[r] * bs[r] * gk - et[r] * gz;
      float sg = et[r] * gz;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sg += __shfl_xor(sg, off);
      float wm = 0.f;
#pragma unroll
      for (int w = 0; w < NWS; ++w) wm += wsum[w];
      if (lane == 0) pr[PT::GC] = sg + misc[0] * wm;
    }
#pragma unroll
    for (int q = 0; q < TILES / NWS; ++q) {
      const int t = wave + NWS * q, m0 = (t >> 1) * 16, n0 = (t & 1) * 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) dM[(m0 + 4 * lgm + u) * SV + n0 + lmm] = nm[q][u];
    }
  }
  __syncthreads();
  if (p.dinit)
    for (int i = tid; i < DK * BVB; i += SNT) {
      const int d = i / BVB, j = i % BVB;
      p.dinit[sstate + (size_t)d * dv + j] = dM[d * SV + j];
    }
}

template <typename E, int DK, int GATE, bool ADD>
__global__ __launch_bounds__(BNT, 1) void bwd_chunk_kernel(BwdParams p) {
  constexpr int SKE = DK + 8;
  typedef Part<DK> PT;
  __shared__ __align__(16) E Kl[BC * SKE];
  __shared__ __align__(16) E Ql[BC * SKE];
  __shared__ float Tl[BC * ST], Pl[BC * ST], Dt[BC * ST], Zl[BC * ST], Sl[BC * ST], Rl[BC * ST];
  __shared__ float bs[BC], gs[BC], dGs[BC], dBs[BC], misc[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H, nb = p.dv / BVB;
  const long slot = blockIdx.x / H;
  const int h = blockIdx.x % H;
  // the sequence that owns the slot: the last n with floor(tok0_n / 64) + n <= slot
  auto tok_start = [&](int sq) -> long { return p.cu_seqlens ? (long)p.cu_seqlens[sq] : (long)sq * p.T; };
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((tok_start(mid) >> 6) + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  long tok0;
  int len;
  if (!seq_extent(p, lo, tok0, len)) return;
  const long c = slot - ((tok0 >> 6) + lo);
  if (c < 0 || 64 * c >= len) return;  // no chunk owns this slot
  const int nv = (int)min(64L, (long)len - 64 * c);
  const size_t tb = (size_t)tok0 + (size_t)c * BC;
  auto K_ = [&](int r, int d) { return to_f(Kl[r * SKE + d]); };
  auto Q_ = [&](int r, int d) { return to_f(Ql[r * SKE + d]); };

  // K, Q: 16-byte loads (rows past the sequence end are zero)
  constexpr int VE = 16 / (int)sizeof(E), NPC = BC * (DK / VE);  // 16-byte pieces
#pragma unroll
  for (int u = 0; u < (NPC + BNT - 1) / BNT; ++u) {
    const int pc = tid + BNT * u, r = pc / (DK / VE), g = pc % (DK / VE);
    if (pc >= NPC) break;
    u32x4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
    if (r < nv) {
      const size_t o = ((tb + r) * H + h) * DK + g * VE;
      kv = *(const u32x4 *)((const E *)p.k + o);
      qv = *(const u32x4 *)((const E *)p.q + o);
    }
    *(u32x4 *)(Kl + r * SKE + g * VE) = kv;
    *(u32x4 *)(Ql + r * SKE + g * VE) = qv;
  }
  // dP and dT summed over the value blocks in a fixed order, and T: 16-byte loads
  const float *pr0 = p.part + ((size_t)slot * H + h) * nb * (size_t)PT::SIZE;
  const float *tm = p.tmat + ((size_t)slot * H + h) * BC * BC;
#pragma unroll
  for (int u = 0; u < BC * BC / 4 / BNT; ++u) {
    // T is row-major; the partials are stored transposed (column i, rows r0 .. r0+3)
    const int i4 = 4 * (tid + BNT * u), r = i4 / BC, col = i4 % BC;
    f32x4 sp = zero4(), st = zero4(), tv = zero4();
    for (int b = 0; b < nb; ++b) {
      sp += *(const f32x4 *)(pr0 + (size_t)b * PT::SIZE + PT::DP + i4);
      if (!ADD) st += *(const f32x4 *)(pr0 + (size_t)b * PT::SIZE + PT::DT + i4);
    }
    if (!ADD) tv = *(const f32x4 *)(tm + i4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Pl[(col + e) * ST + r] = sp[e];
      if (!ADD) {  // no T for the additive write (its LDS then goes unused)
        Dt[(col + e) * ST + r] = st[e];
        Tl[r * ST + col + e] = tv[e];
      }
    }
  }
  if (tid < BC) {
    const bool ok = tid < nv;
    bs[tid] = (!ADD && ok) ? p.beta[(tb + tid) * H + h] : 0.f;
    gs[tid] = (GATE == GATE_HEAD && ok) ? p.log_alpha[(tb + tid) * p.la_stride + h] : 0.f;
    float sg = 0.f, sb = 0.f;
    for (int b = 0; b < nb; ++b) {
      sg += pr0[(size_t)b * PT::SIZE + PT::DG + tid];
      if (!ADD) sb += pr0[(size_t)b * PT::SIZE + PT::DB + tid];
    }
    dGs[tid] = sg;
    dBs[tid] = sb;
  }
  if (tid == 0) {
    float sc = 0.f;
    for (int b = 0; b < nb; ++b) sc += pr0[(size_t)b * PT::SIZE + PT::GC];
    misc[0] = sc;
  }
  __syncthreads();
  if (wave == 0) {
    float g = gs[lane];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(g, off);
      if (lane >= off) g += y;
    }
    gs[lane] = g;
  }
  __syncthreads();
  // S = K K^T, R = Q K^T (only their lower tiles are used: the upper ones are set to
  // zero);  Z = dT T^T
  for (int t = wave; t < 16; t += BNW) {
    const int m0 = (t >> 2) * 16, n0 = (t & 3) * 16;
    f32x4 sv = zero4(), rv = zero4();
    if (n0 <= m0) {
      if constexpr (std::is_same<E, bf16>::value) {  // bf16 rows read whole
        const E *kr = Kl + (m0 + lm) * SKE + 8 * lg, *qr = Ql + (m0 + lm) * SKE + 8 * lg;
        const E *kc = Kl + (n0 + lm) * SKE + 8 * lg;
        if (!ADD) sv = tile_frag<DK>([&](int k0) { return ld8(kr + k0); }, [&](int k0) { return ld8(kc + k0); });
        rv = tile_frag<DK>([&](int k0) { return ld8(qr + k0); }, [&](int k0) { return ld8(kc + k0); });
      } else {
        if (!ADD) sv = tile_g<E, DK, true, true>(m0, n0, lg, lm, K_, [&](int d, int i) { return K_(i, d); });
        rv = tile_g<E, DK, true, true>(m0, n0, lg, lm, Q_, [&](int d, int i) { return K_(i, d); });
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!ADD) Sl[(m0 + 4 * lg + u) * ST + n0 + lm] = sv[u];
      Rl[(m0 + 4 * lg + u) * ST + n0 + lm] = rv[u];
    }
    // T^T is upper triangular: T[i][k] = 0 for k > i (no T for the additive write)
    f32x4 zv = zero4();
    if (!ADD)
      zv = tile_g<E, BC, false, false>(m0, n0, lg, lm, [&](int r, int k) { return Dt[r * ST + k]; },
                                       [&](int k, int i) { return Tl[i * ST + k]; }, 0, n0 + 16);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (!ADD) Zl[(m0 + 4 * lg + u) * ST + n0 + lm] = zv[u];
  }
  __syncthreads();
  // dA = -strict(T^T Z), then per entry: Gamma, Ea = dA beta_r Gamma, Ep = dP Gamma,
  // wG = (dA beta_r S + dP R) Gamma, and dA S Gamma (for dbeta).  Each wave's tiles
  // are computed first (Zl is read), then written after a barrier.
  {
    f32x4 da[16 / BNW];
#pragma unroll
    for (int q = 0; q < 16 / BNW; ++q) {
      const int t = wave + BNW * q, m0 = (t >> 2) * 16, n0 = (t & 3) * 16;
      da[q] = zero4();  // only the strictly lower part is kept (none for the additive write)
      if (!ADD && n0 <= m0)
        da[q] = tile_g<E, BC, false, false>(m0, n0, lg, lm, [&](int r, int k) { return Tl[k * ST + r]; },
                                            [&](int k, int i) { return Zl[k * ST + i]; }, m0);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16 / BNW; ++q) {
      const int t = wave + BNW * q, m0 = (t >> 2) * 16, n0 = (t & 3) * 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = m0 + 4 * lg + u, i = n0 + lm;
        const float gam = i <= r ? (GATE == GATE_HEAD ? __expf(gs[r] - gs[i]) : 1.f) : 0.f;
        const float dA = i < r ? -da[q][u] : 0.f;
        const float dP = Pl[r * ST + i];
        const float S = ADD ? 0.f : Sl[r * ST + i], R = Rl[r * ST + i];
        Pl[r * ST + i] = dP * gam;  // Ep
        if (ADD) {
          Rl[r * ST + i] = dP * R * gam;  // wG, in place of R (the additive write needs no more)
        } else {
          Zl[r * ST + i] = dA * bs[r] * gam;                 // Ea
          Sl[r * ST + i] = (dA * bs[r] * S + dP * R) * gam;  // wG
          Rl[r * ST + i] = dA * S * gam;                     // dbeta terms
        }
      }
    }
  }
  __syncthreads();
  // row / column sums: dG and dbeta; then d log alpha = reverse prefix of dG (+ dG_C)
  if (tid < BC) {
    float rs = 0.f, cs = 0.f, bsum = 0.f;
    for (int i = 0; i < BC; ++i) {
      const float *Wl = ADD ? Rl : Sl;  // wG
      rs += Wl[tid * ST + i];
      cs += Wl[i * ST + tid];
      if (!ADD) bsum += Rl[tid * ST + i];
    }
    dGs[tid] += rs - cs + (tid == BC - 1 ? misc[0] : 0.f);
    dBs[tid] += bsum;
  }
  __syncthreads();
  if (wave == 0) {
    float g = dGs[BC - 1 - lane];  // suffix sums as a prefix over the reversed rows
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(g, off);
      if (lane >= off) g += y;
    }
    const int t = BC - 1 - lane;
    if (t < nv) {
      if (!ADD) p.dbeta[(tb + t) * H + h] = dBs[t];
      if (GATE == GATE_HEAD) p.dlog_alpha[(tb + t) * H + h] = g;
    }
  }
  // dq = Ep K + (partials), dk = (Ea + Ea^T) K + Ep^T Q + (partials); the partials of a
  // tile are loaded before its products, so the loads overlap them
  for (int t = wave; t < (DK / 16) * 4; t += BNW) {
    const int m0 = (t / (DK / 16)) * 16, n0 = (t % (DK / 16)) * 16;
    f32x4 pq_ = zero4(), pk_ = zero4();  // partials stored [d][r]: this lane's 4 rows are contiguous
    for (int b = 0; b < nb; ++b) {
      const size_t o = (size_t)b * PT::SIZE + (size_t)(n0 + lm) * BC + m0 + 4 * lg;
      pq_ += *(const f32x4 *)(pr0 + PT::DQ + o);
      pk_ += *(const f32x4 *)(pr0 + PT::DKO + o);
    }
    const f32x4 q_ = tile_g<E, BC, false, true>(m0, n0, lg, lm, [&](int r, int i) { return Pl[r * ST + i]; },
                                                [&](int i, int d) { return K_(i, d); }, 0, m0 + 16);
    f32x4 k_ = zero4();
    if (!ADD)
      k_ = tile_g<E, BC, false, true>(m0, n0, lg, lm, [&](int r, int i) { return Zl[r * ST + i] + Zl[i * ST + r]; },
                                      [&](int i, int d) { return K_(i, d); });
    k_ += tile_g<E, BC, false, true>(m0, n0, lg, lm, [&](int r, int i) { return Pl[i * ST + r]; },
                                     [&](int i, int d) { return Q_(i, d); }, m0);
    const int d = n0 + lm;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = m0 + 4 * lg + u;
      if (r >= nv) continue;
      ((E *)p.dq)[((tb + r) * H + h) * DK + d] = to_e<E>(q_[u] + pq_[u]);
      ((E *)p.dk)[((tb + r) * H + h) * DK + d] = to_e<E>(k_[u] + pk_[u]);
    }
  }
}

template <typename E, int DK, int GATE, bool ADD>
void launch_bg(const BwdParams &p, hipStream_t stream) {
  const int nb = p.dv / BVB;
  hipLaunchKernelGGL((bwd_prep_kernel<E, DK, GATE, ADD>), dim3((unsigned)(p.slots * p.H)), dim3(256), 0, stream, p);
  hipLaunchKernelGGL((bwd_state_kernel<E, DK, GATE, ADD>), dim3(p.N * p.H * nb), dim3(state_threads<ADD>()), 0,
                     stream, p);
  hipLaunchKernelGGL((bwd_chunk_kernel<E, DK, GATE, ADD>), dim3((unsigned)(p.slots * p.H)), dim3(BNT), 0, stream, p);
}

template <typename E, int DK>
hipError_t launch_b(const BwdParams &p, int gate, bool add, hipStream_t stream) {
  if (p.N == 0 || p.slots * p.H == 0) return hipSuccess;
  if (gate == GATE_HEAD)
    add ? launch_bg<E, DK, GATE_HEAD, true>(p, stream) : launch_bg<E, DK, GATE_HEAD, false>(p, stream);
  else if (gate == GATE_NONE)
    add ? launch_bg<E, DK, GATE_NONE, true>(p, stream) : launch_bg<E, DK, GATE_NONE, false>(p, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// out[h] = sum over t of x[t * H + h], in a fixed order (deterministic): one workgroup
// of 1024 threads per head, eight independent partial sums per thread (loads in
// flight together), then a tree in LDS.
__global__ __launch_bounds__(1024) void sum_tokens_kernel(const float *x, long tokens, int H, float *out) {
  __shared__ float part[1024];
  const int h = blockIdx.x, tid = threadIdx.x;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (long t0 = tid; t0 < tokens; t0 += 8 * 1024) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const long t = t0 + (long)u * 1024;
      if (t < tokens) acc[u] += x[t * H + h];
    }
  }
  part[tid] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) out[h] = part[0];
}

// x[0 .. n) = 0 (a kernel rather than a memset, so that graph capture records no
// memset node)
__global__ void fill_zero_kernel(float *x, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    x[i] = 0.f;
}

}  // namespace

size_t bwd_part_floats(int dk) { return dk == 128 ? Part<128>::SIZE : Part<64>::SIZE; }

hipError_t launch_fill_zero(float *x, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream, x, n);
  return hipGetLastError();
}

hipError_t launch_sum_tokens(const float *x, long tokens, int H, float *out, hipStream_t stream) {
  if (H <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_tokens_kernel, dim3(H), dim3(1024), 0, stream, x, tokens, H, out);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams &p, int dtype, int dk, int gate, bool add, hipStream_t stream) {
  if (dtype == 1) {
    if (dk == 128) return launch_b<bf16, 128>(p, gate, add, stream);
    if (dk == 64) return launch_b<bf16, 64>(p, gate, add, stream);
  } else {
    if (dk == 64) return launch_b<float, 64>(p, gate, add, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

// gdn_bwd.hip -- gradients of the chunked (gated) delta rule.
//
// Reverse mode through the chunk equations of the forward ("Decoding Hybrid Linear
// Attention Architectures", sec. 5; the WY / UT form of "Linear Attention Variants",
// DeltaNet section), for the delta write with no gate or one decay per (token, head).
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
// Three launches:
//  1. the fused forward with chunk-state output: every chunk's entering state M0;
//  2. bwd_state_kernel, one workgroup per (sequence, head, 32 value columns), walks the
//     chunks in reverse carrying dM: it writes dV, the entering-state gradient and T,
//     and per value block the partial sums of dP, dT, dQ, dK, dG, dbeta and dG_C
//     (the terms that sum over value columns);
//  3. bwd_chunk_kernel, one workgroup per (chunk, head), fully parallel: it sums the
//     partials in a fixed order (deterministic), forms dA and the Gram / Gamma terms
//     and writes dq, dk, dbeta and d log alpha.
// All arithmetic is fp32 (inputs in bf16 or fp32), on LDS tiles.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int BC = 64;    // chunk length
constexpr int BNT = 256;  // threads per workgroup
constexpr int BVB = 32;   // value columns per workgroup of the reverse-state kernel
constexpr int SV = BVB + 1, ST = BC + 1;  // fp32 row strides (padded)

// acc[TM][TN] += sum_k a(r, k) b(k, c) over this thread's TM x TN patch of an M x N
// product computed by NTH threads (thread t: rows (t / (N/TN)) TM.., columns (t % (N/TN)) TN..)
template <int M, int N, int K, int TM, int TN, int NTH, class FA, class FB>
__device__ __forceinline__ void mm(float (&acc)[TM][TN], int t, FA a, FB b) {
  static_assert(M * N == NTH * TM * TN && N % TN == 0 && M % TM == 0, "product tiling");
  const int r0 = (t / (N / TN)) * TM, c0 = (t % (N / TN)) * TN;
#pragma unroll 2
  for (int k = 0; k < K; ++k) {
    float av[TM], bv[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) av[i] = a(r0 + i, k);
#pragma unroll
    for (int j = 0; j < TN; ++j) bv[j] = b(k, c0 + j);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] += av[i] * bv[j];
  }
}
template <int N, int TM, int TN> __device__ __forceinline__ int tile_r0(int t) { return (t / (N / TN)) * TM; }
template <int N, int TN> __device__ __forceinline__ int tile_c0(int t) { return (t % (N / TN)) * TN; }
template <int TM, int TN> __device__ __forceinline__ void zero(float (&a)[TM][TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) a[i][j] = 0.f;
}

// floats of one partial record (per chunk slot, head and value block)
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

template <typename E, int DK, int GATE>
__global__ __launch_bounds__(BNT, 1) void bwd_state_kernel(BwdParams p) {
  constexpr int SKE = DK + 8;
  constexpr int TNK = DK / 16;  // 64 x DK products: 16 threads per row group
  typedef Part<DK> PT;
  __shared__ E Kl[BC * SKE], Ql[BC * SKE];
  __shared__ float Vb[BC * SV], dOb[BC * SV], M0[DK * SV], dM[DK * SV];
  __shared__ float Tl[BC * ST], Pl[BC * ST];
  __shared__ float Xl[BC * SV], Dl[BC * SV], dDl[BC * SV], Yl[BC * SV];
  __shared__ float bs[BC], gs[BC], eg[BC], et[BC], red[BC], wsum[4], misc[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = p.H, dv = p.dv, nb = dv / BVB;
  const int jb = blockIdx.x % nb, pair = blockIdx.x / nb;
  const int n = pair / H, h = pair % H, col0 = jb * BVB;
  long tok0;
  int len;
  if (!seq_extent(p, n, tok0, len)) return;
  const int nchunks = (len + BC - 1) / BC;
  const long slot0 = (tok0 >> 6) + n;
  const size_t sstate = ((size_t)n * H + h) * DK * dv + col0;

  for (int i = tid; i < DK * BVB; i += BNT) {
    const int d = i / BVB, j = i % BVB;
    dM[d * SV + j] = p.dfinal ? p.dfinal[sstate + (size_t)d * dv + j] : 0.f;
  }
  for (int c = nchunks - 1; c >= 0; --c) {
    const int nv = min(BC, len - c * BC);
    const size_t tb = (size_t)tok0 + (size_t)c * BC;  // token of row 0
    const size_t slot = (size_t)(slot0 + c);
    __syncthreads();  // the previous chunk is done with every buffer
    // ---- inputs of the chunk (rows past the sequence end are zero)
    for (int i = tid; i < BC * DK; i += BNT) {
      const int r = i / DK, d = i % DK;
      const size_t o = ((tb + r) * H + h) * DK + d;
      Kl[r * SKE + d] = r < nv ? ((const E *)p.k)[o] : to_e<E>(0.f);
      Ql[r * SKE + d] = r < nv ? ((const E *)p.q)[o] : to_e<E>(0.f);
    }
    for (int i = tid; i < BC * BVB; i += BNT) {
      const int r = i / BVB, j = i % BVB;
      const size_t o = ((tb + r) * H + h) * dv + col0 + j;
      Vb[r * SV + j] = r < nv ? to_f(((const E *)p.v)[o]) : 0.f;
      dOb[r * SV + j] = r < nv ? to_f(((const E *)p.dout)[o]) : 0.f;
    }
    for (int i = tid; i < DK * BVB; i += BNT) {
      const int d = i / BVB, j = i % BVB;
      M0[d * SV + j] = p.states[((slot * H + h) * DK + d) * dv + col0 + j];
    }
    if (tid < BC) {
      const bool ok = tid < nv;
      bs[tid] = ok ? p.beta[(tb + tid) * H + h] : 0.f;
      gs[tid] = (GATE == GATE_HEAD && ok) ? p.log_alpha[(tb + tid) * H + h] : 0.f;
    }
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
    // ---- A (strictly lower) into Tl and P (lower inclusive) into Pl
    {
      float aa[4][4], pp[4][4];
      zero(aa);
      zero(pp);
      mm<BC, BC, DK, 4, 4, BNT>(aa, tid, [&](int r, int d) { return to_f(Kl[r * SKE + d]); },
                                [&](int d, int i) { return to_f(Kl[i * SKE + d]); });
      mm<BC, BC, DK, 4, 4, BNT>(pp, tid, [&](int r, int d) { return to_f(Ql[r * SKE + d]); },
                                [&](int d, int i) { return to_f(Kl[i * SKE + d]); });
      const int r0 = tile_r0<BC, 4, 4>(tid), c0 = tile_c0<BC, 4>(tid);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = r0 + u, i = c0 + v;
          const float gam = i <= r ? (GATE == GATE_HEAD ? __expf(gs[r] - gs[i]) : 1.f) : 0.f;
          Tl[r * ST + i] = i < r ? bs[r] * aa[u][v] * gam : 0.f;
          Pl[r * ST + i] = pp[u][v] * gam;
        }
    }
    __syncthreads();
    if (wave == 0) {
      // T = (I + A)^-1 in place: lane owns column `lane`; row r of T needs A[r][i < r]
      // (read by every lane in the same step) and the column's earlier entries
      float x[BC];
#pragma unroll
      for (int r = 0; r < BC; ++r) {
        float acc = r == lane ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) acc -= Tl[r * ST + i] * x[i];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < BC; ++r) Tl[r * ST + lane] = x[r];
    } else if (wave < 3) {
      // V - Kt M0 into Xl (64 x 32, two waves)
      float xx[4][4];
      zero(xx);
      const int t = tid - 64;
      mm<BC, BVB, DK, 4, 4, 128>(xx, t, [&](int r, int d) { return to_f(Kl[r * SKE + d]); },
                                 [&](int d, int j) { return M0[d * SV + j]; });
      const int r0 = tile_r0<BVB, 4, 4>(t), c0 = tile_c0<BVB, 4>(t);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = r0 + u, j = c0 + v;
          Xl[r * SV + j] = Vb[r * SV + j] - eg[r] * xx[u][v];
        }
    }
    __syncthreads();
    if (jb == 0)  // T for the per-chunk kernel
      for (int i = tid; i < BC * BC; i += BNT) p.tmat[(slot * H + h) * BC * BC + i] = Tl[(i / BC) * ST + i % BC];
    // ---- Delta = T diag(beta) (V - Kt M0);  dDelta = P^T dO + diag(e^{G_C - G}) K dM
    {
      float dd[2][4], d1[2][4], d2[2][4];
      zero(dd);
      zero(d1);
      zero(d2);
      mm<BC, BVB, BC, 2, 4, BNT>(dd, tid, [&](int r, int i) { return Tl[r * ST + i]; },
                                 [&](int i, int j) { return bs[i] * Xl[i * SV + j]; });
      mm<BC, BVB, BC, 2, 4, BNT>(d1, tid, [&](int r, int i) { return Pl[i * ST + r]; },
                                 [&](int i, int j) { return dOb[i * SV + j]; });
      mm<BC, BVB, DK, 2, 4, BNT>(d2, tid, [&](int r, int d) { return to_f(Kl[r * SKE + d]); },
                                 [&](int d, int j) { return dM[d * SV + j]; });
      const int r0 = tile_r0<BVB, 2, 4>(tid), c0 = tile_c0<BVB, 4>(tid);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = r0 + u, j = c0 + v;
          Dl[r * SV + j] = dd[u][v];
          dDl[r * SV + j] = d1[u][v] + et[r] * d2[u][v];
        }
    }
    __syncthreads();
    // ---- Y = T^T dDelta
    {
      float yy[2][4];
      zero(yy);
      mm<BC, BVB, BC, 2, 4, BNT>(yy, tid, [&](int r, int i) { return Tl[i * ST + r]; },
                                 [&](int i, int j) { return dDl[i * SV + j]; });
      const int r0 = tile_r0<BVB, 2, 4>(tid), c0 = tile_c0<BVB, 4>(tid);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) Yl[(r0 + u) * SV + c0 + v] = yy[u][v];
    }
    __syncthreads();
    // ---- dV (complete for this value block)
    for (int i = tid; i < BC * BVB; i += BNT) {
      const int r = i / BVB, j = i % BVB;
      if (r < nv) ((E *)p.dv_out)[((tb + r) * H + h) * dv + col0 + j] = to_e<E>(bs[r] * Yl[r * SV + j]);
    }
    float *pr = p.part + ((slot * H + h) * nb + jb) * (size_t)PT::SIZE;
    // ---- dP = incl(dO Delta^T), dT = dDelta (diag(beta) X)^T  (partial over value columns)
    {
      float ap[4][4], at[4][4];
      zero(ap);
      zero(at);
      mm<BC, BC, BVB, 4, 4, BNT>(ap, tid, [&](int r, int j) { return dOb[r * SV + j]; },
                                 [&](int j, int i) { return Dl[i * SV + j]; });
      mm<BC, BC, BVB, 4, 4, BNT>(at, tid, [&](int r, int j) { return dDl[r * SV + j]; },
                                 [&](int j, int i) { return bs[i] * Xl[i * SV + j]; });
      const int r0 = tile_r0<BC, 4, 4>(tid), c0 = tile_c0<BC, 4>(tid);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = r0 + u, i = c0 + v;
          pr[PT::DP + r * BC + i] = i <= r ? ap[u][v] : 0.f;
          pr[PT::DT + r * BC + i] = at[u][v];
        }
    }
    // ---- dQ = e^G dO M0^T, dK = -e^G beta Y M0^T + e^{G_C - G} Delta dM^T, and the row
    // sums of dG: e^G (dO M0^T).Q - e^G beta (Y M0^T).K - e^{G_C - G} (Delta dM^T).K
    {
      float w[4][TNK], uu[4][TNK], z[4][TNK];
      zero(w);
      zero(uu);
      zero(z);
      mm<BC, DK, BVB, 4, TNK, BNT>(w, tid, [&](int r, int j) { return dOb[r * SV + j]; },
                                   [&](int j, int d) { return M0[d * SV + j]; });
      mm<BC, DK, BVB, 4, TNK, BNT>(uu, tid, [&](int r, int j) { return Yl[r * SV + j]; },
                                   [&](int j, int d) { return M0[d * SV + j]; });
      mm<BC, DK, BVB, 4, TNK, BNT>(z, tid, [&](int r, int j) { return Dl[r * SV + j]; },
                                   [&](int j, int d) { return dM[d * SV + j]; });
      const int r0 = tile_r0<DK, 4, TNK>(tid), c0 = tile_c0<DK, TNK>(tid);
      float gq[4], gk[4], gz[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u;
        gq[u] = gk[u] = gz[u] = 0.f;
#pragma unroll
        for (int v = 0; v < TNK; ++v) {
          const int d = c0 + v;
          const float qv = to_f(Ql[r * SKE + d]), kv = to_f(Kl[r * SKE + d]);
          pr[PT::DQ + r * DK + d] = eg[r] * w[u][v];
          pr[PT::DKO + r * DK + d] = -eg[r] * bs[r] * uu[u][v] + et[r] * z[u][v];
          gq[u] += w[u][v] * qv;
          gk[u] += uu[u][v] * kv;
          gz[u] += z[u][v] * kv;
        }
      }
      // a row group's 16 threads are 16 consecutive lanes
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          gq[u] += __shfl_xor(gq[u], off);
          gk[u] += __shfl_xor(gk[u], off);
          gz[u] += __shfl_xor(gz[u], off);
        }
      if ((lane & 15) == 0)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = r0 + u;
          pr[PT::DG + r] = eg[r] * gq[u] - eg[r] * bs[r] * gk[u] - et[r] * gz[u];
          red[r] = et[r] * gz[u];  // this row's term of dG_C
        }
    }
    // ---- dbeta rows: Y . (V - Kt M0);  dG_C: the e^{G_C - G} terms plus gam <M0, dM>
    float part_m = 0.f;
    for (int i = tid; i < DK * BVB; i += BNT) part_m += M0[(i / BVB) * SV + i % BVB] * dM[(i / BVB) * SV + i % BVB];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part_m += __shfl_xor(part_m, off);
    if (lane == 0) wsum[wave] = part_m;
    if (tid < BC) {
      float s = 0.f;
      for (int j = 0; j < BVB; ++j) s += Yl[tid * SV + j] * Xl[tid * SV + j];
      pr[PT::DB + tid] = s;
    }
    __syncthreads();
    if (wave == 0) {
      float s = red[lane];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) pr[PT::GC] = s + misc[0] * (wsum[0] + wsum[1] + wsum[2] + wsum[3]);
    }
    // ---- dM <- gam dM + Qt^T dO - Kt^T diag(beta) Y   (DK x 32)
    {
      constexpr int TMD = DK / 32;
      float n1[TMD][4], n2[TMD][4];
      zero(n1);
      zero(n2);
      mm<DK, BVB, BC, TMD, 4, BNT>(n1, tid, [&](int d, int r) { return eg[r] * to_f(Ql[r * SKE + d]); },
                                   [&](int r, int j) { return dOb[r * SV + j]; });
      mm<DK, BVB, BC, TMD, 4, BNT>(n2, tid, [&](int d, int r) { return eg[r] * bs[r] * to_f(Kl[r * SKE + d]); },
                                   [&](int r, int j) { return Yl[r * SV + j]; });
      const int r0 = tile_r0<BVB, TMD, 4>(tid), c0 = tile_c0<BVB, 4>(tid);
      const float gam = misc[0];
      float nm[TMD][4];
#pragma unroll
      for (int u = 0; u < TMD; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) nm[u][v] = gam * dM[(r0 + u) * SV + c0 + v] + n1[u][v] - n2[u][v];
      __syncthreads();  // every read of the old dM is done
#pragma unroll
      for (int u = 0; u < TMD; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) dM[(r0 + u) * SV + c0 + v] = nm[u][v];
    }
  }
  __syncthreads();
  if (p.dinit)
    for (int i = tid; i < DK * BVB; i += BNT) {
      const int d = i / BVB, j = i % BVB;
      p.dinit[sstate + (size_t)d * dv + j] = dM[d * SV + j];
    }
}

template <typename E, int DK, int GATE>
__global__ __launch_bounds__(BNT, 1) void bwd_chunk_kernel(BwdParams p) {
  constexpr int SKE = DK + 8;
  constexpr int TNK = DK / 16;
  typedef Part<DK> PT;
  __shared__ E Kl[BC * SKE], Ql[BC * SKE];
  __shared__ float Tl[BC * ST], Pl[BC * ST], Dt[BC * ST], Zl[BC * ST], Sl[BC * ST], Rl[BC * ST];
  __shared__ float bs[BC], gs[BC], dGs[BC], dBs[BC], misc[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  for (int i = tid; i < BC * DK; i += BNT) {
    const int r = i / DK, d = i % DK;
    const size_t o = ((tb + r) * H + h) * DK + d;
    Kl[r * SKE + d] = r < nv ? ((const E *)p.k)[o] : to_e<E>(0.f);
    Ql[r * SKE + d] = r < nv ? ((const E *)p.q)[o] : to_e<E>(0.f);
  }
  const float *pr0 = p.part + ((size_t)slot * H + h) * nb * (size_t)PT::SIZE;
  for (int i = tid; i < BC * BC; i += BNT) {
    const int r = i / BC, col = i % BC;
    float sp = 0.f, st = 0.f;
    for (int b = 0; b < nb; ++b) {
      sp += pr0[(size_t)b * PT::SIZE + PT::DP + i];
      st += pr0[(size_t)b * PT::SIZE + PT::DT + i];
    }
    Pl[r * ST + col] = sp;
    Dt[r * ST + col] = st;
    Tl[r * ST + col] = p.tmat[((size_t)slot * H + h) * BC * BC + i];
  }
  if (tid < BC) {
    const bool ok = tid < nv;
    bs[tid] = ok ? p.beta[(tb + tid) * H + h] : 0.f;
    gs[tid] = (GATE == GATE_HEAD && ok) ? p.log_alpha[(tb + tid) * H + h] : 0.f;
    float sg = 0.f, sb = 0.f;
    for (int b = 0; b < nb; ++b) {
      sg += pr0[(size_t)b * PT::SIZE + PT::DG + tid];
      sb += pr0[(size_t)b * PT::SIZE + PT::DB + tid];
    }
    dGs[tid] = sg;
    dBs[tid] = sb;
  }
  if (tid == 0) {
    float s = 0.f;
    for (int b = 0; b < nb; ++b) s += pr0[(size_t)b * PT::SIZE + PT::GC];
    misc[0] = s;
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
  // S = K K^T, R = Q K^T;  Z = dT T^T
  {
    float s_[4][4], r_[4][4], z_[4][4];
    zero(s_);
    zero(r_);
    zero(z_);
    mm<BC, BC, DK, 4, 4, BNT>(s_, tid, [&](int r, int d) { return to_f(Kl[r * SKE + d]); },
                              [&](int d, int i) { return to_f(Kl[i * SKE + d]); });
    mm<BC, BC, DK, 4, 4, BNT>(r_, tid, [&](int r, int d) { return to_f(Ql[r * SKE + d]); },
                              [&](int d, int i) { return to_f(Kl[i * SKE + d]); });
    mm<BC, BC, BC, 4, 4, BNT>(z_, tid, [&](int r, int k) { return Dt[r * ST + k]; },
                              [&](int k, int i) { return Tl[i * ST + k]; });
    const int r0 = tile_r0<BC, 4, 4>(tid), c0 = tile_c0<BC, 4>(tid);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = r0 + u, i = c0 + v;
        Sl[r * ST + i] = s_[u][v];
        Rl[r * ST + i] = r_[u][v];
        Zl[r * ST + i] = z_[u][v];
      }
  }
  __syncthreads();
  // dA = -strict(T^T Z), then per entry: Gamma, Ea = dA beta_r Gamma, Ep = dP Gamma,
  // wG = (dA beta_r S + dP R) Gamma, and dA S Gamma (for dbeta)
  {
    float a_[4][4];
    zero(a_);
    mm<BC, BC, BC, 4, 4, BNT>(a_, tid, [&](int r, int k) { return Tl[k * ST + r]; },
                              [&](int k, int i) { return Zl[k * ST + i]; });
    const int r0 = tile_r0<BC, 4, 4>(tid), c0 = tile_c0<BC, 4>(tid);
    __syncthreads();  // Zl is rewritten below
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = r0 + u, i = c0 + v;
        const float gam = i <= r ? (GATE == GATE_HEAD ? __expf(gs[r] - gs[i]) : 1.f) : 0.f;
        const float dA = i < r ? -a_[u][v] : 0.f;
        const float dP = Pl[r * ST + i];
        const float S = Sl[r * ST + i], R = Rl[r * ST + i];
        Zl[r * ST + i] = dA * bs[r] * gam;            // Ea
        Pl[r * ST + i] = dP * gam;                    // Ep
        Sl[r * ST + i] = (dA * bs[r] * S + dP * R) * gam;  // wG
        Rl[r * ST + i] = dA * S * gam;                // dbeta terms
      }
  }
  __syncthreads();
  // row / column sums: dG and dbeta; then d log alpha = reverse prefix of dG (+ dG_C)
  if (tid < BC) {
    float rs = 0.f, cs = 0.f, bsum = 0.f;
    for (int i = 0; i < BC; ++i) {
      rs += Sl[tid * ST + i];
      cs += Sl[i * ST + tid];
      bsum += Rl[tid * ST + i];
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
      p.dbeta[(tb + t) * H + h] = dBs[t];
      if (GATE == GATE_HEAD) p.dlog_alpha[(tb + t) * H + h] = g;
    }
  }
  // dq = Ep K + (partials), dk = (Ea + Ea^T) K + Ep^T Q + (partials)
  {
    float q_[4][TNK], k_[4][TNK];
    zero(q_);
    zero(k_);
    mm<BC, DK, BC, 4, TNK, BNT>(q_, tid, [&](int r, int i) { return Pl[r * ST + i]; },
                                [&](int i, int d) { return to_f(Kl[i * SKE + d]); });
    mm<BC, DK, BC, 4, TNK, BNT>(k_, tid, [&](int r, int i) { return Zl[r * ST + i] + Zl[i * ST + r]; },
                                [&](int i, int d) { return to_f(Kl[i * SKE + d]); });
    mm<BC, DK, BC, 4, TNK, BNT>(k_, tid, [&](int r, int i) { return Pl[i * ST + r]; },
                                [&](int i, int d) { return to_f(Ql[i * SKE + d]); });
    const int r0 = tile_r0<DK, 4, TNK>(tid), c0 = tile_c0<DK, TNK>(tid);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = r0 + u;
      if (r >= nv) continue;
#pragma unroll
      for (int v = 0; v < TNK; ++v) {
        const int d = c0 + v;
        float sq = q_[u][v], sk = k_[u][v];
        for (int b = 0; b < nb; ++b) {
          sq += pr0[(size_t)b * PT::SIZE + PT::DQ + r * DK + d];
          sk += pr0[(size_t)b * PT::SIZE + PT::DKO + r * DK + d];
        }
        ((E *)p.dq)[((tb + r) * H + h) * DK + d] = to_e<E>(sq);
        ((E *)p.dk)[((tb + r) * H + h) * DK + d] = to_e<E>(sk);
      }
    }
  }
}

template <typename E, int DK>
hipError_t launch_b(const BwdParams &p, int gate, hipStream_t stream) {
  const int nb = p.dv / BVB;
  const long items = p.slots * p.H;
  if (p.N == 0 || items == 0) return hipSuccess;
  if (gate == GATE_HEAD) {
    hipLaunchKernelGGL((bwd_state_kernel<E, DK, GATE_HEAD>), dim3(p.N * p.H * nb), dim3(BNT), 0, stream, p);
    hipLaunchKernelGGL((bwd_chunk_kernel<E, DK, GATE_HEAD>), dim3((unsigned)items), dim3(BNT), 0, stream, p);
  } else if (gate == GATE_NONE) {
    hipLaunchKernelGGL((bwd_state_kernel<E, DK, GATE_NONE>), dim3(p.N * p.H * nb), dim3(BNT), 0, stream, p);
    hipLaunchKernelGGL((bwd_chunk_kernel<E, DK, GATE_NONE>), dim3((unsigned)items), dim3(BNT), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t bwd_part_floats(int dk) { return dk == 128 ? Part<128>::SIZE : Part<64>::SIZE; }

hipError_t launch_bwd(const BwdParams &p, int dtype, int dk, int gate, hipStream_t stream) {
  if (dtype == 1) {
    if (dk == 128) return launch_b<bf16, 128>(p, gate, stream);
    if (dk == 64) return launch_b<bf16, 64>(p, gate, stream);
  } else {
    if (dk == 64) return launch_b<float, 64>(p, gate, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

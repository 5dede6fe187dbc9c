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
// Four launches, everything in between in the caller's workspace (fp32):
//  1. a forward that stores every chunk's entering state M0 instead of o: the
//     pipelined kernel's STATES variant for bf16 with d_k = 128, the fused kernel
//     otherwise;
//  2. bwd_prep_kernel, one workgroup per (chunk, head), fully parallel: T, T^T and P^T of
//     every chunk, and the other operands of the reverse pass (Q^T, K^T, e^G and e^{G_C -
//     G} per row, gam);
//  3. the reverse state pass of the per-key-channel gradients in its scalar-gate form
//     (launch_bwdk_rev): one workgroup per (sequence, head, value block) walks the chunks
//     in reverse with dM in matrix-core accumulators and writes dM and dDelta of every
//     chunk, dV and the initial-state gradient;
//  4. bwd_chunk_kernel, one workgroup per (chunk, head), fully parallel: every product
//     over the value columns at full width (X, Delta, Y, dP, dT, dQt, dKt, dKh) from the
//     stored M0, dM and dDelta, 32 columns at a time, then dA, the Gram and Gamma terms,
//     dq, dk, dbeta and d log alpha.  Nothing sums across workgroups: the result is
//     deterministic.
// All arithmetic is fp32 or its equivalent (inputs in bf16 or fp32).  The products run
// on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16): an operand whose values are bf16
// inputs (q, k, v, dO) is taken exactly, any other (and every fp32 input) is split into
// a hi + lo pair of bf16 terms (about 2^-17 relative error per product).  The Gram and
// Gamma phase of the per-chunk kernel runs on v_mfma_f32_16x16x4f32 for fp32 I/O.
#include "gdn_common.h"
#include "gdn_kernels.h"
#include "gdn_tile.h"
#include "gdn_bwd_slices.h"

namespace gdn {

namespace {

constexpr int BC = 64;      // chunk length
constexpr int ST = BC + 1;  // fp32 pitch of 64-column tiles

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

// decay prefix of a chunk (wave 0, lane = row): gs <- G, eg <- e^G, et <- e^{G_C - G},
// *gC <- e^{G_C}
__device__ __forceinline__ void decay_prefix(float *gs, float *eg, float *et, float *gC, int lane) {
  float g = gs[lane];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(g, off);
    if (lane >= off) g += y;
  }
  const float gc = __shfl(g, 63);
  gs[lane] = g;
  eg[lane] = __expf(g);
  et[lane] = __expf(gc - g);
  if (lane == 0) *gC = __expf(gc);
}

// One workgroup per (chunk slot, head), fully parallel: P = incl(Q K^T * Gamma) and, for
// the delta write, T = (I + A)^-1 with A = strict(diag(beta) K K^T * Gamma) (blocked
// inverse, tri_inv64); into the workspace P^T, T, T^T, and for the reverse pass Q^T, K^T
// (channel-major copies of the inputs), e^G and e^{G_C - G} per row and gam = e^{G_C}
// repeated over the key channels.  The Gram tiles take the bf16 inputs exactly.
template <typename E, int DK, int GATE, bool ADD>
__global__ __launch_bounds__(256, 2) void bwd_prep_kernel(BwdParams p) {
  constexpr int SKE = DK + 8;
  __shared__ __align__(16) E Kl[BC * SKE];
  __shared__ __align__(16) E Ql[BC * SKE];
  __shared__ float Al[BC * ST], Tl[BC * ST];
  __shared__ float ys[3 * 16 * 17];
  __shared__ float bs[BC], gs[BC], eg[BC], et[BC], gcs[1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H;
  const long slot = blockIdx.x / H;
  const int h = blockIdx.x % H;
  size_t tb;
  int nv;
  if (!slot_chunk(p, slot, tb, nv)) return;
  const size_t sh = (size_t)slot * H + h;
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
  if (wave == 0) decay_prefix(gs, eg, et, gcs, lane);
  __syncthreads();
  // Gram tiles: P^T straight to the workspace (a lane's four rows of a tile are four
  // consecutive floats of the transpose), A into LDS
  float *pmT = p.pmT + sh * BC * BC;
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
    f32x4 pt;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = m0 + 4 * lg + u, i = n0 + lm;
      const float gam = i <= r ? (GATE == GATE_HEAD ? __expf(gs[r] - gs[i]) : 1.f) : 0.f;
      if (!ADD) Al[r * ST + i] = i < r ? bs[r] * av[u] * gam : 0.f;
      pt[u] = pv[u] * gam;
    }
    *(f32x4 *)(pmT + (n0 + lm) * BC + m0 + 4 * lg) = pt;
  }
  // Q^T and K^T (channel-major, the I/O dtype; 8 consecutive rows per thread), the row
  // factors e^G and e^{G_C - G} (0 past the sequence end) and gam
  for (int i = 8 * tid; i < DK * BC; i += 8 * 256) {
    const int d = i / BC, r = i % BC;
    E q8[8], k8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      q8[e] = Ql[(r + e) * SKE + d];
      k8[e] = Kl[(r + e) * SKE + d];
    }
    E *qt = (E *)p.qT + sh * DK * BC + i, *kt = (E *)p.kT + sh * DK * BC + i;
#pragma unroll
    for (int e = 0; e < 8; e += 16 / (int)sizeof(E)) {
      u32x4 wq, wk;
      __builtin_memcpy(&wq, q8 + e, 16);
      __builtin_memcpy(&wk, k8 + e, 16);
      *(u32x4 *)(qt + e) = wq;
      if (!ADD) *(u32x4 *)(kt + e) = wk;
    }
  }
  if (tid < BC) {
    p.egr[sh * BC + tid] = tid < nv ? eg[tid] : 0.f;
    p.etr[sh * BC + tid] = tid < nv ? et[tid] : 0.f;
  }
  if (tid < DK) p.gam[sh * DK + tid] = gcs[0];
  if constexpr (!ADD) {
    __syncthreads();
    tri_inv64<1>(Al, ST, Tl, ST, ys);
    float *tm = p.tm + sh * BC * BC, *tmT = p.tmT + sh * BC * BC;
    for (int i4 = 4 * tid; i4 < BC * BC; i4 += 4 * 256) {
      const int r = i4 / BC, i = i4 % BC;
      *(f32x4 *)(tm + i4) = (f32x4){Tl[r * ST + i], Tl[r * ST + i + 1], Tl[r * ST + i + 2], Tl[r * ST + i + 3]};
      *(f32x4 *)(tmT + i4) =
          (f32x4){Tl[i * ST + r], Tl[(i + 1) * ST + r], Tl[(i + 2) * ST + r], Tl[(i + 3) * ST + r]};
    }
  }
}

// One workgroup of eight waves per (chunk slot, head), fully parallel.
// First part, 32 value columns at a time (the slice of M0, dM, dDelta, dO and V staged
// in LDS, the next slice's loads in flight meanwhile):
//   X = V - e^G (K M0), Delta = T diag(beta) X, Y = T^T dDelta,
//   dP += dO Delta^T, dT += dDelta (diag(beta) X)^T,
//   dQt += dO M0^T, dKt -= diag(beta) Y M0^T, dKh += Delta dM^T,
//   dbeta_r += Y_r . X_r, <M0, dM>;
// the sums stay in matrix-core accumulators.  Every B operand and every computed A
// operand is staged once per slice as split bf16 halves in the layout its fragments
// read (two 16-byte reads); K and dO are taken exactly.
// Second part: dA = -strict(T^T dT T^T), the Gram and Gamma terms, dq, dk, dbeta and
// d log alpha (the reverse prefix of dG plus dG_C).
template <typename E, int DK, int GATE, bool ADD>
__global__ __launch_bounds__(512, 1) void bwd_chunk_kernel(BwdParams p) {
  constexpr int NT = 512, NW = 8, PK = DK + 8, SKE = PK;
  // the second part's LDS (Q and six fp32 64 x 64 tiles) shares U with the first's
  constexpr int B_BYTES = BC * PK * (int)sizeof(E) + 6 * BC * ST * 4, A_BYTES = SliceLds<E, DK, ADD>::BYTES;
  __shared__ __align__(16) E Kl[BC * PK];
  __shared__ __align__(16) char U[A_BYTES > B_BYTES ? A_BYTES : B_BYTES];
  __shared__ float bs[BC], gs[BC], eg[BC], et[BC], dGs[BC], dBs[BC], misc[4];
  __shared__ float rq[2][3][BC], dbp[2][BC], wsum[NW], rsp[2][NW][BC];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, lm = lane & 15;
  const int H = p.H, dv = p.dv;
  const long slot = blockIdx.x / H;
  const int h = blockIdx.x % H;
  size_t tb;
  int nv;
  if (!slot_chunk(p, slot, tb, nv)) return;
  const size_t sh = (size_t)slot * H + h;
  auto K_ = [&](int r, int d) { return to_f(Kl[r * PK + d]); };

  {  // K (16-byte loads, rows past the end zero), beta and the decay prefix
    constexpr int VE = 16 / (int)sizeof(E), NPC = BC * (DK / VE);
#pragma unroll
    for (int q = 0; q < (NPC + NT - 1) / NT; ++q) {
      const int pc = tid + NT * q, r = pc / (DK / VE), g = pc % (DK / VE);
      if (pc >= NPC) break;
      u32x4 kv = {0u, 0u, 0u, 0u};
      if (r < nv) kv = *(const u32x4 *)((const E *)p.k + ((tb + r) * H + h) * DK + g * VE);
      *(u32x4 *)(Kl + r * PK + g * VE) = kv;
    }
    if (tid < BC) {
      const bool ok = tid < nv;
      bs[tid] = (!ADD && ok) ? p.beta[(tb + tid) * H + h] : 0.f;
      gs[tid] = (GATE == GATE_HEAD && ok) ? p.log_alpha[(tb + tid) * p.la_stride + h] : 0.f;
    }
    __syncthreads();
    if (wave == 0) decay_prefix(gs, eg, et, misc + 1, lane);
  }

  // ---- first part: the sums over the value columns
  constexpr int NCT = DK / 32;
  const int a = wave >> 1, ct = wave & 1, wa = wave & 3, wc = wave >> 2;
  SliceSums<DK> S;
  {
    SliceIn in;
    in.st = p.states + sh * DK * dv;
    in.dmc = p.dmc + sh * DK * dv;
    in.dd = p.dd + sh * BC * dv;
    in.tm = p.tm + sh * BC * BC;
    in.tmT = p.tmT + sh * BC * BC;
    in.kt = nullptr;
    in.v = p.v;
    in.dout = p.dout;
    in.tb = tb;
    in.nv = nv;
    in.H = H;
    in.h = h;
    in.dv = dv;
    slice_sums<E, DK, ADD, false>(in, U, Kl, eg, bs, S);
  }
  f32x4 *const aP = S.aP, *const aT = S.aT, *const aQ = S.aQ, *const aK = S.aK, *const aH = S.aH;
  f32x4 dby = S.dby;
  float dgm = 0.f;
#pragma unroll
  for (int q = 0; q < SliceSums<DK>::NM; ++q) dgm += S.dgm[q];

  // ---- second part's LDS
  E *const Ql = (E *)U;
  float *const Tl = (float *)(U + BC * PK * sizeof(E));
  float *const Pl = Tl + BC * ST, *const Dt = Pl + BC * ST, *const Zl = Dt + BC * ST, *const Sl = Zl + BC * ST,
               *const Rl = Sl + BC * ST;
  auto Q_ = [&](int r, int d) { return to_f(Ql[r * PK + d]); };
  {  // Q and T, and dP (inclusive lower) / dT from the accumulators
    constexpr int VE = 16 / (int)sizeof(E), NPC = BC * (DK / VE);
#pragma unroll
    for (int q = 0; q < (NPC + NT - 1) / NT; ++q) {
      const int pc = tid + NT * q, r = pc / (DK / VE), g = pc % (DK / VE);
      if (pc >= NPC) break;
      u32x4 qv = {0u, 0u, 0u, 0u};
      if (r < nv) qv = *(const u32x4 *)((const E *)p.q + ((tb + r) * H + h) * DK + g * VE);
      *(u32x4 *)(Ql + r * PK + g * VE) = qv;
    }
    if constexpr (!ADD) {
      const float *tm = p.tm + sh * BC * BC;
      for (int i4 = 4 * tid; i4 < BC * BC; i4 += 4 * NT) {
        const f32x4 tv = *(const f32x4 *)(tm + i4);
        const int r = i4 / BC, c = i4 % BC;
#pragma unroll
        for (int e = 0; e < 4; ++e) Tl[r * ST + c + e] = tv[e];
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int t = wave + 8 * q, m0 = 16 * (t >> 2), n0 = 16 * (t & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = m0 + 4 * lg + j, i = n0 + lm;
        Pl[r * ST + i] = i <= r ? aP[q][j] : 0.f;
        if (!ADD) Dt[r * ST + i] = aT[q][j];
      }
    }
  }
  // <M0, dM> over the workgroup
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dgm += __shfl_xor(dgm, off);
  if (lane == 0) wsum[wave] = dgm;
  // dbeta rows: Y . X over the tile's 16 columns, the two column tiles meet in LDS
  if constexpr (!ADD) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) dby[j] += __shfl_xor(dby[j], off);
    if (lm == 0)
#pragma unroll
      for (int j = 0; j < 4; ++j) dbp[ct][16 * a + 4 * lg + j] = dby[j];
  }
  __syncthreads();
  {  // the rows of dG from the value-width sums: dQt . Q, dKt . K, dKh . K
    float gq[4] = {0.f, 0.f, 0.f, 0.f}, gk[4] = {0.f, 0.f, 0.f, 0.f}, gz[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NCT; ++q) {
      const int c = 16 * (wc + 2 * q) + lm;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * wa + 4 * lg + j;
        gq[j] += aQ[q][j] * Q_(r, c);
        gk[j] += aK[q][j] * K_(r, c);
        gz[j] += aH[q][j] * K_(r, c);
      }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gq[j] += __shfl_xor(gq[j], off);
        gk[j] += __shfl_xor(gk[j], off);
        gz[j] += __shfl_xor(gz[j], off);
      }
    if (lm == 0)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * wa + 4 * lg + j;
        rq[wc][0][r] = gq[j];
        rq[wc][1][r] = gk[j];
        rq[wc][2][r] = gz[j];
      }
  }
  __syncthreads();
  if (wave == 0) {  // lane = row: dG and dbeta rows, and dG_C = sum of e^{G_C - G} dKh . K + gam <M0, dM>
    const int r = lane;
    const float gq = rq[0][0][r] + rq[1][0][r], gk = rq[0][1][r] + rq[1][1][r], gz = rq[0][2][r] + rq[1][2][r];
    dGs[r] = eg[r] * (gq + gk) - et[r] * gz;
    dBs[r] = ADD ? 0.f : dbp[0][r] + dbp[1][r];
    float sg = et[r] * gz;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sg += __shfl_xor(sg, off);
    float wm = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) wm += wsum[w];
    if (lane == 0) misc[0] = sg + misc[1] * wm;
  }
  __syncthreads();
  // S = K K^T, R = Q K^T (only their lower tiles are used: the upper ones are set to
  // zero);  Z = dT T^T
  for (int t = wave; t < 16; t += NW) {
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
    f32x4 da[16 / NW];
#pragma unroll
    for (int q = 0; q < 16 / NW; ++q) {
      const int t = wave + NW * q, m0 = (t >> 2) * 16, n0 = (t & 3) * 16;
      da[q] = zero4();  // only the strictly lower part is kept (none for the additive write)
      if (!ADD && n0 <= m0)
        da[q] = tile_g<E, BC, false, false>(m0, n0, lg, lm, [&](int r, int k) { return Tl[k * ST + r]; },
                                            [&](int k, int i) { return Zl[k * ST + i]; }, m0);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16 / NW; ++q) {
      const int t = wave + NW * q, m0 = (t >> 2) * 16, n0 = (t & 3) * 16;
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
  // row / column sums: dG and dbeta (eight parts of eight columns, then the parts in a
  // fixed order); then d log alpha = reverse prefix of dG (+ dG_C)
  {
    const int r = tid & (BC - 1), part = tid >> 6;
    const float *Wl = ADD ? Rl : Sl;  // wG
    float rs = 0.f, cs = 0.f, bsum = 0.f;
#pragma unroll
    for (int i = 8 * part; i < 8 * part + 8; ++i) {
      rs += Wl[r * ST + i];
      cs += Wl[i * ST + r];
      if (!ADD) bsum += Rl[r * ST + i];
    }
    rsp[0][part][r] = rs - cs;
    rsp[1][part][r] = bsum;
  }
  __syncthreads();
  if (tid < BC) {
    float g = 0.f, b = 0.f;
#pragma unroll
    for (int part = 0; part < NW; ++part) {
      g += rsp[0][part][tid];
      b += rsp[1][part][tid];
    }
    dGs[tid] += g + (tid == BC - 1 ? misc[0] : 0.f);
    dBs[tid] += b;
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
  // dq = Ep K + e^G dQt, dk = (Ea + Ea^T) K + Ep^T Q + e^G dKt + e^{G_C - G} dKh: the
  // tiles whose value-width sums this wave holds
#pragma unroll
  for (int q = 0; q < NCT; ++q) {
    const int m0 = 16 * wa, n0 = 16 * (wc + 2 * q);
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
    for (int j = 0; j < 4; ++j) {
      const int r = m0 + 4 * lg + j;
      if (r >= nv) continue;
      ((E *)p.dq)[((tb + r) * H + h) * DK + d] = to_e<E>(q_[j] + eg[r] * aQ[q][j]);
      ((E *)p.dk)[((tb + r) * H + h) * DK + d] = to_e<E>(k_[j] + eg[r] * aK[q][j] + et[r] * aH[q][j]);
    }
  }
}

template <typename E, int DK, int GATE, bool ADD>
hipError_t launch_bg(const BwdParams &p, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_prep_kernel<E, DK, GATE, ADD>), dim3((unsigned)(p.slots * p.H)), dim3(256), 0, stream, p);
  BwdKeyParams kp{};
  kp.q = p.q;
  kp.k = p.k;
  kp.v = p.v;
  kp.dout = p.dout;
  kp.beta = p.beta;
  kp.dfinal = p.dfinal;
  kp.cu_seqlens = p.cu_seqlens;
  kp.states = const_cast<float *>(p.states);
  kp.dmc = p.dmc;
  kp.dd = p.dd;
  kp.tmT = p.tmT;
  kp.pmT = p.pmT;
  kp.qT = p.qT;
  kp.kT = p.kT;
  kp.egr = p.egr;
  kp.etr = p.etr;
  kp.gam = p.gam;
  kp.dv_out = p.dv_out;
  kp.dinit = p.dinit;
  kp.N = p.N;
  kp.H = p.H;
  kp.T = p.T;
  kp.dv = p.dv;
  kp.slots = p.slots;
  kp.states_ready = 1;
  const hipError_t e = launch_bwdk_rev(kp, std::is_same<E, bf16>::value ? 1 : 0, DK, ADD, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_chunk_kernel<E, DK, GATE, ADD>), dim3((unsigned)(p.slots * p.H)), dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <typename E, int DK>
hipError_t launch_b(const BwdParams &p, int gate, bool add, hipStream_t stream) {
  if (p.N == 0 || p.slots * p.H == 0) return hipSuccess;
  if (gate == GATE_HEAD)
    return add ? launch_bg<E, DK, GATE_HEAD, true>(p, stream) : launch_bg<E, DK, GATE_HEAD, false>(p, stream);
  if (gate == GATE_NONE)
    return add ? launch_bg<E, DK, GATE_NONE, true>(p, stream) : launch_bg<E, DK, GATE_NONE, false>(p, stream);
  return hipErrorInvalidValue;
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

// gdn_bwd_slices.h -- the sums over the value columns of one (chunk, head) that the
// per-chunk gradient kernels need (no gate or a scalar gate, and one decay per key
// channel), formed at full value width from the chunk's entering state M0, its chunk-end
// state gradient dM and dDelta, 32 value columns at a time.
#pragma once
#include <type_traits>

#include "gdn_common.h"
#include "gdn_tile.h"

namespace gdn {

// an input row piece as an MFMA fragment: exact in bf16, split into hi + lo from fp32
__device__ __forceinline__ bf16x8 in8(const bf16 *p) { return ld8(p); }
__device__ __forceinline__ Split in8(const float *p) { return split8(ld8(p)); }
// an fp32 array kept in LDS as two bf16 arrays (hi, lo)
struct Halves {
  bf16 *h, *l;
};
__device__ __forceinline__ Split sfrag(const Halves &x, int o) { return Split{ld8(x.h + o), ld8(x.l + o)}; }
__device__ __forceinline__ void sput(const Halves &x, int o, float v) {
  const bf16 hv = (bf16)v;
  x.h[o] = hv;
  x.l[o] = (bf16)(v - (float)hv);
}
__device__ __forceinline__ void sput4(const Halves &x, int o, const f32x4 &v) {
  bf16x4 hv, lv;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hv[j] = (bf16)v[j];
    lv[j] = (bf16)(v[j] - (float)hv[j]);
  }
  *(bf16x4 *)(x.h + o) = hv;
  *(bf16x4 *)(x.l + o) = lv;
}

// LDS of one slice (bytes): M0^T (delta write), M0 and dM (d_k rows), Delta, then dO and
// V (I/O dtype), then for the delta write dDelta, dDelta^T, (beta X)^T, beta X and
// -beta Y; every fp32 matrix as bf16 halves in the layout its fragments read
template <typename E, int DK, bool ADD> struct SliceLds {
  static constexpr int PMT = DK + 8, PC = 40, PR = 64 + 8;  // bf16 pitches
  static constexpr int HM = 32 * PMT, HR = DK * PC, H6 = 64 * PC, HT = 32 * PR;
  static constexpr int BYTES = 4 * ((ADD ? 0 : HM) + 2 * HR + H6) + 2 * H6 * (int)sizeof(E) +
                               (ADD ? 0 : 4 * (3 * H6 + 2 * HT));
};

// The sums, in the matrix-core accumulators of eight waves (wave w):
//   dP = dO Delta^T (lower tiles) and dT = dDelta (diag(beta) X)^T: tiles w and w + 8 of
//   the 4 x 4 (row block t / 4, column block t % 4);
//   dQt = dO M0^T, dKt = -diag(beta) Y M0^T, dKh = Delta dM^T: row block w % 4, key-
//   channel blocks w / 4 + 2 q;
//   dby: Y * X of the lane's four rows (row block w / 2, column block w % 2 of the
//   slice), to be summed over the lanes' columns and the slices;
//   dgm[q]: <M0[d], dM[d]> over this thread's staged pieces of key row
//   d = (tid + 512 q) / 8 (eight consecutive threads share a row).
template <int DK> struct SliceSums {
  static constexpr int NCT = DK / 32, NM = DK * 8 / 512;
  f32x4 aP[2], aT[2], aQ[NCT], aK[NCT], aH[NCT], dby;
  float dgm[NM];
};

// The chunk's operands: its rows start at token tb (nv valid), the fp32 workspace
// arrays are this chunk's (M0 and dM [d_k][d_v], dDelta [64][d_v], T and T^T
// [64][64]); kt: K e^G [64][d_k] for one decay per key channel, NULL for a scalar
// gate (then K comes from LDS, exact, and X takes the row factor e^G).
struct SliceIn {
  const float *st, *dmc, *dd, *tm, *tmT, *kt;
  const void *v, *dout;
  size_t tb;
  int nv, H, h, dv;
};

// X = V - Kt M0, Delta = T diag(beta) X (the additive write: Delta = V), Y = T^T dDelta,
// and the sums above, over all d_v / 32 slices (the next slice's loads in flight while
// one computes).  U: SliceLds::BYTES of LDS; Kl: K rows (pitch DK + 8) for a scalar
// gate; eg, bs: e^G and beta per row (LDS).  512 threads; ends with a barrier, after
// which U is free.
template <typename E, int DK, bool ADD, bool KEY>
__device__ __forceinline__ void slice_sums(const SliceIn &in, char *U, const E *Kl, const float *eg,
                                           const float *bs, SliceSums<DK> &S) {
  typedef SliceLds<E, DK, ADD> L;
  constexpr int NT = 512, PMT = L::PMT, PC = L::PC, PR = L::PR, PK = DK + 8;
  constexpr int NCT = SliceSums<DK>::NCT, NM = SliceSums<DK>::NM;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, lm = lane & 15;
  const int nv = in.nv, H = in.H, h = in.h, dv = in.dv;
  char *u = U;
  auto halves = [&](int n) {
    Halves x{(bf16 *)u, (bf16 *)u + n};
    u += 4 * n;
    return x;
  };
  const Halves M0T = ADD ? Halves{nullptr, nullptr} : halves(L::HM);
  const Halves M0r = halves(L::HR), dMr = halves(L::HR), Dr = halves(L::H6);
  E *const dOr = (E *)u;
  u += L::H6 * sizeof(E);
  E *const Vr = (E *)u;
  u += L::H6 * sizeof(E);
  Halves dDr{nullptr, nullptr}, dDT{nullptr, nullptr}, XbT{nullptr, nullptr}, Xbr{nullptr, nullptr},
      nYr{nullptr, nullptr};
  if constexpr (!ADD) {
    dDr = halves(L::H6);
    dDT = halves(L::HT);
    XbT = halves(L::HT);
    Xbr = halves(L::H6);
    nYr = halves(L::H6);
  }
  const int a = wave >> 1, ct = wave & 1;   // X, Delta, Y tiles: row block a, column block ct
  const int wa = wave & 3, wc = wave >> 2;  // dQt / dKt / dKh tiles
  // T (rows of block a, k-steps 0 .. a / 2) and T^T (k-steps a / 2 .. 1) as A fragments,
  // split once
  Split fT[2], fTt[2];
  if constexpr (!ADD) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int o = (16 * a + lm) * 64 + 32 * s + 8 * lg;
      if (s <= (a >> 1)) fT[s] = split8(ld8(in.tm + o));
      if (s >= (a >> 1)) fTt[s] = split8(ld8(in.tmT + o));
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) S.aP[q] = S.aT[q] = zero4();
#pragma unroll
  for (int q = 0; q < NCT; ++q) S.aQ[q] = S.aK[q] = S.aH[q] = zero4();
  S.dby = zero4();
#pragma unroll
  for (int q = 0; q < NM; ++q) S.dgm[q] = 0.f;
  // a slice's loads: 16-byte pieces of M0, dM (DK x 32 fp32), dDelta (64 x 32 fp32),
  // dO and V (64 x 32, I/O dtype; rows past the end re-read the last row, zeroed when
  // staged).  No branch around a load but the thread-count guard.
  constexpr int VE = 16 / (int)sizeof(E), NVP = 64 * 32 / VE;  // dO / V pieces
  f32x4 rm[NM], rdm[NM], rdd;
  u32x4 rv, ro;
  auto fetch = [&](int col0) {
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      const int pc = tid + NT * q, d = pc >> 3, g = pc & 7;
      rm[q] = *(const f32x4 *)(in.st + (size_t)d * dv + col0 + 4 * g);
      rdm[q] = *(const f32x4 *)(in.dmc + (size_t)d * dv + col0 + 4 * g);
    }
    if constexpr (!ADD) rdd = *(const f32x4 *)(in.dd + (size_t)(tid >> 3) * dv + col0 + 4 * (tid & 7));
    if (tid < NVP) {
      const int r = min(tid / (32 / VE), nv - 1), g = tid % (32 / VE);
      const size_t o = ((in.tb + r) * H + h) * dv + col0 + g * VE;
      rv = *(const u32x4 *)((const E *)in.v + o);
      ro = *(const u32x4 *)((const E *)in.dout + o);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      const int pc = tid + NT * q, d = pc >> 3, g = pc & 7;
      sput4(M0r, d * PC + 4 * g, rm[q]);
      sput4(dMr, d * PC + 4 * g, rdm[q]);
      if constexpr (!ADD)
#pragma unroll
        for (int e = 0; e < 4; ++e) sput(M0T, (4 * g + e) * PMT + d, rm[q][e]);
      S.dgm[q] += rm[q][0] * rdm[q][0] + rm[q][1] * rdm[q][1] + rm[q][2] * rdm[q][2] + rm[q][3] * rdm[q][3];
    }
    if constexpr (!ADD) {
      const int r = tid >> 3, g = tid & 7;
      sput4(dDr, r * PC + 4 * g, rdd);
#pragma unroll
      for (int e = 0; e < 4; ++e) sput(dDT, (4 * g + e) * PR + r, rdd[e]);
    }
    if (tid < NVP) {
      const int r = tid / (32 / VE), g = tid % (32 / VE);
      const bool ok = r < nv;
      const u32x4 z = {0u, 0u, 0u, 0u};
      *(u32x4 *)(dOr + r * PC + g * VE) = ok ? ro : z;
      if constexpr (ADD) {  // Delta = V
        typedef E EV __attribute__((ext_vector_type(16 / sizeof(E))));
        const EV ev = __builtin_bit_cast(EV, rv);
#pragma unroll
        for (int e = 0; e < VE; ++e) sput(Dr, r * PC + g * VE + e, ok ? to_f(ev[e]) : 0.f);
      } else {
        *(u32x4 *)(Vr + r * PC + g * VE) = ok ? rv : z;
      }
    }
  };
  fetch(0);
  for (int col0 = 0; col0 < dv; col0 += 32) {
    if (col0) __syncthreads();  // every read of the previous slice is done
    stage();
    if (col0 + 32 < dv) fetch(col0 + 32);
    __syncthreads();
    if constexpr (!ADD) {
      // X = V - Kt M0: tile (a, ct); with a scalar gate K exact and the row factor e^G
      f32x4 acc = zero4();
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += 32) {
        const Split fm = sfrag(M0T, (16 * ct + lm) * PMT + k0 + 8 * lg);
        if constexpr (KEY)
          acc = mm(split8(ld8(in.kt + (16 * a + lm) * DK + k0 + 8 * lg)), fm, acc);
        else
          acc = mm(in8(Kl + (16 * a + lm) * PK + k0 + 8 * lg), fm, acc);
      }
      const int col = 16 * ct + lm;
      f32x4 xv, bx;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * a + 4 * lg + j;
        xv[j] = to_f(Vr[r * PC + col]) - (KEY ? acc[j] : eg[r] * acc[j]);
        bx[j] = bs[r] * xv[j];
        sput(Xbr, r * PC + col, bx[j]);
      }
      sput4(XbT, col * PR + 16 * a + 4 * lg, bx);
      __syncthreads();
      // Delta = T (beta X), Y = T^T dDelta: tile (a, ct)
      f32x4 D = zero4(), Y = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s <= (a >> 1)) D = mm(fT[s], sfrag(XbT, col * PR + 32 * s + 8 * lg), D);
        if (s >= (a >> 1)) Y = mm(fTt[s], sfrag(dDT, col * PR + 32 * s + 8 * lg), Y);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * a + 4 * lg + j;
        sput(Dr, r * PC + col, D[j]);
        sput(nYr, r * PC + col, -bs[r] * Y[j]);
        S.dby[j] += Y[j] * xv[j];
      }
      __syncthreads();
    }
    // dP (lower tiles) and dT: tiles wave and wave + 8 of the 4 x 4
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int t = wave + 8 * q, m0 = 16 * (t >> 2), n0 = 16 * (t & 3);
      if (n0 <= m0) S.aP[q] = mm(in8(dOr + (m0 + lm) * PC + 8 * lg), sfrag(Dr, (n0 + lm) * PC + 8 * lg), S.aP[q]);
      if constexpr (!ADD)
        S.aT[q] = mm(sfrag(dDr, (m0 + lm) * PC + 8 * lg), sfrag(Xbr, (n0 + lm) * PC + 8 * lg), S.aT[q]);
    }
    // dQt, dKt, dKh: row block wa, channel blocks wc + 2 q
    {
      const auto fo = in8(dOr + (16 * wa + lm) * PC + 8 * lg);
      const Split fd = sfrag(Dr, (16 * wa + lm) * PC + 8 * lg);
      Split fy;
      if constexpr (!ADD) fy = sfrag(nYr, (16 * wa + lm) * PC + 8 * lg);
#pragma unroll
      for (int q = 0; q < NCT; ++q) {
        const int n0 = 16 * (wc + 2 * q);
        const Split fm = sfrag(M0r, (n0 + lm) * PC + 8 * lg);
        S.aQ[q] = mm(fo, fm, S.aQ[q]);
        if constexpr (!ADD) S.aK[q] = mm(fy, fm, S.aK[q]);
        S.aH[q] = mm(fd, sfrag(dMr, (n0 + lm) * PC + 8 * lg), S.aH[q]);
      }
    }
  }
  __syncthreads();  // U is free
}

}  // namespace gdn

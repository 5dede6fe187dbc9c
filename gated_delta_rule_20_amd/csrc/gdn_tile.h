// gdn_tile.h -- 16x16 fp32 matrix-core tiles with gathered operands (backward and the
// diagonal-plus-low-rank forward).
#pragma once
#include <type_traits>

#include "gdn_common.h"

namespace gdn {

// One 16x16 tile of C = A B on the matrix cores in fp32 (v_mfma_f32_16x16x4f32, eight
// per 32-deep step; K a multiple of 32).  Operands are gathered through a(m, k) and
// b(k, n); lane (lg, lm) supplies A row m0 + lm and B column n0 + lm at k = k0 + 8 lg
// + i, and ends with C[m0 + 4 lg + j][n0 + lm], j = 0..3.
template <int K, class FA, class FB>
__device__ __forceinline__ f32x4 tile(int m0, int n0, int lg, int lm, FA a, FB b) {
  f32x4 acc = zero4();
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    f32x8 af, bf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      af[i] = a(m0 + lm, k0 + 8 * lg + i);
      bf[i] = b(k0 + 8 * lg + i, n0 + lm);
    }
    acc = mma(af, bf, acc);
  }
  return acc;
}
// Every 16x16 tile of an M x N product, spread over NW waves (this one is w of them);
// epi(r, c, v) receives C[r + j][c] = v[j], j = 0..3.
template <int M, int N, int K, int NW, class FA, class FB, class EPI>
__device__ __forceinline__ void mfma_mm(int w, int lane, FA a, FB b, EPI epi) {
  const int lg = lane >> 4, lm = lane & 15;
  constexpr int TN = N / 16, TILES = (M / 16) * TN;
  for (int t = w; t < TILES; t += NW) {
    const int m0 = (t / TN) * 16, n0 = (t % TN) * 16;
    epi(m0 + 4 * lg, n0 + lm, tile<K>(m0, n0, lg, lm, a, b));
  }
}

// ---- bf16 matrix cores on fp32 data: a split into two bf16 terms.
// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi) (both round to nearest even):
// |x - hi| <= 2^-9 |x| and |x - hi - lo| <= 2^-18 |x|.  A product then takes three bf16
// MFMAs (lo*hi', hi*lo', hi*hi'; the dropped lo*lo' is below 2^-18 of it), or two when
// one operand is exactly bf16 already (an input), for a relative error near 2^-17
// where one bf16 rounding would give 2^-9.  Accumulation is fp32.
struct Split {
  bf16x8 hi, lo;
};
__device__ __forceinline__ Split split8(const f32x8 &x) {
  Split s;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s.hi[i] = (bf16)x[i];
    s.lo[i] = (bf16)(x[i] - (float)s.hi[i]);
  }
  return s;
}
__device__ __forceinline__ f32x8 widen8(const bf16x8 &x) {
  f32x8 y;
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (float)x[i];
  return y;
}
__device__ __forceinline__ f32x4 mm(const bf16x8 &a, const bf16x8 &b, f32x4 c) { return mma(a, b, c); }
__device__ __forceinline__ f32x4 mm(const bf16x8 &a, const Split &b, f32x4 c) { return mma(a, b.hi, mma(a, b.lo, c)); }
__device__ __forceinline__ f32x4 mm(const Split &a, const bf16x8 &b, f32x4 c) { return mma(a.hi, b, mma(a.lo, b, c)); }
__device__ __forceinline__ f32x4 mm(const Split &a, const Split &b, f32x4 c) {
  return mma(a.hi, b.hi, mma(a.hi, b.lo, mma(a.lo, b.hi, c)));
}
// One 16x16 tile of C = A B from fragment loaders: fa(k0) gives this lane's A
// fragment (its row, k = k0 + 8 lg .. + 7), fb(k0) its B fragment (its column, the
// same k), each a bf16x8 (exact) or a Split.  32-deep steps from k0 = kend on are
// skipped (known zeros of a triangular operand); kend must be wave-uniform.
template <int K, class FA, class FB>
__device__ __forceinline__ f32x4 tile_frag(FA fa, FB fb, int kend = K) {
  f32x4 acc = zero4();
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32)
    if (k0 < kend) acc = mm(fa(k0), fb(k0), acc);
  return acc;
}
__device__ __forceinline__ bf16x8 to_bf8(const f32x8 &x) {
  bf16x8 y;
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (bf16)x[i];
  return y;
}
// One 16x16 tile of C = A B with operands gathered through a(m, k) and b(k, n), as
// `tile`: on the fp32 matrix cores when E is float; when E is bf16, on the bf16 matrix
// cores, an operand whose values are bf16 inputs (XA, XB) taken exactly and any other
// as a Split pair.  On the bf16 path 32-deep steps outside [kbeg, kend) (known zeros of
// a triangular operand; wave-uniform bounds) are skipped.
template <typename E, int K, bool XA, bool XB, class FA, class FB>
__device__ __forceinline__ f32x4 tile_g(int m0, int n0, int lg, int lm, FA a, FB b, int kbeg = 0, int kend = K) {
  if constexpr (!std::is_same<E, bf16>::value) {
    return tile<K>(m0, n0, lg, lm, a, b);
  } else {
    f32x4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      if (k0 + 32 <= kbeg || k0 >= kend) continue;
      f32x8 af, bv;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        af[i] = a(m0 + lm, k0 + 8 * lg + i);
        bv[i] = b(k0 + 8 * lg + i, n0 + lm);
      }
      if constexpr (XA && XB)
        acc = mm(to_bf8(af), to_bf8(bv), acc);
      else if constexpr (XA)
        acc = mm(to_bf8(af), split8(bv), acc);
      else if constexpr (XB)
        acc = mm(split8(af), to_bf8(bv), acc);
      else
        acc = mm(split8(af), split8(bv), acc);
    }
    return acc;
  }
}
// Every 16x16 tile of an M x N product through tile_g, spread over NW waves (as mfma_mm).
template <typename E, int M, int N, int K, int NW, bool XA, bool XB, class FA, class FB, class EPI>
__device__ __forceinline__ void mm_g(int w, int lane, FA a, FB b, EPI epi) {
  const int lg = lane >> 4, lm = lane & 15;
  constexpr int TN = N / 16, TILES = (M / 16) * TN;
  for (int t = w; t < TILES; t += NW) {
    const int m0 = (t / TN) * 16, n0 = (t % TN) * 16;
    epi(m0 + 4 * lg, n0 + lm, tile_g<E, K, XA, XB>(m0, n0, lg, lm, a, b));
  }
}
// Four bf16 of one column of a row-major bf16 matrix per lane, through the gfx950
// transposing LDS read: within each 16-lane group, lane L receives element j
// (j = 0..3) from the 8 bytes that lane 4j + L/4 addressed, at position L % 4.
__device__ __forceinline__ bf16x4 lds_tr4(const bf16 *p) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t *)p);
  return __builtin_bit_cast(bf16x4, v);
}
// The 8-deep column fragment X[k0 + 8 lg + j][c0 + lm], j = 0..7, of a row-major bf16
// matrix X in LDS with row pitch `pitch` (elements; rows 8-byte aligned).
__device__ __forceinline__ bf16x8 col_frag(const bf16 *X, int pitch, int k0, int c0, int lg, int lm) {
  const bf16 *p0 = X + (k0 + 8 * lg + (lm >> 2)) * pitch + c0 + 4 * (lm & 3);
  const bf16x4 a = lds_tr4(p0), b = lds_tr4(p0 + 4 * pitch);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Workgroup bid of a grid of `pairs` (sequence, head) pairs x nb value blocks -> (pair,
// value block), such that the nb blocks of one pair get ids equal mod 8: consecutive
// ids go to the eight XCDs in turn, so the blocks of a pair run on one XCD and share its
// L2 for the operands that every block of the pair reads.
__device__ __forceinline__ void xcd_pair_block(int bid, int pairs, int nb, int &pair, int &jb) {
  const int grp = 8 * nb, full = (pairs * nb / grp) * grp;
  if (bid < full) {
    const int slot = bid >> 3;
    pair = (slot / nb) * 8 + (bid & 7);
    jb = slot % nb;
  } else {
    pair = bid / nb;
    jb = bid % nb;
  }
}

// x as a hi + lo pair of bf16 (see Split) stored at hi[i] and lo[i].
__device__ __forceinline__ void store_split(bf16 *hi, bf16 *lo, size_t i, float x) {
  const bf16 h = (bf16)x;
  hi[i] = h;
  lo[i] = (bf16)(x - (float)h);
}
// The fragment (8 contiguous elements) of a matrix stored as hi and lo bf16 halves.
__device__ __forceinline__ Split ld_split(const bf16 *hi, const bf16 *lo) { return Split{ld8(hi), ld8(lo)}; }

// Inclusive prefix sum over the 64 lanes of a wave, in fp32: within each 16-lane row
// by four DPP row shifts (1, 2, 4, 8; lanes without a source add 0), then the totals
// of the earlier rows, read from their last lanes.  Every lane of the wave must be
// active.
__device__ __forceinline__ float wave_scan64(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f);
}

// Forward substitution of one unit lower triangular 16 x 16 system per 16-lane row of
// a wave, in fp32: on entry lane lm holds nl[i] = -L[lm][i] (zero for i >= lm); on
// return t[0..15] is row lm of (I + L)^-1.  Step i adds nl[i] times row i of the result
// to every later row; row i is final once steps 0 .. i-1 are done, and it reaches the
// other lanes of its 16-lane row by DPP broadcast (row_newbcast), so no LDS round trip
// sits in the dependent chain.  Each step is one asm block that starts with the two
// wait states a DPP read needs after a VALU write of the same register.
__device__ __forceinline__ void lower_solve16(float (&t)[16], const float (&nl)[16]) {
  const int lm = threadIdx.x & 15;
#pragma unroll
  for (int c = 0; c < 16; ++c) t[c] = (c == lm) ? 1.f : 0.f;
#define GDN_LS_FMA(I, C) "v_fmac_f32_dpp %" #C ", %" #C ", %16 row_newbcast:" #I " row_mask:0xf bank_mask:0xf\n"
#define GDN_LS_STEP(I, BODY)                                                                        \
  asm volatile("s_nop 1\n" BODY                                                                    \
               : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]), \
                 "+v"(t[7]), "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]),           \
                 "+v"(t[13]), "+v"(t[14]), "+v"(t[15])                                               \
               : "v"(nl[I]))
  GDN_LS_STEP(0, GDN_LS_FMA(0, 0));
  GDN_LS_STEP(1, GDN_LS_FMA(1, 0) GDN_LS_FMA(1, 1));
  GDN_LS_STEP(2, GDN_LS_FMA(2, 0) GDN_LS_FMA(2, 1) GDN_LS_FMA(2, 2));
  GDN_LS_STEP(3, GDN_LS_FMA(3, 0) GDN_LS_FMA(3, 1) GDN_LS_FMA(3, 2) GDN_LS_FMA(3, 3));
  GDN_LS_STEP(4, GDN_LS_FMA(4, 0) GDN_LS_FMA(4, 1) GDN_LS_FMA(4, 2) GDN_LS_FMA(4, 3) GDN_LS_FMA(4, 4));
  GDN_LS_STEP(5, GDN_LS_FMA(5, 0) GDN_LS_FMA(5, 1) GDN_LS_FMA(5, 2) GDN_LS_FMA(5, 3) GDN_LS_FMA(5, 4)
                     GDN_LS_FMA(5, 5));
  GDN_LS_STEP(6, GDN_LS_FMA(6, 0) GDN_LS_FMA(6, 1) GDN_LS_FMA(6, 2) GDN_LS_FMA(6, 3) GDN_LS_FMA(6, 4)
                     GDN_LS_FMA(6, 5) GDN_LS_FMA(6, 6));
  GDN_LS_STEP(7, GDN_LS_FMA(7, 0) GDN_LS_FMA(7, 1) GDN_LS_FMA(7, 2) GDN_LS_FMA(7, 3) GDN_LS_FMA(7, 4)
                     GDN_LS_FMA(7, 5) GDN_LS_FMA(7, 6) GDN_LS_FMA(7, 7));
  GDN_LS_STEP(8, GDN_LS_FMA(8, 0) GDN_LS_FMA(8, 1) GDN_LS_FMA(8, 2) GDN_LS_FMA(8, 3) GDN_LS_FMA(8, 4)
                     GDN_LS_FMA(8, 5) GDN_LS_FMA(8, 6) GDN_LS_FMA(8, 7) GDN_LS_FMA(8, 8));
  GDN_LS_STEP(9, GDN_LS_FMA(9, 0) GDN_LS_FMA(9, 1) GDN_LS_FMA(9, 2) GDN_LS_FMA(9, 3) GDN_LS_FMA(9, 4)
                     GDN_LS_FMA(9, 5) GDN_LS_FMA(9, 6) GDN_LS_FMA(9, 7) GDN_LS_FMA(9, 8) GDN_LS_FMA(9, 9));
  GDN_LS_STEP(10, GDN_LS_FMA(10, 0) GDN_LS_FMA(10, 1) GDN_LS_FMA(10, 2) GDN_LS_FMA(10, 3) GDN_LS_FMA(10, 4)
                      GDN_LS_FMA(10, 5) GDN_LS_FMA(10, 6) GDN_LS_FMA(10, 7) GDN_LS_FMA(10, 8) GDN_LS_FMA(10, 9)
                          GDN_LS_FMA(10, 10));
  GDN_LS_STEP(11, GDN_LS_FMA(11, 0) GDN_LS_FMA(11, 1) GDN_LS_FMA(11, 2) GDN_LS_FMA(11, 3) GDN_LS_FMA(11, 4)
                      GDN_LS_FMA(11, 5) GDN_LS_FMA(11, 6) GDN_LS_FMA(11, 7) GDN_LS_FMA(11, 8) GDN_LS_FMA(11, 9)
                          GDN_LS_FMA(11, 10) GDN_LS_FMA(11, 11));
  GDN_LS_STEP(12, GDN_LS_FMA(12, 0) GDN_LS_FMA(12, 1) GDN_LS_FMA(12, 2) GDN_LS_FMA(12, 3) GDN_LS_FMA(12, 4)
                      GDN_LS_FMA(12, 5) GDN_LS_FMA(12, 6) GDN_LS_FMA(12, 7) GDN_LS_FMA(12, 8) GDN_LS_FMA(12, 9)
                          GDN_LS_FMA(12, 10) GDN_LS_FMA(12, 11) GDN_LS_FMA(12, 12));
  GDN_LS_STEP(13, GDN_LS_FMA(13, 0) GDN_LS_FMA(13, 1) GDN_LS_FMA(13, 2) GDN_LS_FMA(13, 3) GDN_LS_FMA(13, 4)
                      GDN_LS_FMA(13, 5) GDN_LS_FMA(13, 6) GDN_LS_FMA(13, 7) GDN_LS_FMA(13, 8) GDN_LS_FMA(13, 9)
                          GDN_LS_FMA(13, 10) GDN_LS_FMA(13, 11) GDN_LS_FMA(13, 12) GDN_LS_FMA(13, 13));
  GDN_LS_STEP(14, GDN_LS_FMA(14, 0) GDN_LS_FMA(14, 1) GDN_LS_FMA(14, 2) GDN_LS_FMA(14, 3) GDN_LS_FMA(14, 4)
                      GDN_LS_FMA(14, 5) GDN_LS_FMA(14, 6) GDN_LS_FMA(14, 7) GDN_LS_FMA(14, 8) GDN_LS_FMA(14, 9)
                          GDN_LS_FMA(14, 10) GDN_LS_FMA(14, 11) GDN_LS_FMA(14, 12) GDN_LS_FMA(14, 13)
                              GDN_LS_FMA(14, 14));
#undef GDN_LS_STEP
#undef GDN_LS_FMA
}

// T = (I + s A)^-1 (s = SGN, +1 or -1) of a strictly lower triangular 64 x 64 fp32
// matrix A in LDS (row pitch sa), written to LDS T (row pitch st; every entry).
// Blocked: wave 0 solves the four 16 x 16 diagonal blocks by forward substitution
// (lane (lg, lm) takes row lm of block lg, lower_solve16); then waves 0-2 each walk down one block
// column b, T[a][b] = -s T[a][a] sum_{b <= k < a} A[a][k] T[k][b] for a = b+1 .. 3, on
// the bf16 matrix cores with split operands (the inner sum passes through the wave's
// 16 x 17 slice of ys).  Every thread of the workgroup (at least four waves) calls it;
// it ends with a barrier.
template <int SGN>
__device__ __forceinline__ void tri_inv64(const float *A, int sa, float *T, int st, float *ys) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lm = lane & 15;
  for (int i = tid; i < 64 * 64; i += blockDim.x) {
    const int r = i >> 6, c = i & 63;
    if ((c >> 4) > (r >> 4)) T[r * st + c] = 0.f;
  }
  if (wave == 0) {
    // lane (lg, lm) solves row lm of diagonal block lg (entries of A on or above the
    // diagonal are not read as zeros: they are masked)
    const int o = 16 * lg;
    const float *ar = A + (o + lm) * sa + o;
    float nl[16], t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) nl[i] = i < lm ? -(float)SGN * ar[i] : 0.f;
    lower_solve16(t, nl);
    float *tr = T + (o + lm) * st + o;
#pragma unroll
    for (int c = 0; c < 16; ++c) tr[c] = t[c];
  }
  __syncthreads();
  if (wave < 3) {
    const int b = wave;
    float *y = ys + wave * (16 * 17);
    for (int a = b + 1; a < 4; ++a) {
      f32x4 acc = zero4();
#pragma unroll
      for (int k0 = 0; k0 < 64; k0 += 32) {
        if (k0 + 32 <= 16 * b || k0 >= 16 * a) continue;
        f32x8 fa, fb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = k0 + 8 * lg + i;
          const bool in = k >= 16 * b && k < 16 * a;
          fa[i] = in ? A[(16 * a + lm) * sa + k] : 0.f;
          fb[i] = in ? T[k * st + 16 * b + lm] : 0.f;
        }
        acc = mm(split8(fa), split8(fb), acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) y[(4 * lg + j) * 17 + lm] = acc[j];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      f32x8 fa, fb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = 8 * lg + i;
        fa[i] = k < 16 ? T[(16 * a + lm) * st + 16 * a + k] : 0.f;
        fb[i] = k < 16 ? y[k * 17 + lm] : 0.f;
      }
      const f32x4 z = mm(split8(fa), split8(fb), zero4());
#pragma unroll
      for (int j = 0; j < 4; ++j) T[(16 * a + 4 * lg + j) * st + 16 * b + lm] = -(float)SGN * z[j];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  __syncthreads();
}

}  // namespace gdn

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

}  // namespace gdn

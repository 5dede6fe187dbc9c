// gdn_tile.h -- 16x16 fp32 matrix-core tiles with gathered operands (backward and the
// diagonal-plus-low-rank forward).
#pragma once
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

}  // namespace gdn

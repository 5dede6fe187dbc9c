// gdn_common.h -- device-side building blocks shared by the gfx950 kernels.
//
// MFMA operand layouts (v_mfma_f32_16x16x32_bf16; lane l, lg = l / 16, lm = l % 16):
//   A (16 x 32):  lane holds row lm, k-slots 8*lg .. 8*lg+7
//   B (32 x 16):  lane holds column lm, k-slots 8*lg .. 8*lg+7
//   C (16 x 16):  lane holds column lm, rows 4*lg .. 4*lg+3
// The k index is a pure contraction index, so any permutation applied to A and B
// alike gives the same product.  Two C tiles (rows 0-15 and 16-31 of a matrix Y)
// therefore feed a B operand directly ("B from C"): slots 8*lg+0..3 take the first
// tile's rows 4*lg+0..3 and slots 8*lg+4..7 the second tile's rows 16+4*lg+0..3;
// the matching A operand reads columns 4*lg+0..3 and 16+4*lg+0..3 ("split" load).
// In fp32 mode the same 8-slot fragments are consumed by eight
// v_mfma_f32_16x16x4_f32 instructions (instruction i takes slot 8*lg+i of every
// lane group), so both modes share one data layout.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename E> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8 &a, const f32x8 &b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

template <typename E> __device__ __forceinline__ E to_e(float x);
template <> __device__ __forceinline__ bf16 to_e<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float to_e<float>(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

// 8 contiguous elements (one A or B fragment in natural k order).
__device__ __forceinline__ bf16x8 ld8(const bf16 *p) { return *(const bf16x8 *)p; }
__device__ __forceinline__ f32x8 ld8(const float *p) {
  f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// 4 + 4 elements from two places (the "split" A operand that matches B-from-C).
__device__ __forceinline__ bf16x8 ld4x2(const bf16 *p0, const bf16 *p1) {
  bf16x4 a = *(const bf16x4 *)p0, b = *(const bf16x4 *)p1;
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x8 ld4x2(const float *p0, const float *p1) {
  f32x4 a = *(const f32x4 *)p0, b = *(const f32x4 *)p1;
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// 4 elements then zeros (a 16-deep contraction on the 32-deep instruction).
__device__ __forceinline__ bf16x8 ld4z(const bf16 *p0) {
  bf16x4 a = *(const bf16x4 *)p0, z = {};
  return __builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x8 ld4z(const float *p0) {
  f32x4 a = *(const f32x4 *)p0, z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7);
}
// 4 contiguous elements as fp32.
__device__ __forceinline__ f32x4 ld4f(const bf16 *p) {
  bf16x4 a = *(const bf16x4 *)p;
  return (f32x4){(float)a[0], (float)a[1], (float)a[2], (float)a[3]};
}
__device__ __forceinline__ f32x4 ld4f(const float *p) { return *(const f32x4 *)p; }

// B operand from two C tiles (see the header comment); scaled variant multiplies
// row-wise by s (the four rows this lane holds in each tile).
template <typename E>
__device__ __forceinline__ typename Frag<E>::type frag_from_c(const f32x4 &lo, const f32x4 &hi) {
  typename Frag<E>::type f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = to_e<E>(lo[j]);
    f[4 + j] = to_e<E>(hi[j]);
  }
  return f;
}
template <typename E>
__device__ __forceinline__ typename Frag<E>::type frag_from_c_half(const f32x4 &lo) {
  typename Frag<E>::type f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = to_e<E>(lo[j]);
    f[4 + j] = to_e<E>(0.f);
  }
  return f;
}

__device__ __forceinline__ f32x4 zero4() { return (f32x4){0.f, 0.f, 0.f, 0.f}; }

// Empty asm that "reads and writes" a register: the compiler must have the value
// (waiting for its load here, not earlier) and cannot hoist later arithmetic on it
// above this point.  Used to keep prefetched tiles in flight until they are stored.
__device__ __forceinline__ void opaque(u32x4 &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void opaque(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void opaque(f32x4 &x) { asm volatile("" : "+v"(x)); }

}  // namespace gdn

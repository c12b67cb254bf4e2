// Device-side helpers shared by the librkv kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native, splits into VGPRs

// bfloat16 <-> float.  Inputs are finite; NaN keeps a NaN payload.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(uint32_t(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// IEEE half (round to nearest even) <-> float.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Row of element r (0..15) of a 32x32 fp32 MFMA accumulator held by `lane`;
// its column is lane % 32.
__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
}

// x as a (hi, lo) bf16 pair, hi = bf16(x) and lo = bf16(x - hi), both
// rounded to nearest even (gfx950 converts in hardware: v_cvt_pk_bf16_f32);
// hi in the low 16 bits.  hi + lo carries about 16 significant bits of x.
__device__ __forceinline__ uint32_t bf16_hi_lo(float x) {
  const __bf16 hi = static_cast<__bf16>(x);
  const float lo = x - static_cast<float>(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, hi)) |
         (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(lo))) << 16);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// Keep the KL smallest (d, j) pairs in ascending (d, j) order, for
// candidates that arrive in increasing j: a newcomer then goes after every
// kept pair of equal d, so the strict comparison d < d_i decides alone.
// Branch-free select network (an infinite d never enters).
template <int KL>
__device__ __forceinline__ void topk_push(float (&bd)[KL], int (&bi)[KL], float d, int j) {
  // compare-and-swap bubble: the smaller pair stays, the larger moves on
  float x = d;
  int xj = j;
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    const bool c = x < bd[i];
    const float nd = c ? x : bd[i];
    const int ni = c ? xj : bi[i];
    x = c ? bd[i] : x;
    xj = c ? bi[i] : xj;
    bd[i] = nd;
    bi[i] = ni;
  }
}

// The same for candidates in any order: (d, j) pairs compare
// lexicographically, so equal distances keep the smaller position.
template <int KL>
__device__ __forceinline__ void topk_push_lex(float (&bd)[KL], int (&bi)[KL], float d, int j) {
  float x = d;
  int xj = j;
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    const bool c = x < bd[i] || (x == bd[i] && xj < bi[i]);
    const float nd = c ? x : bd[i];
    const int ni = c ? xj : bi[i];
    x = c ? bd[i] : x;
    xj = c ? bi[i] : xj;
    bd[i] = nd;
    bi[i] = ni;
  }
}

}  // namespace rkv

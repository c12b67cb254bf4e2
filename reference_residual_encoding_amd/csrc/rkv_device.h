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

// FP8 reference storage: OCP E4M3 (bias 7, 3 mantissa bits, subnormals
// k * 2^-9, largest finite 448, no infinities), round to nearest even,
// saturating at +-448.  Every E4M3 value is exact in bf16 and fp32.
__device__ __forceinline__ uint32_t f32_to_fp8_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t r;
  if (!(a < 448.0f)) {
    r = a != a ? 0x7Fu : 0x7Eu;                          // NaN stays NaN, the rest saturates
  } else if (a < 0.015625f) {
    r = uint32_t(rintf(a * 512.0f));                     // k * 2^-9; k = 8 is 2^-6 (field 1)
  } else {
    const uint32_t ua = __float_as_uint(a);              // 3 mantissa bits, ties to even
    r = ((ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20) - (120u << 3);
    r = r > 0x7Eu ? 0x7Eu : r;                           // rounding past 448 saturates
  }
  return sign | r;
}
__device__ __forceinline__ float fp8_e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;
  return (b & 0x80u) ? -v : v;
}
__device__ __forceinline__ float fp8_round(float x) { return fp8_e4m3_to_f32(f32_to_fp8_e4m3(x)); }

// Where the schedule ([RKV] §2.6) puts its references: the closed form of a
// fixed stride after the sinks, or a device copy of the host's positions.
struct SchedView {
  const int* rpos;  // nullptr: fixed stride
  int nref, s0, n_sink;
};

__device__ __forceinline__ int ref_position(const SchedView& v, int j) {
  if (v.rpos) return v.rpos[j];
  return j < v.n_sink ? j : v.n_sink + (j - v.n_sink) * v.s0;
}

// Number of references before position t (the index of t when t is one),
// and whether t is one.
__device__ __forceinline__ int refs_before(const SchedView& v, int t, bool& is_ref) {
  if (!v.rpos) {
    const int u = t - v.n_sink;
    is_ref = u < 0 || u % v.s0 == 0;
    return u < 0 ? t : v.n_sink + (u + v.s0 - 1) / v.s0;
  }
  int lo = 0, hi = v.nref;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (v.rpos[mid] < t) lo = mid + 1; else hi = mid;
  }
  is_ref = lo < v.nref && v.rpos[lo] == t;
  return lo;
}

// Keep the KL smallest (d, j) pairs in ascending (d, j) order, for
// candidates that arrive in increasing j: a newcomer then goes after every
// kept pair of equal d, so the strict comparison d < d_i decides alone.
// Every slot takes its new pair from the compares with the old list: it
// keeps its own, takes the newcomer, or takes the pair of the slot before
// it (the distances through min / med3), so no slot waits on another and a
// pair displaced into a run of equal distances moves down with the run
// instead of dropping out.  Branch-free; d must not be NaN (an infinite d
// never enters).
template <int KL>
__device__ __forceinline__ void topk_push(float (&bd)[KL], int (&bi)[KL], float d, int j) {
  bool c[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) c[i] = d < bd[i];
  float nd[KL];
  int ni[KL];
  nd[0] = fminf(bd[0], d);
  ni[0] = c[0] ? j : bi[0];
#pragma unroll
  for (int i = 1; i < KL; ++i) {
    nd[i] = __builtin_amdgcn_fmed3f(bd[i - 1], bd[i], d);
    ni[i] = c[i - 1] ? bi[i - 1] : (c[i] ? j : bi[i]);
  }
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    bd[i] = nd[i];
    bi[i] = ni[i];
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
    // bitwise, not short-circuit: no branch per comparison
    const bool c = (x < bd[i]) | ((x == bd[i]) & (xj < bi[i]));
    const float nd = c ? x : bd[i];
    const int ni = c ? xj : bi[i];
    x = c ? bd[i] : x;
    xj = c ? bi[i] : xj;
    bd[i] = nd;
    bi[i] = ni;
  }
}

// The KL smallest (d, j) pairs of two lists each in ascending (d, j) order,
// in ascending order, into (ad, ai): the elementwise lexicographic minima of
// a and of b reversed form a bitonic sequence that holds them, which the
// half-cleaners of a bitonic sort then order (KL a power of two).  Gives
// the same list as pushing b's pairs into a with topk_push_lex.
template <int KL>
__device__ __forceinline__ void merge_sorted_lex(float (&ad)[KL], int (&ai)[KL],
                                                 const float (&bd)[KL], const int (&bi)[KL]) {
  static_assert((KL & (KL - 1)) == 0, "a power of two");
  auto less = [](float d, int j, float d2, int j2) { return (d < d2) | ((d == d2) & (j < j2)); };
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    const float d2 = bd[KL - 1 - i];
    const int j2 = bi[KL - 1 - i];
    const bool t = less(d2, j2, ad[i], ai[i]);
    ad[i] = t ? d2 : ad[i];
    ai[i] = t ? j2 : ai[i];
  }
#pragma unroll
  for (int h = KL / 2; h >= 1; h >>= 1)
#pragma unroll
    for (int i = 0; i < KL; ++i)
      if ((i & h) == 0) {
        const int q = i + h;
        const bool t = less(ad[q], ai[q], ad[i], ai[i]);
        const float dl = t ? ad[q] : ad[i], dh = t ? ad[i] : ad[q];
        const int jl = t ? ai[q] : ai[i], jh = t ? ai[i] : ai[q];
        ad[i] = dl; ai[i] = jl;
        ad[q] = dh; ai[q] = jh;
      }
}

}  // namespace rkv

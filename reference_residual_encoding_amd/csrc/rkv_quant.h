// Group min-max quantiser of one latent row ([RKV] §2.4), shared by the
// encode's W3 epilogue, the stand-alone quantiser and the append path.
// A lane owns 8 consecutive latent values; the G8 = g / 8 lanes of a group
// are consecutive and aligned, and call together.
#pragma once
#include "rkv_device.h"

namespace rkv {

// Lane-to-lane exchange inside groups of G8 lanes (8 latent values per lane).
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float swz_xor4(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));
}
template <int G8>
__device__ __forceinline__ void group_minmax(float& mn, float& mx) {
  if constexpr (G8 >= 2) { mn = fminf(mn, dpp_xor1(mn)); mx = fmaxf(mx, dpp_xor1(mx)); }
  if constexpr (G8 >= 4) { mn = fminf(mn, dpp_xor2(mn)); mx = fmaxf(mx, dpp_xor2(mx)); }
  if constexpr (G8 >= 8) { mn = fminf(mn, swz_xor4(mn)); mx = fmaxf(mx, swz_xor4(mx)); }
}

// rint(x / d) exactly as the correctly rounded fp32 division would give it,
// for quotients below 2^4 in magnitude plus the few steps an fp16-rounded
// step or minimum can add.  x * rcp(d) (rcp within 1 ulp) lies within
// 2 ulp(16) < 4e-6 of the rounded quotient, so the two round alike unless
// the product is within 1e-5 of a half-integer; only then, and only where a
// lane of the wave needs it, is the division itself done.
__device__ __forceinline__ float rint_div(float x, float d, float rd) {
  const float y = x * rd;
  float r = rintf(y);
  // |y - rint(y)| <= 0.5; within 1e-5 of 0.5 means y is within 1e-5 of a
  // half-integer
  const bool near_half = fabsf(y - r) > 0.5f - 1e-5f;
  if (__any(near_half)) r = near_half ? rintf(x / d) : r;
  return r;
}

// Quantise the 8 consecutive latent values a lane owns ([RKV] §2.4); the
// G8 lanes of a group must all call it together.  Returns the packed codes;
// Delta_h and m_h as fp16 bits.  Integer decisions are those of fp32
// arithmetic: Delta = (max - min) / (2^b - 1), q = clamp(rint((z - m_h) /
// Delta_h)), q = 0 when Delta_h == 0 (a constant group keeps m_h, no
// division).
template <int BITS, int G8>
__device__ __forceinline__ uint32_t quant8(const float (&v)[8], uint16_t& dh_bits,
                                           uint16_t& mh_bits) {
  constexpr float kLevels = float((1 << BITS) - 1);
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) { mn = fminf(mn, v[e]); mx = fmaxf(mx, v[e]); }
  group_minmax<G8>(mn, mx);
  const float delta = (mx - mn) / kLevels;
  dh_bits = f32_to_f16_bits(delta);
  mh_bits = f32_to_f16_bits(mn);
  const float dh = f16_bits_to_f32(dh_bits), mh = f16_bits_to_f32(mh_bits);
  uint32_t word = 0;
  if (dh != 0.0f) {
    const float rd = __builtin_amdgcn_rcpf(dh);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = rint_div(v[e] - mh, dh, rd);
      word |= uint32_t(__builtin_amdgcn_fmed3f(t, 0.0f, kLevels)) << (BITS * e);   // clamp
    }
  }
  return word;
}

template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* codes, int64_t unit, uint32_t word) {
  if constexpr (BITS == 4)
    *reinterpret_cast<uint32_t*>(codes + unit * 4) = word;
  else
    *reinterpret_cast<uint16_t*>(codes + unit * 2) = uint16_t(word);
}

// Quantisation off ([RKV] §2.4: Q is the identity): the 8 latents as fp16
// bits, rounded to nearest even, little-endian, 16 bytes per lane.
constexpr int kIdentityBits = 16;
__device__ __forceinline__ u32x4 fp16x8(const float (&v)[8]) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = uint32_t(f32_to_f16_bits(v[2 * e])) | (uint32_t(f32_to_f16_bits(v[2 * e + 1])) << 16);
  return w;
}

// The record of the 8 consecutive latents of flat unit `unit` (latent
// index 8*unit over [rows][d_c]): codes, and Delta_h / m_h once per group
// (by the first of its G8 lanes).  Every lane of a group calls it (the
// quantiser exchanges min and max between them); only lanes with `act`
// write.  Identity mode writes the fp16 latents and no group numbers.
template <int BITS, int G8>
__device__ __forceinline__ void write_record8(const float (&v)[8], bool act, int lane,
                                              int64_t unit, uint8_t* codes, uint16_t* scale,
                                              uint16_t* zmin) {
  if constexpr (BITS == kIdentityBits) {
    if (act) *reinterpret_cast<u32x4*>(codes + unit * 16) = fp16x8(v);
  } else {
    uint16_t dhb, mhb;
    const uint32_t word = quant8<BITS, G8>(v, dhb, mhb);
    if (act) {
      store_codes<BITS>(codes, unit, word);
      if ((lane % G8) == 0) {
        scale[unit / G8] = dhb;
        zmin[unit / G8] = mhb;
      }
    }
  }
}

// The 8 dequantised latents of flat unit `unit` of record row `row`
// (z~ = fmaf(q, Delta_h, m_h), or the stored fp16 values in identity mode).
template <int BITS>
__device__ __forceinline__ void read_record8(const uint8_t* codes, const uint16_t* scale,
                                             const uint16_t* zmin, int64_t row, int o, int d_c,
                                             int g, float (&v)[8]) {
  if constexpr (BITS == kIdentityBits) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(codes + row * (d_c * 2) + o * 2);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = f16_bits_to_f32(uint16_t(w[e] & 0xFFFFu));
      v[2 * e + 1] = f16_bits_to_f32(uint16_t(w[e] >> 16));
    }
  } else {
    constexpr uint32_t kMask = (1u << BITS) - 1;
    uint32_t word;
    if constexpr (BITS == 4)
      word = *reinterpret_cast<const uint32_t*>(codes + row * (d_c / 2) + o / 2);
    else
      word = *reinterpret_cast<const uint16_t*>(codes + row * (d_c / 4) + o / 4);
    const int64_t grp = row * (d_c / g) + o / g;
    const float dh = f16_bits_to_f32(scale[grp]), mh = f16_bits_to_f32(zmin[grp]);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = fmaf(float((word >> (BITS * e)) & kMask), dh, mh);
  }
}

}  // namespace rkv

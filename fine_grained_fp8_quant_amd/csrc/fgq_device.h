// Device helpers shared by the gfx950 kernels of libfgq.
//
// E4M3 here is the OCP 8-bit format (bias 7, largest finite 448), which is
// what gfx950's v_cvt_pk_fp8_f32 produces; the conversion rounds to nearest
// even and keeps subnormals.  Inputs are clamped to +-448 first, so no code
// depends on the converter's overflow behaviour and no NaN code is produced.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgq {

constexpr float kE4M3Max = 448.0f;
constexpr float kFltMax = 3.40282346638528859811704183484516925e+38f;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint: the data is read once).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 8-byte streaming store (non-temporal hint: the codes are not re-read here).
__device__ __forceinline__ void store_nt8(void* p, uint2 v) {
  const u32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}

// clamp(y, -448, 448); v_med3_f32 returns y itself (sign of zero included)
// whenever y is inside the interval.
__device__ __forceinline__ float clamp448(float y) {
  return __builtin_amdgcn_fmed3f(y, -kE4M3Max, kE4M3Max);
}

// Four already-clamped floats to four E4M3 codes, byte i <- value i.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
  return (uint32_t)w;
}

// BF16 pair packed in a 32-bit word -> the two binary32 values (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// DPP lane exchange inside a row of 16 lanes (compile-time control word).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Maximum over each aligned group of 16 lanes; every lane gets the result.
// max is exact and order-free, so any pairing that covers the group works:
// swap neighbours, swap pairs, mirror halves of 8, mirror the 16.
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp<0x140>(v));  // row_mirror
  return v;
}

// Scale pair of a group from its max-abs a (binary32, correctly rounded):
// s = a / 448 (stored), r = min(448 / a, FLT_MAX) (cast multiplier).
__device__ __forceinline__ void group_scales(float a, float& s, float& r) {
  s = a / kE4M3Max;
  r = fminf(kE4M3Max / a, kFltMax);
}

// Power-of-two scale of a group from its max-abs a (finite, >= 0): the
// smallest 2^e with 448 * 2^e >= a, e >= -127, as the E8M0 byte e + 127, and
// the exact cast multiplier r = 2^-e.  With a = f * 2^E (1 <= f < 2) and
// 448 = 1.75 * 2^8, e = E - 8 when f <= 1.75 and E - 7 otherwise; f > 1.75 is
// a mantissa field above 0x600000.  Zero and subnormal a give byte 0 (their
// true e is below -127).  Bytes stay <= 247 for finite a, so 2^-e is normal.
__device__ __forceinline__ void group_scales_e8m0(float a, uint8_t& byte, float& r) {
  const uint32_t u = __float_as_uint(a);
  int b = (int)(u >> 23) - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  b = b < 0 ? 0 : b;
  byte = (uint8_t)b;
  r = __uint_as_float((uint32_t)(254 - b) << 23);  // 2^(127 - b)
}

// Scale formats of the quantisers: the stored scale type and its derivation
// from the group max-abs (stored scale s, cast multiplier r).
struct ScaleF32 {
  using T = float;
  static __device__ __forceinline__ void derive(float a, T& s, float& r) { group_scales(a, s, r); }
};
struct ScaleE8M0 {
  using T = uint8_t;
  static __device__ __forceinline__ void derive(float a, T& s, float& r) { group_scales_e8m0(a, s, r); }
};

// Eight binary32 values times r, clamped and encoded; returns 8 codes.
__device__ __forceinline__ uint2 cast8(const float* f, float r) {
  uint2 o;
  o.x = e4m3x4(clamp448(f[0] * r), clamp448(f[1] * r), clamp448(f[2] * r), clamp448(f[3] * r));
  o.y = e4m3x4(clamp448(f[4] * r), clamp448(f[5] * r), clamp448(f[6] * r), clamp448(f[7] * r));
  return o;
}

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ float absmax8(const float* f) {
  float m0 = fmaxf(fabsf(f[0]), fabsf(f[1]));
  float m1 = fmaxf(fabsf(f[2]), fabsf(f[3]));
  float m2 = fmaxf(fabsf(f[4]), fabsf(f[5]));
  float m3 = fmaxf(fabsf(f[6]), fabsf(f[7]));
  return fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
}

// binary32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace fgq

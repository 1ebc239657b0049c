// Device-side helpers for gfx950: vector types, BF16 / E4M3FN / E2M1 codecs.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pkd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> BF16 bits, round to nearest even (the gfx950 pack instruction).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed BF16 pair (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// E4M3FN encode of an already divided value y, bit for bit the rounding the
// cache format uses: nearest, ties to even code, saturate at 448, NaN -> 0x7F,
// sign of y kept. Written from the format's definition (exponent bias 7,
// subnormal step 2^-9).
__device__ __forceinline__ uint32_t e4m3_from_f32(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7Fu;  // NaN
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {                    // below 2^-6: multiples of 2^-9
    const float q = __builtin_rintf(a * 512.0f);   // exact scaling; ties to even
    return sign | uint32_t(q);            // q in [0, 8]; 8 is the code of 2^-6
  }
  const uint32_t ua = __float_as_uint(a);
  int e = int(ua >> 23) - 127;            // -6 .. 8
  uint32_t mant = (ua >> 20) & 7u;
  const uint32_t rem = ua & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (mant & 1u))) {
    ++mant;
    if (mant == 8u) { mant = 0; ++e; }
  }
  return sign | (uint32_t(e + 7) << 3) | mant;
}

// E4M3FN code -> float, exact; 0x7F / 0xFF -> NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 15u && m == 7u) return __uint_as_float(0x7FC00000u | s);
  float mag;
  if (e == 0) mag = float(m) * 0.001953125f;                       // m * 2^-9
  else mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(mag) | s);
}

// E2M1 code of y: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even
// code, saturating at 6, sign bit from y.
__device__ __forceinline__ uint32_t e2m1_from_f32(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 28) & 0x8u;
  const float a = __builtin_fabsf(y);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;                               // also NaN / inf (outside the contract)
  return sign | c;
}

// Two already divided values -> two E4M3FN codes (low byte: a), the same
// codes as e4m3_from_f32: NaN is 0x7F, magnitudes at or past 448 are clamped
// to 448 first, and the gfx950 convert rounds the rest to nearest, ties to
// even, sign kept (its subnormal codes are multiples of 2^-9).
__device__ __forceinline__ uint32_t e4m3x2_from_f32(float a, float b) {
  const float ca = fminf(fmaxf(a, -448.0f), 448.0f);
  const float cb = fminf(fmaxf(b, -448.0f), 448.0f);
  uint32_t r = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false)) & 0xFFFFu;
  if (a != a) r = (r & 0xFF00u) | 0x7Fu;
  if (b != b) r = (r & 0x00FFu) | 0x7F00u;
  return r;
}

// Eight BF16 values (one 16-byte load) -> eight E4M3FN codes of x / scale
// (IEEE float32 division; scale 0 gives code 0), little-endian in 8 bytes.
__device__ __forceinline__ u32x2 fp8_encode8(u32x4 v, float scale) {
  if (scale == 0.0f) return u32x2{0u, 0u};
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i];
    const uint32_t pair = e4m3x2_from_f32(bf16_lo(w) / scale, bf16_hi(w) / scale);
    if (i < 2) lo |= pair << (16 * i);
    else hi |= pair << (16 * (i - 2));
  }
  return u32x2{lo, hi};
}

// One NVFP4 group: sixteen BF16 values (two 16-byte loads) -> eight code
// bytes (element 2k in the low nibble of byte k) and the E4M3FN group scale
// E4M3(amax / 6); a scale that decodes to 0 gives all-zero codes.
__device__ __forceinline__ u32x2 nvfp4_encode16(u32x4 v0, u32x4 v1, uint32_t& scale_code) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(v0[i]);
    x[2 * i + 1] = bf16_hi(v0[i]);
    x[8 + 2 * i] = bf16_lo(v1[i]);
    x[8 + 2 * i + 1] = bf16_hi(v1[i]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, __builtin_fabsf(x[i]));
  scale_code = e4m3x2_from_f32(amax / 6.0f, 0.0f) & 0xFFu;
  const float S = e4m3_to_f32(scale_code);
  uint32_t w0 = 0, w1 = 0;
  if (S != 0.0f) {
    // E2M1(x / S) without the division: every threshold t of e2m1_from_f32
    // times S is exact (t has at most 3 significant bits, S at most 4), and a
    // BF16 x (8 significant bits) that differs from t * S differs by far more
    // than half an fp32 ulp of the quotient, so x / S rounds to t exactly when
    // x == t * S: comparing |x| with t * S takes the same decision.
    const float t0 = 0.25f * S, t1 = 0.75f * S, t2 = 1.25f * S, t3 = 1.75f * S;
    const float t4 = 2.5f * S, t5 = 3.5f * S, t6 = 5.0f * S;
    auto code = [&](float v) -> uint32_t {
      const float a = __builtin_fabsf(v);
      const uint32_t c = (a <= t0) ? 0u : (a < t1) ? 1u : (a <= t2) ? 2u : (a < t3) ? 3u
                       : (a <= t4) ? 4u : (a < t5) ? 5u : (a <= t6) ? 6u : 7u;
      return ((__float_as_uint(v) >> 28) & 0x8u) | c;
    };
#pragma unroll
    for (int i = 0; i < 8; ++i) w0 |= code(x[i]) << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) w1 |= code(x[8 + i]) << (4 * i);
  }
  return u32x2{w0, w1};
}

// Max / sum over the four 16-lane rows of a wave (lanes n, n+16, n+32, n+48),
// with the gfx950 row-swap permutes (VALU only, no LDS round trip).
__device__ __forceinline__ float max_over_rows(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

// x from lane l ^ 1, l ^ 2 (quad permutes), 7 - l and 15 - l within the row
// (half-row and row mirrors): four DPP moves bring every lane of a row of 16
// into each lane's reduction.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// wave64 reductions (full wave), every lane gets the result: within rows of
// 16 by DPP, then across the four rows by the row swaps.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));      // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_f32<0x4E>(v));      // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_f32<0x141>(v));     // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));     // row_mirror
  return max_over_rows(v);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return sum_over_rows(v);
}

}  // namespace pkd

// codec.hpp -- device-side MXFP8 codec for gfx950: E8M0 scale selection from a block
// amax, RNE + saturating FP8 encode, FP8 decode, bf16 rounding.
//
// Sources ("Low-Precision GPU Programming"):
//   "Format taxonomy": E4M3 bias 7 / 3 mantissa bits / max 448 / NaN 0x7F,0xFF, no Inf;
//                      E5M2 bias 15 / 2 mantissa bits / max 57,344 / min subnormal 2^-16.
//   "Numerical hazards": RNE with ties to even; saturating conversion to +-fmax; signed
//                      zero kept for negative values that round to zero.
//   "Microscaling: the two-row experiment": E8M0 byte c = 2^(c-127), 255 NaN; the block
//                      scale rounds amax/fmax up to a power of two, exponent >= -127,
//                      zero block -> 1.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

enum : int { kE4M3 = 0, kE5M2 = 1 };

// Exponent of fmax's leading bit: 448 = 1.75 * 2^8, 57344 = 1.75 * 2^15.
template <int F> struct Fp8;
template <> struct Fp8<kE4M3> {
  static constexpr int emax = 8;
  static constexpr uint32_t max_bits = 0x43E00000u;   // 448.0f
  static constexpr uint32_t min_normal = 0x3C800000u; // 2^-6
  static constexpr float sub_scale = 512.0f;          // 1 / 2^-9 (subnormal spacing)
  static constexpr uint32_t max_code = 0x7Eu;
  static constexpr int mant_shift = 20;               // 23 - 3
  static constexpr uint32_t exp_rebias = (127u - 7u) << 3;
};
template <> struct Fp8<kE5M2> {
  static constexpr int emax = 15;
  static constexpr uint32_t max_bits = 0x47600000u;   // 57344.0f
  static constexpr uint32_t min_normal = 0x38800000u; // 2^-14
  static constexpr float sub_scale = 65536.0f;        // 1 / 2^-16
  static constexpr uint32_t max_code = 0x7Bu;
  static constexpr int mant_shift = 21;               // 23 - 2
  static constexpr uint32_t exp_rebias = (127u - 15u) << 2;
};

// E8M0 scale byte of a block from the fp32 bit pattern of its amax (sign already
// cleared).  With amax = 1.f * 2^E, amax <= 1.75 * 2^(emax + e) holds for
// e >= E - emax when f <= 0.75 and for e >= E - emax + 1 otherwise; the byte is
// e + 127 clamped below at 0.  Subnormal amax always clamps (byte 0); zero -> 127;
// Inf/NaN -> 255.
template <int F>
__device__ __forceinline__ uint32_t scale_byte_from_amax(uint32_t abits) {
  if (abits >= 0x7F800000u) return 255u;
  if (abits == 0u) return 127u;
  int eb = (int)(abits >> 23);
  int byte = eb - Fp8<F>::emax + ((abits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return eb == 0 ? 0u : (uint32_t)(byte < 0 ? 0 : byte);
}

// E8M0 scale byte under the scale rule of the OCP Microscaling Formats (MX) Specification
// v1.0, which "Low-Precision GPU Programming", "Microscaling: the two-row experiment" names
// as the other scale-selection algorithm: e = floor(log2 amax) - emax, clamped at -127.  For a normal
// amax floor(log2 amax) is its unbiased exponent, so the byte is eb - emax clamped at 0;
// a subnormal amax always clamps.  Zero -> 127, Inf/NaN -> 255, as for the pages' rule.
// The scaled values can then exceed fmax (by less than a factor 8/7); the encoder
// saturates them (satfinite).
template <int F>
__device__ __forceinline__ uint32_t scale_byte_ocp(uint32_t abits) {
  if (abits >= 0x7F800000u) return 255u;
  if (abits == 0u) return 127u;
  const int byte = (int)(abits >> 23) - Fp8<F>::emax;
  return byte < 0 ? 0u : (uint32_t)byte;
}

// Scale rule selector: kRuleCeil is the pages' rule (amax / fmax rounded up to a power of
// two), kRuleOcp the specification's (floor(log2 amax) - emax, satfinite codes).
enum : int { kRuleCeil = 0, kRuleOcp = 1 };

template <int F, int R>
__device__ __forceinline__ uint32_t scale_byte_rule(uint32_t abits) {
  return R == kRuleOcp ? scale_byte_ocp<F>(abits) : scale_byte_from_amax<F>(abits);
}

// fp32 value of 2^-e for a finite scale byte (e = byte - 127, byte in [0, 254]):
// the biased exponent of 2^-e is 127 - e = 254 - byte, which stays in [1, 254] for
// every byte the scale rule can produce from finite data (byte <= 247).
__device__ __forceinline__ float inv_scale_from_byte(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

// RNE + saturating encode of an fp32 value (already divided by the block scale).
// Normal range: round the fp32 pattern at the FP8 mantissa width (the carry moves into
// the exponent), then re-bias.  Subnormal range: the FP8 grid is uniform with spacing
// 2^-9 / 2^-16, so round |a| / spacing to an integer (the product is exact).  The sign
// bit is copied, so negative values that round to zero give 0x80.  NaN inputs are the
// caller's concern (whole blocks are replaced).
template <int F>
__device__ __forceinline__ uint32_t encode_rne_sat(float a) {
  uint32_t u = __float_as_uint(a);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t m = u & 0x7FFFFFFFu;
  uint32_t code;
  if (m >= Fp8<F>::max_bits) {
    code = Fp8<F>::max_code;
  } else if (m < Fp8<F>::min_normal) {
    code = (uint32_t)__builtin_rintf(__uint_as_float(m) * Fp8<F>::sub_scale);
  } else {
    constexpr int s = Fp8<F>::mant_shift;
    code = ((m + ((1u << (s - 1)) - 1u) + ((m >> s) & 1u)) >> s) - Fp8<F>::exp_rebias;
  }
  return code | sign;
}

// Exact fp32 value of an FP8 code (NaN for NaN codes, +-Inf for E5M2 Inf codes).
template <int F>
__device__ __forceinline__ float decode_fp8(uint32_t c) {
  uint32_t sign = (c & 0x80u) << 24;
  uint32_t mag = c & 0x7Fu;
  float v;
  if (F == kE4M3) {
    uint32_t e = mag >> 3, m = mag & 7u;
    if (mag == 0x7Fu) return __uint_as_float(0x7FC00000u);
    v = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  } else {
    uint32_t e = mag >> 2, m = mag & 3u;
    if (e == 31u) return __uint_as_float(sign | (m == 0 ? 0x7F800000u : 0x7FC00000u));
    v = e == 0 ? (float)m * 0x1p-16f : __uint_as_float(((e + 112u) << 23) | (m << 21));
  }
  return __uint_as_float(__float_as_uint(v) | sign);
}

// fp32 value 2^(byte-127) of an E8M0 scale byte: ldexp of the subnormal 2^-127 by the byte
// (byte 0 stays 2^-127, byte 254 is 2^127, byte 255 gives +Inf), then v * 0 + v, which is v
// for every finite v and NaN for +Inf: byte 255 is NaN, with no compare.
__device__ __forceinline__ float e8m0_to_f32(uint32_t byte) {
  const float v = __builtin_amdgcn_ldexpf(__uint_as_float(0x00400000u), (int)byte);
  return __builtin_fmaf(v, 0.0f, v);
}

// Two codes of a dword (bytes 2*hi, 2*hi+1) times the scale s = e8m0_to_f32(byte), as two
// bf16 values (the dword's bits), by the format's scaled conversion
// (v_cvt_scalef32_pk_bf16_{fp8,bf8}: for every code and scale byte, 255 and the subnormal
// 2^-127 included, the bf16 RNE of the exact product code * 2^(byte-127), NaN for NaN).
template <int F>
__device__ __forceinline__ uint32_t cvt_pk_bf16(uint32_t codes, float s, bool hi) {
  if (F == kE4M3)
    return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, s, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, s, false));
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(codes, s, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(codes, s, false));
}

// bf16 round-to-nearest-even of an fp32 value (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u | ((u >> 16) & 0x8000u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace mxq

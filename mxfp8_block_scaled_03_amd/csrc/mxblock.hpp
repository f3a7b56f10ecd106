// mxblock.hpp -- one 32-element MX block in registers on gfx950: abs-max of bf16 / fp32
// values, and their codes under a chosen E8M0 scale byte.  Shared by the quantize
// kernels and the GEMM's quantizing epilogue, so both produce the same bytes.
//
// "Low-Precision GPU Programming", "Microscaling: the two-row experiment": codes are
// RNE(x / S) with the block's power-of-two scale S; "Numerical hazards": saturating RNE,
// signed zero kept.  The hardware scaled conversion (v_cvt_scalef32_pk_{fp8,bf8}_*)
// computes RNE(x / S) for a normal fp32 S; scale byte 0 (S = 2^-127) takes the software
// encoder of codec.hpp, byte 255 (a NaN/Inf block) writes 0x7F everywhere.
#pragma once
#include "codec.hpp"

namespace mxq {
namespace mxblock {

typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// Max over 32-bit patterns of the four lanes of a quad (quad_perm DPP: 1,0,3,2 then 2,3,0,1).
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  v = v > o ? v : o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  return v > o ? v : o;
}

__device__ __forceinline__ uint32_t pk_abs_max_bf16(uint32_t acc, uint32_t w) {
  v2u16 a = __builtin_bit_cast(v2u16, acc);
  v2u16 b = __builtin_bit_cast(v2u16, w & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// Encode two bf16 values (packed in one dword, element 0 in the low half) with the
// hardware scaled conversion; result bytes in the low 16 bits (hi = false) or high.
template <int F>
__device__ __forceinline__ uint32_t cvt2_bf16(uint32_t old, uint32_t w, float scale, bool hi) {
  v2s o = __builtin_bit_cast(v2s, old);
  v2bf x = __builtin_bit_cast(v2bf, w);
  v2s r;
  if (hi) {
    if (F == kE4M3) r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, x, scale, true);
    else r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(o, x, scale, true);
  } else {
    if (F == kE4M3) r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, x, scale, false);
    else r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(o, x, scale, false);
  }
  return __builtin_bit_cast(uint32_t, r);
}

template <int F>
__device__ __forceinline__ uint32_t cvt2_f32(uint32_t old, uint32_t a, uint32_t b, float scale, bool hi) {
  v2s o = __builtin_bit_cast(v2s, old);
  v2s r;
  if (hi) {
    if (F == kE4M3) r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, __uint_as_float(a), __uint_as_float(b), scale, true);
    else r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(o, __uint_as_float(a), __uint_as_float(b), scale, true);
  } else {
    if (F == kE4M3) r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, __uint_as_float(a), __uint_as_float(b), scale, false);
    else r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(o, __uint_as_float(a), __uint_as_float(b), scale, false);
  }
  return __builtin_bit_cast(uint32_t, r);
}

// 8 source values of one chunk, kept as they were loaded:
//   bf16: 4 dwords, two values each (element 2i low, 2i+1 high); f32: 8 dwords.
template <int SRC_BF16> struct Chunk;
template <> struct Chunk<1> { uint32_t w[4]; };
template <> struct Chunk<0> { uint32_t w[8]; };

template <int SRC_BF16>
__device__ __forceinline__ uint32_t value_bits(const Chunk<SRC_BF16>& c, int i) {
  if (SRC_BF16) return (i & 1) ? (c.w[i >> 1] & 0xFFFF0000u) : (c.w[i >> 1] << 16);
  return c.w[i];
}

// Codes of the 8 values of a chunk under scale byte sb (1..254: hardware conversion;
// 0: software RNE after multiplying by 2^127, exact for such tiny blocks; 255: NaN
// block, all 0x7F).  Returns 8 code bytes in two dwords.
template <int SRC_BF16, int F>
__device__ __forceinline__ void encode_chunk(const Chunk<SRC_BF16>& c, uint32_t sb, uint32_t& d0, uint32_t& d1) {
  if (sb == 255u) {
    d0 = d1 = 0x7F7F7F7Fu;
    return;
  }
  if (sb == 0u) {
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = encode_rne_sat<F>(__uint_as_float(value_bits<SRC_BF16>(c, i)) * 0x1p127f);
    d0 = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    d1 = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    return;
  }
  const float scale = __uint_as_float(sb << 23);  // 2^(sb-127)
  if (SRC_BF16) {
    d0 = cvt2_bf16<F>(0u, c.w[0], scale, false);
    d0 = cvt2_bf16<F>(d0, c.w[1], scale, true);
    d1 = cvt2_bf16<F>(0u, c.w[2], scale, false);
    d1 = cvt2_bf16<F>(d1, c.w[3], scale, true);
  } else {
    d0 = cvt2_f32<F>(0u, c.w[0], c.w[1], scale, false);
    d0 = cvt2_f32<F>(d0, c.w[2], c.w[3], scale, true);
    d1 = cvt2_f32<F>(0u, c.w[4], c.w[5], scale, false);
    d1 = cvt2_f32<F>(d1, c.w[6], c.w[7], scale, true);
  }
}

template <int SRC_BF16>
__device__ __forceinline__ uint32_t chunk_abs_max(const Chunk<SRC_BF16>& c) {
  if (SRC_BF16) {
    uint32_t m = pk_abs_max_bf16(0u, c.w[0]);
    m = pk_abs_max_bf16(m, c.w[1]);
    m = pk_abs_max_bf16(m, c.w[2]);
    m = pk_abs_max_bf16(m, c.w[3]);
    uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    return (lo > hi ? lo : hi) << 16;
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t a = c.w[i] & 0x7FFFFFFFu;
      m = m > a ? m : a;
    }
    return m;
  }
}

}  // namespace mxblock
}  // namespace mxq

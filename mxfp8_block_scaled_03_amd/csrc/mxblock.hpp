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

// Magnitude caps at fmax * S for a finite scale byte sb (1..254) whose fmax * S is a
// normal number (sb + emax <= 254, which every byte of a finite block meets): fmax is
// 1.75 * 2^emax in both formats, so the cap's significand bits are 0x60 (bf16) /
// 0x600000 (fp32).  Clamping |x| to the cap before the hardware conversion makes it
// saturate: RNE(cap / S) = fmax, and any |x| <= cap converts as before.  Only the OCP
// scale rule needs it; under the pages' rule |x| <= cap holds already.
template <int F>
__device__ __forceinline__ uint32_t clamp_pk_bf16(uint32_t w, uint32_t sb) {
  const uint32_t cap = ((sb + (uint32_t)Fp8<F>::emax) << 7) | 0x60u;
  const v2u16 m = __builtin_elementwise_min(__builtin_bit_cast(v2u16, w & 0x7FFF7FFFu),
                                            __builtin_bit_cast(v2u16, cap | (cap << 16)));
  return __builtin_bit_cast(uint32_t, m) | (w & 0x80008000u);
}

template <int F>
__device__ __forceinline__ uint32_t clamp_f32(uint32_t w, uint32_t sb) {
  const uint32_t cap = ((sb + (uint32_t)Fp8<F>::emax) << 23) | 0x600000u;
  const uint32_t m = w & 0x7FFFFFFFu;
  return (m < cap ? m : cap) | (w & 0x80000000u);
}

// Codes of the 8 values of a chunk under scale byte sb (1..254: hardware conversion;
// 0: software RNE after multiplying by 2^127, exact for such tiny blocks; 255: NaN
// block, all 0x7F).  Returns 8 code bytes in two dwords.  R = kRuleOcp clamps the
// magnitudes to fmax * S first (the software encoder saturates by itself).
template <int SRC_BF16, int F, int R = kRuleCeil>
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
  Chunk<SRC_BF16> x = c;
  if (R == kRuleOcp) {
#pragma unroll
    for (int i = 0; i < (SRC_BF16 ? 4 : 8); ++i) x.w[i] = SRC_BF16 ? clamp_pk_bf16<F>(c.w[i], sb) : clamp_f32<F>(c.w[i], sb);
  }
  if (SRC_BF16) {
    d0 = cvt2_bf16<F>(0u, x.w[0], scale, false);
    d0 = cvt2_bf16<F>(d0, x.w[1], scale, true);
    d1 = cvt2_bf16<F>(0u, x.w[2], scale, false);
    d1 = cvt2_bf16<F>(d1, x.w[3], scale, true);
  } else {
    d0 = cvt2_f32<F>(0u, x.w[0], x.w[1], scale, false);
    d0 = cvt2_f32<F>(d0, x.w[2], x.w[3], scale, true);
    d1 = cvt2_f32<F>(0u, x.w[4], x.w[5], scale, false);
    d1 = cvt2_f32<F>(d1, x.w[6], x.w[7], scale, true);
  }
}

// Codes of a 32-value block held as fp32 bit patterns (the columnwise kernels' layout)
// under scale byte sb, with the same three cases and the same clamp as encode_chunk.
template <int F, int R = kRuleCeil>
__device__ __forceinline__ void encode_block32(const uint32_t v[32], uint32_t sb, uint32_t out[8]) {
  if (sb == 255u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = 0x7F7F7F7Fu;
  } else if (sb == 0u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) w |= encode_rne_sat<F>(__uint_as_float(v[4 * i + j]) * 0x1p127f) << (8 * j);
      out[i] = w;
    }
  } else {
    const float scale = __uint_as_float(sb << 23);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = R == kRuleOcp ? clamp_f32<F>(v[4 * i + j], sb) : v[4 * i + j];
      const uint32_t w = cvt2_f32<F>(0u, a[0], a[1], scale, false);
      out[i] = cvt2_f32<F>(w, a[2], a[3], scale, true);
    }
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

// Codes of one column of 32 bf16 values held in the low (hi = false) or high halves of
// 32 dwords w[i] (row i of the block; the other half belongs to the neighbouring column):
// for a normal scale byte, pairs of rows are gathered into one packed bf16 dword
// (v_perm_b32) and converted two at a time; scale bytes 0 and 255 take encode_block32.
template <int F, int R = kRuleCeil>
__device__ __forceinline__ void encode_block32_bf16_half(const uint32_t w[32], bool hi, uint32_t sb, uint32_t out[8]) {
  if (sb == 255u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = 0x7F7F7F7Fu;
    return;
  }
  if (sb == 0u) {                                  // value by value, as encode_block32
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t v = hi ? (w[4 * i + j] & 0xFFFF0000u) : (w[4 * i + j] << 16);
        c |= encode_rne_sat<F>(__uint_as_float(v) * 0x1p127f) << (8 * j);
      }
      out[i] = c;
    }
    return;
  }
  const float scale = __uint_as_float(sb << 23);
  const uint32_t sel = hi ? 0x07060302u : 0x05040100u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t p0 = __builtin_amdgcn_perm(w[4 * j + 1], w[4 * j], sel);
    uint32_t p1 = __builtin_amdgcn_perm(w[4 * j + 3], w[4 * j + 2], sel);
    if (R == kRuleOcp) {
      p0 = clamp_pk_bf16<F>(p0, sb);
      p1 = clamp_pk_bf16<F>(p1, sb);
    }
    out[j] = cvt2_bf16<F>(cvt2_bf16<F>(0u, p0, scale, false), p1, scale, true);
  }
}

// ---- stochastic rounding ("Rounding: RNE versus stochastic rounding": between the
//      neighbouring representable values l <= |a| < u, round up with probability
//      (|a| - l) / (u - l); representable values stay)

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC 2011): ten rounds of two 32x32 -> 64-bit products (multipliers 0xD2511F53 and
// 0xCD9E8D57) whose high halves are xored with the other counter words and the key, the
// key bumped by 0x9E3779B9 / 0xBB67AE85 between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32x32 -> 64-bit multiply each (v_mad_u64_u32)
    const uint64_t p0 = (uint64_t)c[0] * 0xD2511F53u, p1 = (uint64_t)c[2] * 0xCD9E8D57u;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// The 24-bit random integers of the 32 elements of block b of line l, whose indices in
// the padded code array are n = (l * nb + b) * 32 + j: element j takes word j % 4 of
// Philox4x32-10(counter = (n / 4 low, n / 4 high, 0, 0), key = seed), top 24 bits.
__device__ __forceinline__ void block_random24(uint64_t block_index, uint64_t seed, uint32_t r[32]) {
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const uint64_t ctr = block_index * 8u + (uint64_t)g;
    uint32_t c[4] = {(uint32_t)ctr, (uint32_t)(ctr >> 32), 0u, 0u};
    philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
#pragma unroll
    for (int w = 0; w < 4; ++w) r[4 * g + w] = c[w] >> 8;
  }
}

// Stochastically rounded FP8 code of the value with fp32 bit pattern vb in a block with
// finite scale byte sb (0..254), under the 24-bit random integer r: up iff r < 2^24 * p.
// Everything is integer arithmetic on |v| = M * 2^(ev - 150) (M < 2^24), so the decision
// is exact even where |v| / S would underflow in fp32: with the FP8 spacing 2^s of the
// interval holding a = v / S, q = |a| / 2^s = M * 2^sh; the floor code comes from the
// integer part, p * 2^24 from the fraction.  The scale rule keeps |a| <= fmax.
template <int F>
__device__ __forceinline__ uint32_t encode_sr(uint32_t vb, uint32_t sb, uint32_t r) {
  constexpr int MB = F == kE4M3 ? 3 : 2;            // mantissa bits
  constexpr int BIAS = F == kE4M3 ? 7 : 15;
  constexpr int EMIN = 1 - BIAS;                    // exponent of the smallest normal
  constexpr int KB = 23 - MB;                       // fp32 mantissa bits below the code's
  const uint32_t sign = (vb >> 24) & 0x80u;
  const uint32_t mag = vb & 0x7FFFFFFFu;
  const int e = (int)sb - 127;
  const int ev0 = (int)(mag >> 23);
  const int xa0 = ev0 - 127 - e;                    // floor(log2 |a|) for an fp32-normal v
  // v an fp32 normal and a = v / S in FP8's normal range (the common case): the steps below
  // with lz = 0 and sh = -KB, so the floor code is v's exponent rebased with its top MB
  // mantissa bits, and the KB bits below them are the fraction: up iff r < frac * 2^(24 - KB)
  if (ev0 != 0 && xa0 >= EMIN) {
    const uint32_t fc = ((uint32_t)(xa0 + BIAS) << MB) | ((mag >> KB) & ((1u << MB) - 1u));
    const uint32_t frac = mag & ((1u << KB) - 1u);
    return sign | (fc + (r < (frac << (24 - KB)) ? 1u : 0u));
  }
  // v an fp32 normal with a below FP8's normal range (or zero, whose code is its sign):
  // the subnormal spacing 2^(EMIN - MB), k = -sh > KB fraction bits, floor code M >> k
  if (ev0 != 0 || mag == 0u) {
    const uint32_t M = (mag & 0x7FFFFFu) | 0x800000u;
    const int k = 150 + e + EMIN - MB - ev0;                   // fraction bits of q
    const uint32_t fc = M >> (k < 31 ? k : 31);
    // up iff r < p * 2^24: while k <= 24, p * 2^24 = frac * 2^(24 - k) with frac the low k
    // bits of M; beyond, q < 1 and r < M / 2^(k - 24) iff r < ceil(M / 2^(k - 24)), which
    // is 1 (r == 0) once k - 24 >= 24
    const int k1 = k < 24 ? k : 24;
    const uint32_t t_lo = (M & ((1u << k1) - 1u)) << (24 - k1);
    const int kk = k - 24 < 24 ? k - 24 : 24;
    const uint32_t t_hi = kk < 24 ? (M + (1u << (kk > 0 ? kk : 0)) - 1u) >> (kk > 0 ? kk : 0) : 1u;
    const uint32_t up = r < (k <= 24 ? t_lo : t_hi) ? 1u : 0u;
    return mag == 0u ? sign : sign | (fc + up);
  }
  // v an fp32 subnormal: the general steps
  const uint32_t M = ev0 ? ((mag & 0x7FFFFFu) | 0x800000u) : (mag & 0x7FFFFFu);
  const int ev = ev0 ? ev0 : 1;
  const int lz = __clz((int)M) - 8;                 // leading zeros within 24 bits
  const int xa = (23 - lz) + ev - 150 - e;          // floor(log2 |a|)
  const int s = xa >= EMIN ? xa - MB : EMIN - MB;   // spacing exponent of the interval
  const int sh = ev - 150 - e - s;                  // q = M * 2^sh
  uint32_t floor_code;
  if (xa >= EMIN) {
    const uint32_t mn = M << lz;                    // leading one at bit 23
    floor_code = ((uint32_t)(xa + BIAS) << MB) | ((mn >> (23 - MB)) & ((1u << MB) - 1u));
  } else {
    floor_code = sh >= 0 ? (M << sh) : (sh > -32 ? (M >> -sh) : 0u);
  }
  uint32_t up = 0u;
  if (sh < 0) {
    const int k = -sh;                              // fraction bits of q
    if (k <= 24) {
      const uint32_t fr = M & ((1u << k) - 1u);     // frac * 2^k
      up = r < (fr << (24 - k)) ? 1u : 0u;
    } else {                                        // q < 1: frac * 2^24 = M / 2^(k - 24)
      const int kk = k - 24;
      up = kk >= 40 ? (r == 0u ? 1u : 0u) : (((uint64_t)r << kk) < (uint64_t)M ? 1u : 0u);
    }
  }
  return sign | (floor_code + up);
}

}  // namespace mxblock
}  // namespace mxq

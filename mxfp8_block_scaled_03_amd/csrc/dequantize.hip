// dequantize.hip -- reconstruction x_hat = S * q (mx_dequantize) for gfx950.
//
// "Low-Precision GPU Programming", "One letter, two reciprocal conventions": S is the
// reconstruction scale, x_hat = S * q.  "Scale ownership and the GEMM dataflow":
// standalone dequantization stays available for debugging and fallback consumers.
// "Microscaling: the two-row experiment": E8M0 byte c is 2^(c-127), 255 is NaN.
//
// The fp32 result dec(code) * 2^(s-127) is formed with v_ldexp_f32, which is exact
// whenever the value is representable (also as an fp32 subnormal) and overflows to Inf
// at or beyond 2^128; bf16 output rounds that exact value once (RNE).
#include "codec.hpp"
#include "internal.hpp"

namespace mxq {
namespace {

constexpr int kThreads = 256;

template <int F>
__device__ __forceinline__ float dequant_one(uint32_t code, uint32_t sb) {
  float v = decode_fp8<F>(code);
  if (sb == 255u) return __uint_as_float(0x7FC00000u);
  return __builtin_amdgcn_ldexpf(v, (int)sb - 127);
}

// One thread per 8-element chunk of a line.  VEC: codes read as 8 bytes, output written
// with 16-byte stores (K % 8 == 0 and aligned pointers / leading dimensions).
template <int F, int OUT_BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t* __restrict__ codes, int64_t ld_codes,
                                                     const uint8_t* __restrict__ scales, int64_t ld_scales,
                                                     int64_t K, int64_t cpl, int64_t nchunks, void* __restrict__ dst,
                                                     int64_t ld_dst) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < nchunks; c += stride) {
    const int64_t l = c / cpl;
    const int64_t k0 = 8 * (c - l * cpl);
    const uint32_t sb = scales[l * ld_scales + k0 / 32];
    const uint8_t* cp = codes + l * ld_codes + k0;
    float v[8];
    if (VEC) {
      uint2 w = *reinterpret_cast<const uint2*>(cp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = dequant_one<F>((w.x >> (8 * i)) & 0xFFu, sb);
        v[4 + i] = dequant_one<F>((w.y >> (8 * i)) & 0xFFu, sb);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (k0 + i < K) ? dequant_one<F>(cp[i], sb) : 0.0f;
    }
    if (OUT_BF16) {
      uint16_t* d = reinterpret_cast<uint16_t*>(dst) + l * ld_dst + k0;
      if (VEC) {
        uint4 o;
        o.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
        o.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
        o.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
        o.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
        *reinterpret_cast<uint4*>(d) = o;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (k0 + i < K) d[i] = (uint16_t)f32_to_bf16_rne(v[i]);
      }
    } else {
      float* d = reinterpret_cast<float*>(dst) + l * ld_dst + k0;
      if (VEC) {
        reinterpret_cast<float4*>(d)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(d)[1] = make_float4(v[4], v[5], v[6], v[7]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (k0 + i < K) d[i] = v[i];
      }
    }
  }
}

template <int F, int OUT_BF16>
hipError_t dequant_t(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales, int64_t ld_scales, int64_t L,
                     int64_t K, void* dst, int64_t ld_dst, bool vec, hipStream_t stream) {
  const int64_t cpl = (K + 7) / 8;
  const int64_t nchunks = L * cpl;
  const int64_t need = (nchunks + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  const int grid = (int)(need < cap ? need : cap);
  if (vec)
    hipLaunchKernelGGL((k_dequant<F, OUT_BF16, true>), dim3(grid), dim3(kThreads), 0, stream, codes, ld_codes, scales,
                       ld_scales, K, cpl, nchunks, dst, ld_dst);
  else
    hipLaunchKernelGGL((k_dequant<F, OUT_BF16, false>), dim3(grid), dim3(kThreads), 0, stream, codes, ld_codes, scales,
                       ld_scales, K, cpl, nchunks, dst, ld_dst);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales, int64_t ld_scales, int fmt,
                          int64_t L, int64_t K, void* dst, int dst_bf16, int64_t ld_dst, bool vec, hipStream_t stream) {
  if (fmt == kE4M3) {
    if (dst_bf16) return dequant_t<kE4M3, 1>(codes, ld_codes, scales, ld_scales, L, K, dst, ld_dst, vec, stream);
    return dequant_t<kE4M3, 0>(codes, ld_codes, scales, ld_scales, L, K, dst, ld_dst, vec, stream);
  }
  if (dst_bf16) return dequant_t<kE5M2, 1>(codes, ld_codes, scales, ld_scales, L, K, dst, ld_dst, vec, stream);
  return dequant_t<kE5M2, 0>(codes, ld_codes, scales, ld_scales, L, K, dst, ld_dst, vec, stream);
}

}  // namespace mxq

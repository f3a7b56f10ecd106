// dequantize.hip -- reconstruction x_hat = S * q (mx_dequantize) for gfx950.
//
// "Low-Precision GPU Programming", "One letter, two reciprocal conventions": S is the
// reconstruction scale, x_hat = S * q.  "Scale ownership and the GEMM dataflow":
// standalone dequantization stays available for debugging and fallback consumers.
// "Microscaling: the two-row experiment": E8M0 byte c is 2^(c-127), 255 is NaN.
//
// The fp32 result dec(code) * 2^(s-127) is formed with v_ldexp_f32, which is exact
// whenever the value is representable (also as an fp32 subnormal) and overflows to Inf
// at or beyond 2^128; bf16 output rounds that exact value once (RNE).  The chunk and block
// kernels form bf16 output with the scaled conversion v_cvt_scalef32_pk_bf16_{fp8,bf8}
// instead, which gives the same bits for every code and scale byte.
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

// Any layout: one thread per 8-element chunk of a line, byte loads and element stores.
template <int F, int OUT_BF16>
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
    const int n = K - k0 < 8 ? (int)(K - k0) : 8;
    for (int i = 0; i < n; ++i) {
      const float v = dequant_one<F>(cp[i], sb);
      if (OUT_BF16)
        reinterpret_cast<uint16_t*>(dst)[l * ld_dst + k0 + i] = (uint16_t)f32_to_bf16_rne(v);
      else
        reinterpret_cast<float*>(dst)[l * ld_dst + k0 + i] = v;
    }
  }
}

// One lane per 32-element block, for K % 8 != 0 when codes and output are 16-byte aligned
// (every block start then is) and the code rows hold whole blocks: two 16-byte code loads,
// the scale byte, and four (bf16) or eight (fp32) 16-byte stores; a line's last block,
// which ends past K, stores element by element.
template <int F, int OUT_BF16>
__global__ __launch_bounds__(kThreads) void k_dequant_blocks(const uint8_t* __restrict__ codes, int64_t ld_codes,
                                                            const uint8_t* __restrict__ scales, int64_t ld_scales,
                                                            int64_t K, int64_t nb, int64_t nblocks,
                                                            void* __restrict__ dst, int64_t ld_dst) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < nblocks; g += stride) {
    const int64_t l = g / nb;
    const int64_t b = g - l * nb;                    // block within line l
    const uint4* cp = reinterpret_cast<const uint4*>(codes + l * ld_codes + 32 * b);
    const uint4 c0 = cp[0], c1 = cp[1];
    const uint32_t sb = scales[l * ld_scales + b];
    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const int64_t k0 = 32 * b;
    const int64_t nvalid = K - k0 < 32 ? K - k0 : 32;
    if (OUT_BF16) {
      const float s = e8m0_to_f32(sb);
      uint32_t o[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o[2 * i] = cvt_pk_bf16<F>(w[i], s, false);
        o[2 * i + 1] = cvt_pk_bf16<F>(w[i], s, true);
      }
      uint16_t* d = reinterpret_cast<uint16_t*>(dst) + l * ld_dst + k0;
      if (nvalid == 32) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          reinterpret_cast<uint4*>(d)[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
      } else {
        for (int i = 0; i < nvalid; ++i) d[i] = (uint16_t)(o[i >> 1] >> (16 * (i & 1)));
      }
    } else {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = dequant_one<F>((w[i >> 2] >> (8 * (i & 3))) & 0xFFu, sb);
      float* d = reinterpret_cast<float*>(dst) + l * ld_dst + k0;
      if (nvalid == 32) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          reinterpret_cast<float4*>(d)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      } else {
        for (int i = 0; i < nvalid; ++i) d[i] = v[i];
      }
    }
  }
}

// Dense chunks of G elements, G = 8 for bf16 and 4 for fp32 output, so that each lane's
// chunk is one 16-byte store (K % 8 == 0, 8-byte-aligned code rows, 16-byte output rows):
// lane t of a wave takes chunks t, t + 64, ... of the wave's 64 * CH, so each load and
// store instruction of the wave covers one contiguous run (64 * G code bytes, 1 KiB of
// output), and all CH chunks' loads are in flight before the first store.
template <int F, int OUT_BF16>
__global__ __launch_bounds__(kThreads) void k_dequant_chunks(const uint8_t* __restrict__ codes, int64_t ld_codes,
                                                            const uint8_t* __restrict__ scales, int64_t ld_scales,
                                                            int64_t cpl, int64_t nchunks, void* __restrict__ dst,
                                                            int64_t ld_dst) {
  constexpr int G = OUT_BF16 ? 8 : 4;                // elements per chunk: 16 bytes of output
  constexpr int CH = 32 / G;                         // chunks per lane
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t c0 = (t >> 6) * (64 * CH) + (t & 63);
  uint32_t w[CH][G / 4];
  uint32_t sb[CH];
  int64_t off[CH];                                   // element offset of the chunk in dst
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    const int64_t c = c0 + 64 * q;
    if (c < nchunks) {
      const int64_t l = c / cpl, k0 = G * (c - l * cpl);
      const uint8_t* cp = codes + l * ld_codes + k0;
      if (G == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(cp);
        w[q][0] = v.x;
        w[q][G / 4 - 1] = v.y;
      } else {
        w[q][0] = *reinterpret_cast<const uint32_t*>(cp);
      }
      sb[q] = scales[l * ld_scales + k0 / 32];
      off[q] = l * ld_dst + k0;
    }
  }
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    if (c0 + 64 * q >= nchunks) break;
    if (OUT_BF16) {
      const float s = e8m0_to_f32(sb[q]);
      const uint4 o = make_uint4(cvt_pk_bf16<F>(w[q][0], s, false), cvt_pk_bf16<F>(w[q][0], s, true),
                                 cvt_pk_bf16<F>(w[q][G / 4 - 1], s, false), cvt_pk_bf16<F>(w[q][G / 4 - 1], s, true));
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(dst) + off[q]) = o;
    } else {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = dequant_one<F>((w[q][0] >> (8 * i)) & 0xFFu, sb[q]);
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(dst) + off[q]) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

template <int F, int OUT_BF16>
hipError_t dequant_chunks_t(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales, int64_t ld_scales,
                            int64_t L, int64_t K, void* dst, int64_t ld_dst, hipStream_t stream) {
  constexpr int64_t G = OUT_BF16 ? 8 : 4;
  const int64_t cpl = K / G;
  const int64_t nchunks = L * cpl;
  const int64_t per_wg = kThreads * (32 / G);
  const int64_t grid = (nchunks + per_wg - 1) / per_wg;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_dequant_chunks<F, OUT_BF16>), dim3((unsigned)grid), dim3(kThreads), 0, stream, codes, ld_codes,
                     scales, ld_scales, cpl, nchunks, dst, ld_dst);
  return hipGetLastError();
}

template <int F, int OUT_BF16>
hipError_t dequant_blocks_t(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales, int64_t ld_scales,
                            int64_t L, int64_t K, void* dst, int64_t ld_dst, hipStream_t stream) {
  const int64_t nb = (K + 31) / 32;
  const int64_t nblocks = L * nb;
  const int64_t need = (nblocks + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cu_count() * 256;   // beyond this, threads loop
  const int grid = (int)(need < cap ? need : cap);
  hipLaunchKernelGGL((k_dequant_blocks<F, OUT_BF16>), dim3(grid), dim3(kThreads), 0, stream, codes, ld_codes, scales,
                     ld_scales, K, nb, nblocks, dst, ld_dst);
  return hipGetLastError();
}

template <int F, int OUT_BF16>
hipError_t dequant_t(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales, int64_t ld_scales, int64_t L,
                     int64_t K, void* dst, int64_t ld_dst, bool vec, hipStream_t stream) {
  constexpr int64_t E = OUT_BF16 ? 2 : 4;
  if (vec) return dequant_chunks_t<F, OUT_BF16>(codes, ld_codes, scales, ld_scales, L, K, dst, ld_dst, stream);
  // the block kernel reads whole 32-byte blocks: the code rows must hold 32 * nb bytes
  if ((uintptr_t)codes % 16 == 0 && ld_codes % 16 == 0 && ld_codes >= 32 * ((K + 31) / 32) &&
      (uintptr_t)dst % 16 == 0 && (ld_dst * E) % 16 == 0)
    return dequant_blocks_t<F, OUT_BF16>(codes, ld_codes, scales, ld_scales, L, K, dst, ld_dst, stream);
  const int64_t cpl = (K + 7) / 8;
  const int64_t nchunks = L * cpl;
  const int64_t need = (nchunks + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cu_count() * 256;   // beyond this, threads loop
  const int grid = (int)(need < cap ? need : cap);
  hipLaunchKernelGGL((k_dequant<F, OUT_BF16>), dim3(grid), dim3(kThreads), 0, stream, codes, ld_codes, scales, ld_scales,
                     K, cpl, nchunks, dst, ld_dst);
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

// gemm_common.hpp -- device helpers shared by the GEMM kernels (gemm_fp8.hip,
// gemm_exact.hip, gemm_fallback.hip): operand and LDS plumbing, the scaled FP8 -> bf16
// decode, the epilogue's SiLU and MX quantization of staged output rows, and the
// XCD-aware tile order.
//
// "Low-Precision GPU Programming", "Scale ownership and the GEMM dataflow": Y = X W with the
// product of the X-block and W-block scales inside the outer sum over 32-element K blocks;
// the epilogue applies the scale (alpha), then bias, then an activation, then the cast, and a
// producer epilogue may emit the MX codes and scales of its output for the next GEMM.
#pragma once
#include <type_traits>

#include "codec.hpp"
#include "internal.hpp"
#include "mxblock.hpp"

namespace mxq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kGroupM = 4;   // tile rows per group in the tile order
constexpr int kXcds = 8;     // accelerator complex dies (each with its own L2)

extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

// Output tile of workgroup `wg`: consecutive workgroup ids go round-robin over the XCDs,
// so tile t is given to the workgroups of one XCD first (neighbouring tiles share that
// XCD's L2), then tiles are walked in groups of kGroupM tile rows, column by column.
// Work item `wg` of `count` launched ones -> its index in XCD-major order (the items of
// one XCD consecutive).
__device__ __forceinline__ int xcd_order(int wg, int count) {
  const int xcd = wg % kXcds, local = wg / kXcds;
  const int q = count / kXcds, r = count % kXcds;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Tile number t -> tile (tm, tn): groups of kGroupM tile rows, column by column.
__device__ __forceinline__ void tile_at(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int first_m = (t / per_group) * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  tm = first_m + (t % per_group) % gsize;
  tn = (t % per_group) / gsize;
}

__device__ __forceinline__ void tile_of(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
  tile_at(xcd_order(wg, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes of LDS at a lane address plus an offset that is a constant after unrolling
// (folded into the ds_read_b128 immediate).
__device__ __forceinline__ v4i lds16(uint32_t addr, int off) {
  return *reinterpret_cast<const v4i*>(smem + addr + off);
}

// SiLU, x * sigmoid(x), in fp32 without an overflowing intermediate: with t = e^-|x| and
// r = 1 / (1 + t) from the hardware reciprocal (v_rcp_f32, ~1 ulp), x r for x >= 0 and
// (x t) r for x < 0: a few ulp from the rounded exact value (an IEEE division instead
// costs ~4 % of an FFN-up GEMM with this epilogue).
__device__ __forceinline__ float silu(float x) {
  const float t = expf(-fabsf(x));
  const float r = __builtin_amdgcn_rcpf(1.0f + t);
  return x >= 0.0f ? x * r : (x * t) * r;
}


// MX-quantize a wave's block of bf16 output values staged in LDS, along its rows: 128 rows
// of 32 * NB values at LDS offset `base`, row pitch PITCH bytes, 16-byte chunk c of row r
// stored at chunk c ^ (r & 7), values past column N staged as +0 (the zero padding of a
// partial block).  Row r, block j becomes block blk0 + j of code row row0 + r ("Microscaling:
// the two-row experiment": amax, power-of-two scale, RNE codes), written only when the row
// is < M and the block < nbq.
template <int NB, int PITCH = 64 * NB>
__device__ __forceinline__ void quantize_staged(uint32_t base, int lane, int row0, int M, int blk0, int nbq,
                                                const GemmEpilogue& ep) {
  static_assert(PITCH >= 64 * NB && PITCH % 128 == 0, "staged row pitch");
#pragma unroll 1
  for (int it = 0; it < 2 * NB; ++it) {
    const int p = 64 * it + lane, r = p / NB, j = p % NB;
    mxblock::Chunk<1> ch[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t phys = (uint32_t)((4 * j + c) ^ (r & 7));
      const v4i v = lds16(base + (uint32_t)(r * PITCH) + (phys << 4), 0);
#pragma unroll
      for (int w = 0; w < 4; ++w) ch[c].w[w] = (uint32_t)v[w];
    }
    const int row = row0 + r, b = blk0 + j;
    if (row < M && b < nbq) {
      uint32_t amax = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t a = mxblock::chunk_abs_max<1>(ch[c]);
        amax = amax > a ? amax : a;
      }
      uint32_t d[8], sb;
      if (ep.q_fmt == kE4M3) {
        sb = scale_byte_from_amax<kE4M3>(amax);
#pragma unroll
        for (int c = 0; c < 4; ++c) mxblock::encode_chunk<1, kE4M3>(ch[c], sb, d[2 * c], d[2 * c + 1]);
      } else {
        sb = scale_byte_from_amax<kE5M2>(amax);
#pragma unroll
        for (int c = 0; c < 4; ++c) mxblock::encode_chunk<1, kE5M2>(ch[c], sb, d[2 * c], d[2 * c + 1]);
      }
      uint4* dst = reinterpret_cast<uint4*>(ep.qc + (int64_t)row * ep.ld_qc + 32 * (int64_t)b);
      dst[0] = make_uint4(d[0], d[1], d[2], d[3]);
      dst[1] = make_uint4(d[4], d[5], d[6], d[7]);
      ep.qs[(int64_t)row * ep.ld_qs + b] = (uint8_t)sb;
    }
  }
}

// Keep the first `lim` bytes of a 16-byte fragment half, zero the rest.
__device__ __forceinline__ v4i mask_bytes(v4i v, int lim) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    int keep = lim - 4 * d;
    uint32_t m = keep >= 4 ? 0xFFFFFFFFu : (keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u));
    v[d] = (int)((uint32_t)v[d] & m);
  }
  return v;
}


// Eight codes (two dwords) -> eight bf16 values code * scale (exact while the product is
// inside bf16's range), with the gfx950 scaled conversion.
template <int F>
__device__ __forceinline__ v8bf codes_to_bf16(uint32_t w0, uint32_t w1, float s) {
  const v4i d = {(int)cvt_pk_bf16<F>(w0, s, false), (int)cvt_pk_bf16<F>(w0, s, true),
                 (int)cvt_pk_bf16<F>(w1, s, false), (int)cvt_pk_bf16<F>(w1, s, true)};
  return __builtin_bit_cast(v8bf, d);
}

// Exact-product accumulation: each lane decodes its codes with their block scale into
// bf16 (exact) and feeds v_mfma_f32_32x32x16_bf16, whose products are exact and whose
// sums are FP32.  Per 32-wide block, lane (i, g) holds k = 16g..16g+15 of the block:

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, v4i rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Raw buffer descriptor (stride 0) over [base, base + bytes), all fields wave-uniform.
__device__ __forceinline__ v4i rsrc_of(uint64_t base, uint32_t bytes) {
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// s_waitcnt with vmcnt(n) and expcnt / lgkmcnt left at their maxima (n < 64).
template <int n>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier ordering LDS accesses only (global DMA completion is handled by the
// explicit vmcnt waits before it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


// Buffer descriptor over an epilogue's bias array (4 * n bytes; range 0 without a bias, so
// every load through it returns zeros without touching memory; kNoBias is then its base).
__device__ const float kNoBias = -0.0f;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bias_rsrc(const float* bias, int n) {
  const int64_t bytes = bias != nullptr ? 4 * (int64_t)n : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(bias != nullptr ? bias : &kNoBias), (short)0,
                                           (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF), 0x00020000);
}

// Round-to-nearest-even float -> bf16 bits of two values, packed (lo = a), by the
// hardware conversion v_cvt_pk_bf16_f32 (the bits of f32_to_bf16_rne for every non-NaN
// value, subnormals included; NaN stays a NaN).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef float v2f_t __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  const v2f_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2bf_t));
}

}  // namespace
}  // namespace mxq

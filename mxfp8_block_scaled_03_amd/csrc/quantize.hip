// quantize.hip -- MX block quantization (mx_quantize) for gfx950.
//
// "Low-Precision GPU Programming", "Microscaling: the two-row experiment": per 32-element
// block along K take amax, choose the power-of-two scale S = 2^e that rounds amax/fmax
// upward (e >= -127; zero block -> S = 1), store e + 127 as the E8M0 byte and the codes
// RNE(x / S).  "Scale ownership and the GEMM dataflow": a partial final block is
// zero-padded.  "Scaling architectures" / "Current scaling": the amax reduction and the
// dependent cast stay on the device -- here in one pass over the data, since the MX amax
// is local to a block of 32 values.
//
// Encoding: v_cvt_scalef32_pk_{fp8,bf8}_{bf16,f32} computes RNE(x / scale) for a
// power-of-two fp32 scale; it is used for every block whose scale byte is 1..254 (the
// scale rule keeps |x / S| <= fmax, so its non-saturating overflow behaviour is never
// reached).  Scale byte 0 (S = 2^-127, not a normal fp32) takes the software encoder.
#include <type_traits>

#include "codec.hpp"
#include "internal.hpp"
#include "mxblock.hpp"

namespace mxq {
namespace {

constexpr int kThreads = 256;
using namespace mxblock;

// Load chunk: elements k0 .. k0+7 of a line starting at `line` (element pointer).
template <int SRC_BF16, bool VEC>
__device__ __forceinline__ void load_chunk(Chunk<SRC_BF16>& c, const void* line, int64_t k0, int64_t K) {
  if (VEC) {
    if (k0 < K) {
      if (SRC_BF16) {
        uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(line) + k0);
        c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(line) + k0);
        uint4 v0 = p[0], v1 = p[1];
        c.w[0] = v0.x; c.w[1] = v0.y; c.w[2] = v0.z; c.w[3] = v0.w;
        c.w[4] = v1.x; c.w[5] = v1.y; c.w[6] = v1.z; c.w[7] = v1.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < (SRC_BF16 ? 4 : 8); ++i) c.w[i] = 0u;
    }
  } else {
    if (SRC_BF16) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(line);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo = (k0 + 2 * i < K) ? p[k0 + 2 * i] : 0u;
        uint32_t hi = (k0 + 2 * i + 1 < K) ? p[k0 + 2 * i + 1] : 0u;
        c.w[i] = lo | (hi << 16);
      }
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(line);
#pragma unroll
      for (int i = 0; i < 8; ++i) c.w[i] = (k0 + i < K) ? p[k0 + i] : 0u;
    }
  }
}

// One lane per 32-element block: the lane loads the block's 64 (bf16) or 128 (fp32) bytes
// with 16-byte loads, reduces the amax in registers, encodes with 16 two-value
// conversions and stores 32 code bytes with two 16-byte stores; a wave covers 64
// consecutive blocks, so its 64 scale bytes form one contiguous run.  Blocks are
// numbered g = row * nb + b (FLAT problems are one dense run: row 0, b = g).  One block
// per thread and a large grid keep enough loads in flight to stream HBM.
template <int SRC_BF16, int F, bool FLAT, bool VEC, int R>
__global__ __launch_bounds__(kThreads) void k_quant_rows(const void* __restrict__ src, int64_t ld_src, int64_t K,
                                                        int64_t nb, int64_t nblocks, uint8_t* __restrict__ codes,
                                                        int64_t ld_codes, uint8_t* __restrict__ scales, int64_t ld_scales) {
  constexpr int ES = SRC_BF16 ? 2 : 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < nblocks; g += stride) {
    const int64_t row = FLAT ? 0 : g / nb;
    const int64_t b = FLAT ? g : g - row * nb;
    const char* line = reinterpret_cast<const char*>(src) + row * ld_src * ES;
    Chunk<SRC_BF16> c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      load_chunk<SRC_BF16, VEC>(c[q], line, 32 * b + 8 * q, FLAT ? (int64_t)INT64_MAX : K);
    uint32_t amax = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = chunk_abs_max<SRC_BF16>(c[q]);
      amax = amax > a ? amax : a;
    }
    const uint32_t sb = scale_byte_rule<F, R>(amax);
    uint32_t d[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) encode_chunk<SRC_BF16, F, R>(c[q], sb, d[2 * q], d[2 * q + 1]);
    uint4* out = reinterpret_cast<uint4*>(codes + row * ld_codes + 32 * b);
    out[0] = make_uint4(d[0], d[1], d[2], d[3]);
    out[1] = make_uint4(d[4], d[5], d[6], d[7]);
    scales[row * ld_scales + b] = (uint8_t)sb;
  }
}

// Columnwise: a workgroup stages a tile of 128 rows (4 blocks of K) x 64 columns in LDS
// (row pitch padded by one dword, which spreads the column reads over the banks), then
// thread t handles column t / 4, block t % 4: it reduces and encodes that block's 32
// values and writes its 32 codes, so the 4 threads of a column write one contiguous
// 128-byte run of the K-contiguous transposed output.
constexpr int kColTileRows = 128;
constexpr int kColTileCols = 64;

template <int SRC_BF16, int F, bool VEC, int R>
__global__ __launch_bounds__(kThreads) void k_quant_cols(const void* __restrict__ src, int64_t rows, int64_t cols,
                                                        int64_t ld_src, int64_t nb, uint8_t* __restrict__ codes,
                                                        int64_t ld_codes, uint8_t* __restrict__ scales, int64_t ld_scales) {
  typedef typename std::conditional<SRC_BF16, uint16_t, uint32_t>::type E;
  constexpr int PW = kColTileCols * (int)sizeof(E) / 4 + 1;      // row pitch in dwords
  __shared__ uint32_t tile[kColTileRows * PW];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kColTileCols;
  const E* s = reinterpret_cast<const E*>(src);
  for (int64_t ty = blockIdx.y; ty * kColTileRows < rows; ty += gridDim.y) {
    const int64_t r0 = ty * kColTileRows;
    // stage: 16-byte pieces of each tile row, written to LDS as 4 dwords
    constexpr int EPV = 16 / sizeof(E);                 // elements per 16-byte piece
    constexpr int PPR = kColTileCols / EPV;             // pieces per tile row
    for (int p = tid; p < kColTileRows * PPR; p += kThreads) {
      const int tr = p / PPR, tc = (p % PPR) * EPV;
      const int64_t r = r0 + tr, cc = c0 + tc;
      uint32_t* dst = &tile[tr * PW + tc * (int)sizeof(E) / 4];
      if (VEC && r < rows && cc + EPV <= cols) {
        const uint4 v = *reinterpret_cast<const uint4*>(s + r * ld_src + cc);
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
      } else {
        E e[EPV];
#pragma unroll
        for (int i = 0; i < EPV; ++i) e[i] = (r < rows && cc + i < cols) ? s[r * ld_src + cc + i] : (E)0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (SRC_BF16) dst[w] = (uint32_t)e[2 * w] | ((uint32_t)e[2 * w + 1] << 16);
          else dst[w] = (uint32_t)e[w];
        }
      }
    }
    __syncthreads();
    const int c = tid >> 2, kb = tid & 3;
    const int64_t col = c0 + c, b = r0 / 32 + kb;
    if (col < cols && b < nb) {
      uint32_t amax = 0;
      uint32_t v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int row = 32 * kb + i;
        uint32_t x;
        if (SRC_BF16) x = (uint32_t)reinterpret_cast<const uint16_t*>(tile)[row * PW * 2 + c] << 16;
        else x = tile[row * PW + c];
        v[i] = x;
        const uint32_t a = x & 0x7FFFFFFFu;
        amax = amax > a ? amax : a;
      }
      const uint32_t sb = scale_byte_rule<F, R>(amax);
      uint32_t out[8];
      encode_block32<F, R>(v, sb, out);
      uint4* dst = reinterpret_cast<uint4*>(codes + col * ld_codes + 32 * b);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
      scales[col * ld_scales + b] = (uint8_t)sb;
    }
    __syncthreads();
  }
}


// Both orientations from one read ("Microscaling: the two-row experiment", last
// paragraph: regrouping from 1x32 to 32x1 changes which values share a scale, so the
// columnwise codes are derived from the wide data, not from the rowwise bytes).  A
// workgroup takes a tile of 128 rows x 64 columns: thread t loads chunks (8 values) of
// rows t/8 + 32k, chunk t%8, and the four lanes holding one 32-value row block reduce it
// with DPP and write its rowwise codes and scale straight from registers; the tile also
// goes to LDS, from which the columnwise blocks are encoded exactly as in k_quant_cols.
template <int SRC_BF16, int F, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_dual(const void* __restrict__ src, int64_t rows, int64_t cols,
                                                        int64_t ld_src, uint8_t* __restrict__ rcodes, int64_t ld_rc,
                                                        uint8_t* __restrict__ rscales, int64_t ld_rs,
                                                        uint8_t* __restrict__ ccodes, int64_t ld_cc,
                                                        uint8_t* __restrict__ cscales, int64_t ld_cs) {
  typedef typename std::conditional<SRC_BF16, uint16_t, uint32_t>::type E;
  constexpr int ES = (int)sizeof(E);
  constexpr int PW = kColTileCols * ES / 4 + 1;      // LDS row pitch in dwords
  __shared__ uint32_t tile[kColTileRows * PW];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kColTileCols;
  const int64_t nb_r = (cols + 31) / 32, nb_c = (rows + 31) / 32;
  const int64_t kp_r = 32 * nb_r;
  const int tq = tid & 7;                             // chunk within the tile row
  for (int64_t ty = blockIdx.y; ty * kColTileRows < rows; ty += gridDim.y) {
    const int64_t r0 = ty * kColTileRows;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int tr = (tid >> 3) + 32 * k;
      const int64_t r = r0 + tr;
      const int64_t cc = c0 + 8 * tq;
      Chunk<SRC_BF16> ch;
      if (r < rows) {
        const char* line = reinterpret_cast<const char*>(src) + r * ld_src * ES;
        load_chunk<SRC_BF16, VEC>(ch, line, cc, cols);
      } else {
#pragma unroll
        for (int i = 0; i < (SRC_BF16 ? 4 : 8); ++i) ch.w[i] = 0u;
      }
      // tile copy for the columnwise pass
      uint32_t* dst = &tile[tr * PW + 8 * tq * ES / 4];
#pragma unroll
      for (int i = 0; i < (SRC_BF16 ? 4 : 8); ++i) dst[i] = ch.w[i];
      // rowwise block of this quad (every lane of the wave takes part in the DPP)
      const uint32_t amax = quad_max(chunk_abs_max<SRC_BF16>(ch));
      const uint32_t sb = scale_byte_from_amax<F>(amax);
      uint32_t d0, d1;
      encode_chunk<SRC_BF16, F>(ch, sb, d0, d1);
      if (r < rows && cc < kp_r) {
        *reinterpret_cast<uint2*>(rcodes + r * ld_rc + cc) = make_uint2(d0, d1);
        if ((tq & 3) == 0) rscales[r * ld_rs + (cc >> 5)] = (uint8_t)sb;
      }
    }
    __syncthreads();
    const int c = tid >> 2, kb = tid & 3;
    const int64_t col = c0 + c, b = r0 / 32 + kb;
    if (col < cols && b < nb_c) {
      uint32_t amax = 0;
      uint32_t v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int row = 32 * kb + i;
        uint32_t x;
        if (SRC_BF16) x = (uint32_t)reinterpret_cast<const uint16_t*>(tile)[row * PW * 2 + c] << 16;
        else x = tile[row * PW + c];
        v[i] = x;
        const uint32_t a = x & 0x7FFFFFFFu;
        amax = amax > a ? amax : a;
      }
      const uint32_t sb = scale_byte_from_amax<F>(amax);
      uint32_t out[8];
      encode_block32<F>(v, sb, out);
      uint4* dst = reinterpret_cast<uint4*>(ccodes + col * ld_cc + 32 * b);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
      cscales[col * ld_cs + b] = (uint8_t)sb;
    }
    __syncthreads();
  }
}
// Rowwise quantize with stochastically rounded codes: one lane per block as in
// k_quant_rows; the block's scale byte is the RNE quantizer's, its 32 codes are drawn by
// encode_sr with the block's Philox words (line l, block b -> block index l * nb + b).
template <int SRC_BF16, int F, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_rows_sr(const void* __restrict__ src, int64_t ld_src, int64_t K,
                                                           int64_t nb, int64_t nblocks, uint8_t* __restrict__ codes,
                                                           int64_t ld_codes, uint8_t* __restrict__ scales,
                                                           int64_t ld_scales, uint64_t seed) {
  constexpr int ES = SRC_BF16 ? 2 : 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < nblocks; g += stride) {
    const int64_t row = g / nb, b = g - row * nb;
    const char* line = reinterpret_cast<const char*>(src) + row * ld_src * ES;
    Chunk<SRC_BF16> c[4];
    uint32_t amax = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      load_chunk<SRC_BF16, VEC>(c[q], line, 32 * b + 8 * q, K);
      const uint32_t a = chunk_abs_max<SRC_BF16>(c[q]);
      amax = amax > a ? amax : a;
    }
    const uint32_t sb = scale_byte_from_amax<F>(amax);
    uint32_t d[8];
    if (sb == 255u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = 0x7F7F7F7Fu;
    } else {
      uint32_t r[32];
      block_random24((uint64_t)g, seed, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int el = 4 * i + j;
          w |= encode_sr<F>(value_bits<SRC_BF16>(c[el >> 3], el & 7), sb, r[el]) << (8 * j);
        }
        d[i] = w;
      }
    }
    uint4* out = reinterpret_cast<uint4*>(codes + row * ld_codes + 32 * b);
    out[0] = make_uint4(d[0], d[1], d[2], d[3]);
    out[1] = make_uint4(d[4], d[5], d[6], d[7]);
    scales[row * ld_scales + b] = (uint8_t)sb;
  }
}

// Columnwise quantize with stochastically rounded codes: the tile scheme of k_quant_cols;
// thread (column c, block kb) draws the Philox words of block index col * nb + b.
template <int SRC_BF16, int F, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_cols_sr(const void* __restrict__ src, int64_t rows, int64_t cols,
                                                           int64_t ld_src, int64_t nb, uint8_t* __restrict__ codes,
                                                           int64_t ld_codes, uint8_t* __restrict__ scales,
                                                           int64_t ld_scales, uint64_t seed) {
  typedef typename std::conditional<SRC_BF16, uint16_t, uint32_t>::type E;
  constexpr int PW = kColTileCols * (int)sizeof(E) / 4 + 1;
  __shared__ uint32_t tile[kColTileRows * PW];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kColTileCols;
  const E* s = reinterpret_cast<const E*>(src);
  for (int64_t ty = blockIdx.y; ty * kColTileRows < rows; ty += gridDim.y) {
    const int64_t r0 = ty * kColTileRows;
    constexpr int EPV = 16 / sizeof(E);
    constexpr int PPR = kColTileCols / EPV;
    for (int p = tid; p < kColTileRows * PPR; p += kThreads) {
      const int tr = p / PPR, tc = (p % PPR) * EPV;
      const int64_t r = r0 + tr, cc = c0 + tc;
      uint32_t* dst = &tile[tr * PW + tc * (int)sizeof(E) / 4];
      if (VEC && r < rows && cc + EPV <= cols) {
        const uint4 v = *reinterpret_cast<const uint4*>(s + r * ld_src + cc);
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
      } else {
        E e[EPV];
#pragma unroll
        for (int i = 0; i < EPV; ++i) e[i] = (r < rows && cc + i < cols) ? s[r * ld_src + cc + i] : (E)0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (SRC_BF16) dst[w] = (uint32_t)e[2 * w] | ((uint32_t)e[2 * w + 1] << 16);
          else dst[w] = (uint32_t)e[w];
        }
      }
    }
    __syncthreads();
    const int c = tid >> 2, kb = tid & 3;
    const int64_t col = c0 + c, b = r0 / 32 + kb;
    if (col < cols && b < nb) {
      uint32_t amax = 0;
      uint32_t v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int row = 32 * kb + i;
        uint32_t x;
        if (SRC_BF16) x = (uint32_t)reinterpret_cast<const uint16_t*>(tile)[row * PW * 2 + c] << 16;
        else x = tile[row * PW + c];
        v[i] = x;
        const uint32_t a = x & 0x7FFFFFFFu;
        amax = amax > a ? amax : a;
      }
      const uint32_t sb = scale_byte_from_amax<F>(amax);
      uint32_t out[8];
      if (sb == 255u) {
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = 0x7F7F7F7Fu;
      } else {
        uint32_t rnd[32];
        block_random24((uint64_t)col * (uint64_t)nb + (uint64_t)b, seed, rnd);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t w = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) w |= encode_sr<F>(v[4 * i + j], sb, rnd[4 * i + j]) << (8 * j);
          out[i] = w;
        }
      }
      uint4* dst = reinterpret_cast<uint4*>(codes + col * ld_codes + 32 * b);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
      scales[col * ld_scales + b] = (uint8_t)sb;
    }
    __syncthreads();
  }
}
// Codes of one 32-value block under a caller-owned scale byte sb ("Worked failure: stale
// delayed scale"): RNE-satfinite(x / S) by the exact software encoder (x / S by ldexp,
// exact unless it over- or underflows fp32, where the code is fmax or zero anyway), NaN ->
// 0x7F, sb = 255 -> the whole block 0x7F.  Counts the elements saturated (|x / S| > fmax)
// and the nonzero ones that become a zero code; returns the block's abs-max bit pattern.
// n_real: elements of the block inside the line (the rest are padding, code 0x00).
template <int F>
__device__ __forceinline__ uint32_t encode_scaled_block(const uint32_t v[32], uint32_t sb, int n_real, uint32_t out[8],
                                                        uint32_t& nclip, uint32_t& nflush) {
  uint32_t amax = 0;
  nclip = nflush = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int el = 4 * i + j;
      const uint32_t x = v[el];
      const uint32_t mag = x & 0x7FFFFFFFu;
      uint32_t c = 0u;
      if (el < n_real) {
        amax = amax > mag ? amax : mag;
        if (sb == 255u || mag > 0x7F800000u) {
          c = 0x7Fu;
        } else {
          const float a = ldexpf(__uint_as_float(x), 127 - (int)sb);
          const bool clip = (__float_as_uint(a) & 0x7FFFFFFFu) > Fp8<F>::max_bits;
          c = encode_rne_sat<F>(a);
          nclip += clip ? 1u : 0u;
          nflush += (mag != 0u && (c & 0x7Fu) == 0u) ? 1u : 0u;
        }
      } else if (sb == 255u) {
        c = 0x7Fu;
      }
      w |= c << (8 * j);
    }
    out[i] = w;
  }
  return amax;
}

// Rowwise quantize with caller-owned scale bytes: one lane per block.
template <int SRC_BF16, int F, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_rows_scaled(
    const void* __restrict__ src, int64_t ld_src, int64_t K, int64_t nb, int64_t nblocks,
    const uint8_t* __restrict__ given, int64_t ld_given, uint8_t* __restrict__ codes, int64_t ld_codes,
    float* __restrict__ amax_out, int64_t ld_amax, uint8_t* __restrict__ clipped, uint8_t* __restrict__ flushed,
    int64_t ld_diag) {
  constexpr int ES = SRC_BF16 ? 2 : 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < nblocks; g += stride) {
    const int64_t row = g / nb, b = g - row * nb;
    const char* line = reinterpret_cast<const char*>(src) + row * ld_src * ES;
    Chunk<SRC_BF16> c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) load_chunk<SRC_BF16, VEC>(c[q], line, 32 * b + 8 * q, K);
    uint32_t v[32];
#pragma unroll
    for (int el = 0; el < 32; ++el) v[el] = value_bits<SRC_BF16>(c[el >> 3], el & 7);
    const int64_t rem = K - 32 * b;
    const int n_real = rem < 32 ? (int)rem : 32;
    const uint32_t sb = given[row * ld_given + b];
    uint32_t d[8], nclip, nflush;
    const uint32_t amax = F == kE4M3 ? encode_scaled_block<kE4M3>(v, sb, n_real, d, nclip, nflush)
                                     : encode_scaled_block<kE5M2>(v, sb, n_real, d, nclip, nflush);
    uint4* out = reinterpret_cast<uint4*>(codes + row * ld_codes + 32 * b);
    out[0] = make_uint4(d[0], d[1], d[2], d[3]);
    out[1] = make_uint4(d[4], d[5], d[6], d[7]);
    if (amax_out) amax_out[row * ld_amax + b] = __uint_as_float(amax);
    if (clipped) clipped[row * ld_diag + b] = (uint8_t)nclip;
    if (flushed) flushed[row * ld_diag + b] = (uint8_t)nflush;
  }
}

// Columnwise quantize with caller-owned scale bytes: the tile scheme of k_quant_cols.
template <int SRC_BF16, int F, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_cols_scaled(
    const void* __restrict__ src, int64_t rows, int64_t cols, int64_t ld_src, int64_t nb,
    const uint8_t* __restrict__ given, int64_t ld_given, uint8_t* __restrict__ codes, int64_t ld_codes,
    float* __restrict__ amax_out, int64_t ld_amax, uint8_t* __restrict__ clipped, uint8_t* __restrict__ flushed,
    int64_t ld_diag) {
  typedef typename std::conditional<SRC_BF16, uint16_t, uint32_t>::type E;
  constexpr int PW = kColTileCols * (int)sizeof(E) / 4 + 1;
  __shared__ uint32_t tile[kColTileRows * PW];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kColTileCols;
  const E* s = reinterpret_cast<const E*>(src);
  for (int64_t ty = blockIdx.y; ty * kColTileRows < rows; ty += gridDim.y) {
    const int64_t r0 = ty * kColTileRows;
    constexpr int EPV = 16 / sizeof(E);
    constexpr int PPR = kColTileCols / EPV;
    for (int p = tid; p < kColTileRows * PPR; p += kThreads) {
      const int tr = p / PPR, tc = (p % PPR) * EPV;
      const int64_t r = r0 + tr, cc = c0 + tc;
      uint32_t* dst = &tile[tr * PW + tc * (int)sizeof(E) / 4];
      if (VEC && r < rows && cc + EPV <= cols) {
        const uint4 v = *reinterpret_cast<const uint4*>(s + r * ld_src + cc);
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
      } else {
        E e[EPV];
#pragma unroll
        for (int i = 0; i < EPV; ++i) e[i] = (r < rows && cc + i < cols) ? s[r * ld_src + cc + i] : (E)0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (SRC_BF16) dst[w] = (uint32_t)e[2 * w] | ((uint32_t)e[2 * w + 1] << 16);
          else dst[w] = (uint32_t)e[w];
        }
      }
    }
    __syncthreads();
    const int c = tid >> 2, kb = tid & 3;
    const int64_t col = c0 + c, b = r0 / 32 + kb;
    if (col < cols && b < nb) {
      uint32_t v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int row = 32 * kb + i;
        if (SRC_BF16) v[i] = (uint32_t)reinterpret_cast<const uint16_t*>(tile)[row * PW * 2 + c] << 16;
        else v[i] = tile[row * PW + c];
      }
      const int64_t rem = rows - 32 * b;
      const int n_real = rem < 32 ? (int)rem : 32;
      const uint32_t sb = given[col * ld_given + b];
      uint32_t out[8], nclip, nflush;
      const uint32_t amax = F == kE4M3 ? encode_scaled_block<kE4M3>(v, sb, n_real, out, nclip, nflush)
                                       : encode_scaled_block<kE5M2>(v, sb, n_real, out, nclip, nflush);
      uint4* dst = reinterpret_cast<uint4*>(codes + col * ld_codes + 32 * b);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
      if (amax_out) amax_out[col * ld_amax + b] = __uint_as_float(amax);
      if (clipped) clipped[col * ld_diag + b] = (uint8_t)nclip;
      if (flushed) flushed[col * ld_diag + b] = (uint8_t)nflush;
    }
    __syncthreads();
  }
}
}  // namespace

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

template <int SRC_BF16, int F, int R>
static hipError_t quant_rows_t(const void* src, int64_t rows, int64_t K, int64_t ld_src, uint8_t* codes,
                               int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool flat, bool vec,
                               hipStream_t stream) {
  const int64_t nb = (K + 31) / 32;
  const int64_t nblocks = rows * nb;
  const int64_t wg_needed = (nblocks + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cu_count() * 256;   // beyond this, threads loop
  const int grid = (int)(wg_needed < cap ? wg_needed : cap);
  if (flat && vec)
    hipLaunchKernelGGL((k_quant_rows<SRC_BF16, F, true, true, R>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src, K,
                       nb, nblocks, codes, ld_codes, scales, ld_scales);
  else if (vec)
    hipLaunchKernelGGL((k_quant_rows<SRC_BF16, F, false, true, R>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src, K,
                       nb, nblocks, codes, ld_codes, scales, ld_scales);
  else
    hipLaunchKernelGGL((k_quant_rows<SRC_BF16, F, false, false, R>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src,
                       K, nb, nblocks, codes, ld_codes, scales, ld_scales);
  return hipGetLastError();
}

template <int R>
static hipError_t quant_rows_r(const void* src, int src_bf16, int64_t rows, int64_t K, int64_t ld_src, int fmt,
                               uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool flat,
                               bool vec, hipStream_t stream) {
  if (src_bf16) {
    if (fmt == kE4M3) return quant_rows_t<1, kE4M3, R>(src, rows, K, ld_src, codes, ld_codes, scales, ld_scales, flat, vec, stream);
    return quant_rows_t<1, kE5M2, R>(src, rows, K, ld_src, codes, ld_codes, scales, ld_scales, flat, vec, stream);
  }
  if (fmt == kE4M3) return quant_rows_t<0, kE4M3, R>(src, rows, K, ld_src, codes, ld_codes, scales, ld_scales, flat, vec, stream);
  return quant_rows_t<0, kE5M2, R>(src, rows, K, ld_src, codes, ld_codes, scales, ld_scales, flat, vec, stream);
}

hipError_t launch_quant_rows(const void* src, int src_bf16, int64_t rows, int64_t K, int64_t ld_src, int fmt,
                             int rule, uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                             bool flat, bool vec, hipStream_t stream) {
  if (rule == kRuleOcp)
    return quant_rows_r<kRuleOcp>(src, src_bf16, rows, K, ld_src, fmt, codes, ld_codes, scales, ld_scales, flat, vec, stream);
  return quant_rows_r<kRuleCeil>(src, src_bf16, rows, K, ld_src, fmt, codes, ld_codes, scales, ld_scales, flat, vec, stream);
}

template <int SRC_BF16, int F, int R>
static hipError_t quant_cols_t(const void* src, int64_t rows, int64_t cols, int64_t ld_src, uint8_t* codes,
                               int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool vec, hipStream_t stream) {
  const int64_t nb = (rows + 31) / 32;
  const int64_t gx = (cols + kColTileCols - 1) / kColTileCols;
  int64_t gy = (rows + kColTileRows - 1) / kColTileRows;
  if (gy > 65535) gy = 65535;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL((k_quant_cols<SRC_BF16, F, true, R>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, stream,
                       src, rows, cols, ld_src, nb, codes, ld_codes, scales, ld_scales);
  else
    hipLaunchKernelGGL((k_quant_cols<SRC_BF16, F, false, R>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, stream,
                       src, rows, cols, ld_src, nb, codes, ld_codes, scales, ld_scales);
  return hipGetLastError();
}

template <int R>
static hipError_t quant_cols_r(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, int fmt,
                               uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool vec,
                               hipStream_t stream) {
  if (src_bf16) {
    if (fmt == kE4M3) return quant_cols_t<1, kE4M3, R>(src, rows, cols, ld_src, codes, ld_codes, scales, ld_scales, vec, stream);
    return quant_cols_t<1, kE5M2, R>(src, rows, cols, ld_src, codes, ld_codes, scales, ld_scales, vec, stream);
  }
  if (fmt == kE4M3) return quant_cols_t<0, kE4M3, R>(src, rows, cols, ld_src, codes, ld_codes, scales, ld_scales, vec, stream);
  return quant_cols_t<0, kE5M2, R>(src, rows, cols, ld_src, codes, ld_codes, scales, ld_scales, vec, stream);
}

hipError_t launch_quant_cols(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, int fmt,
                             int rule, uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool vec,
                             hipStream_t stream) {
  if (rule == kRuleOcp)
    return quant_cols_r<kRuleOcp>(src, src_bf16, rows, cols, ld_src, fmt, codes, ld_codes, scales, ld_scales, vec, stream);
  return quant_cols_r<kRuleCeil>(src, src_bf16, rows, cols, ld_src, fmt, codes, ld_codes, scales, ld_scales, vec, stream);
}

template <int SRC_BF16, int F>
static hipError_t quant_dual_t(const void* src, int64_t rows, int64_t cols, int64_t ld_src, uint8_t* rcodes,
                               int64_t ld_rc, uint8_t* rscales, int64_t ld_rs, uint8_t* ccodes, int64_t ld_cc,
                               uint8_t* cscales, int64_t ld_cs, bool vec, hipStream_t stream) {
  const int64_t gx = (cols + kColTileCols - 1) / kColTileCols;
  int64_t gy = (rows + kColTileRows - 1) / kColTileRows;
  if (gy > 65535) gy = 65535;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL((k_quant_dual<SRC_BF16, F, true>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, stream,
                       src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs);
  else
    hipLaunchKernelGGL((k_quant_dual<SRC_BF16, F, false>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, stream,
                       src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs);
  return hipGetLastError();
}

hipError_t launch_quant_dual(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, int fmt,
                             uint8_t* rcodes, int64_t ld_rc, uint8_t* rscales, int64_t ld_rs, uint8_t* ccodes,
                             int64_t ld_cc, uint8_t* cscales, int64_t ld_cs, bool vec, hipStream_t stream) {
  if (src_bf16) {
    if (fmt == kE4M3)
      return quant_dual_t<1, kE4M3>(src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs, vec, stream);
    return quant_dual_t<1, kE5M2>(src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs, vec, stream);
  }
  if (fmt == kE4M3)
    return quant_dual_t<0, kE4M3>(src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs, vec, stream);
  return quant_dual_t<0, kE5M2>(src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs, vec, stream);
}

template <int SRC_BF16, int F>
static hipError_t quant_sr_t(const void* src, int64_t rows, int64_t cols, int64_t ld_src, bool colwise,
                             uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool vec,
                             uint64_t seed, hipStream_t stream) {
  if (!colwise) {
    const int64_t nb = (cols + 31) / 32, nblocks = rows * nb;
    const int64_t wg_needed = (nblocks + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)device_cu_count() * 256;
    const int grid = (int)(wg_needed < cap ? wg_needed : cap);
    if (vec)
      hipLaunchKernelGGL((k_quant_rows_sr<SRC_BF16, F, true>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src, cols,
                         nb, nblocks, codes, ld_codes, scales, ld_scales, seed);
    else
      hipLaunchKernelGGL((k_quant_rows_sr<SRC_BF16, F, false>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src,
                         cols, nb, nblocks, codes, ld_codes, scales, ld_scales, seed);
    return hipGetLastError();
  }
  const int64_t nb = (rows + 31) / 32;
  const int64_t gx = (cols + kColTileCols - 1) / kColTileCols;
  int64_t gy = (rows + kColTileRows - 1) / kColTileRows;
  if (gy > 65535) gy = 65535;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL((k_quant_cols_sr<SRC_BF16, F, true>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       stream, src, rows, cols, ld_src, nb, codes, ld_codes, scales, ld_scales, seed);
  else
    hipLaunchKernelGGL((k_quant_cols_sr<SRC_BF16, F, false>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       stream, src, rows, cols, ld_src, nb, codes, ld_codes, scales, ld_scales, seed);
  return hipGetLastError();
}

template <int SRC_BF16, int F>
static hipError_t quant_scaled_t(const void* src, int64_t rows, int64_t cols, int64_t ld_src, bool colwise,
                                 const uint8_t* given, int64_t ld_given, uint8_t* codes, int64_t ld_codes,
                                 float* amax, int64_t ld_amax, uint8_t* clipped, uint8_t* flushed, int64_t ld_diag,
                                 bool vec, hipStream_t stream) {
  if (!colwise) {
    const int64_t nb = (cols + 31) / 32, nblocks = rows * nb;
    const int64_t wg_needed = (nblocks + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)device_cu_count() * 256;
    const int grid = (int)(wg_needed < cap ? wg_needed : cap);
    if (vec)
      hipLaunchKernelGGL((k_quant_rows_scaled<SRC_BF16, F, true>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src,
                         cols, nb, nblocks, given, ld_given, codes, ld_codes, amax, ld_amax, clipped, flushed, ld_diag);
    else
      hipLaunchKernelGGL((k_quant_rows_scaled<SRC_BF16, F, false>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src,
                         cols, nb, nblocks, given, ld_given, codes, ld_codes, amax, ld_amax, clipped, flushed, ld_diag);
    return hipGetLastError();
  }
  const int64_t nb = (rows + 31) / 32;
  const int64_t gx = (cols + kColTileCols - 1) / kColTileCols;
  int64_t gy = (rows + kColTileRows - 1) / kColTileRows;
  if (gy > 65535) gy = 65535;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL((k_quant_cols_scaled<SRC_BF16, F, true>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       stream, src, rows, cols, ld_src, nb, given, ld_given, codes, ld_codes, amax, ld_amax, clipped,
                       flushed, ld_diag);
  else
    hipLaunchKernelGGL((k_quant_cols_scaled<SRC_BF16, F, false>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       stream, src, rows, cols, ld_src, nb, given, ld_given, codes, ld_codes, amax, ld_amax, clipped,
                       flushed, ld_diag);
  return hipGetLastError();
}

hipError_t launch_quant_scaled(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, bool colwise,
                               int fmt, const uint8_t* given, int64_t ld_given, uint8_t* codes, int64_t ld_codes,
                               float* amax, int64_t ld_amax, uint8_t* clipped, uint8_t* flushed, int64_t ld_diag,
                               bool vec, hipStream_t stream) {
  if (src_bf16) {
    if (fmt == kE4M3)
      return quant_scaled_t<1, kE4M3>(src, rows, cols, ld_src, colwise, given, ld_given, codes, ld_codes, amax, ld_amax,
                                      clipped, flushed, ld_diag, vec, stream);
    return quant_scaled_t<1, kE5M2>(src, rows, cols, ld_src, colwise, given, ld_given, codes, ld_codes, amax, ld_amax,
                                    clipped, flushed, ld_diag, vec, stream);
  }
  if (fmt == kE4M3)
    return quant_scaled_t<0, kE4M3>(src, rows, cols, ld_src, colwise, given, ld_given, codes, ld_codes, amax, ld_amax,
                                    clipped, flushed, ld_diag, vec, stream);
  return quant_scaled_t<0, kE5M2>(src, rows, cols, ld_src, colwise, given, ld_given, codes, ld_codes, amax, ld_amax,
                                  clipped, flushed, ld_diag, vec, stream);
}

hipError_t launch_quant_sr(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, bool colwise,
                           int fmt, uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool vec,
                           uint64_t seed, hipStream_t stream) {
  if (src_bf16) {
    if (fmt == kE4M3)
      return quant_sr_t<1, kE4M3>(src, rows, cols, ld_src, colwise, codes, ld_codes, scales, ld_scales, vec, seed, stream);
    return quant_sr_t<1, kE5M2>(src, rows, cols, ld_src, colwise, codes, ld_codes, scales, ld_scales, vec, seed, stream);
  }
  if (fmt == kE4M3)
    return quant_sr_t<0, kE4M3>(src, rows, cols, ld_src, colwise, codes, ld_codes, scales, ld_scales, vec, seed, stream);
  return quant_sr_t<0, kE5M2>(src, rows, cols, ld_src, colwise, codes, ld_codes, scales, ld_scales, vec, seed, stream);
}

}  // namespace mxq

// gemm.hip -- block-scaled FP8 GEMM (mx_gemm) on gfx950 scaled MFMA.
//
// "Low-Precision GPU Programming", "Scale ownership and the GEMM dataflow": Y = X W; with
// 32-element blocks along K the product of the X-block and W-block scales stays inside
// the outer sum over blocks, a partial final block is zero-padded, and block-scaled
// matrix instructions may consume the scale operands directly; summation order and
// internal precision are implementation-defined.  "Accumulator type isn't the whole
// arithmetic contract": accumulation is FP32.  "Hardware support and kernel ABI
// contracts": X row-major (1x32 groups), W column-major packed (32x1 groups), E8M0
// scales, epilogue applies the scale (alpha), then bias, then the output cast.
//
// Matrix core: v_mfma_scale_f32_32x32x64_f8f6f4.  Its operand layout (measured on
// gfx950): lane l = 32*g + i supplies row i of A (column i of B); its 32 bytes are two
// 16-byte halves holding k = 16g..16g+15 and k = 32+16g..32+16g+15 of the 64-wide K
// step, and its scale operand is the E8M0 byte of block g (k = 32g..32g+31) of that row,
// taken from byte 0 or 2 of the register by opsel.  Output: lane l, register r holds
// D[8*(r/4) + 4*g + r%4][i].
//
// Fallback kernel (scale rows that are not 16-byte aligned, both accumulation modes).
// Tiling: 256x256 output tile per workgroup of 4 waves (2x2 waves of 128x128), K step of
// 128 bytes.  Code tiles move global -> LDS with buffer_load ... lds (16 bytes per lane,
// no VGPR staging), double-buffered, with a 16-byte-chunk XOR swizzle so the fragment
// reads (ds_read_b128) are bank-conflict free.  Out-of-range rows and K positions past the
// row read as zero through the buffer descriptor's bound; code bytes at k >= K inside the
// last step are masked in registers and scale bytes of blocks >= nb are replaced by 127
// (a finite 1.0, so zero codes contribute exactly zero).  Workgroups are mapped to tiles
// XCD-first (consecutive tiles on the same XCD share its L2), then in groups of 4 tile rows.
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

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kTileBytes = BM * BK;      // 32 KiB: one operand tile of one stage
constexpr int kOffB = 2 * kTileBytes;    // LDS: A stage 0 | A stage 1 | B stage 0 | B stage 1
constexpr int kLdsBytes = 4 * kTileBytes;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes of LDS at a lane address plus an offset that is a constant after unrolling
// (folded into the ds_read_b128 immediate).
__device__ __forceinline__ v4i lds16(uint32_t addr, int off) {
  return *reinterpret_cast<const v4i*>(smem + addr + off);
}

// SiLU, x * sigmoid(x), in fp32 without an overflowing intermediate: with t = e^-|x|,
// x / (1 + t) for x >= 0 and x * t / (1 + t) for x < 0.
__device__ __forceinline__ float silu(float x) {
  const float t = expf(-fabsf(x));
  return x >= 0.0f ? x / (1.0f + t) : x * t / (1.0f + t);
}


// MX-quantize a wave's block of bf16 output values staged in LDS, along its rows: 128 rows
// of 32 * NB values at LDS offset `base`, row pitch 64 * NB bytes, 16-byte chunk c of row r
// stored at chunk c ^ (r & 7), values past column N staged as +0 (the zero padding of a
// partial block).  Row r, block j becomes block blk0 + j of code row row0 + r ("Microscaling:
// the two-row experiment": amax, power-of-two scale, RNE codes), written only when the row
// is < M and the block < nbq.
template <int NB>
__device__ __forceinline__ void quantize_staged(uint32_t base, int lane, int row0, int M, int blk0, int nbq,
                                                const GemmEpilogue& ep) {
  constexpr int PITCH = 64 * NB;
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

// Scale operand of one fragment row for K step t: byte 0 = block 4t+g, byte 2 = block
// 4t+2+g (g = lane / 32).  Blocks past the end read a valid byte and are replaced by 127
// (scale 1.0: their codes are zero, so they contribute exactly zero).
__device__ __forceinline__ uint32_t load_scale_pair(const uint8_t* rowp, int t, int g, int nb) {
  const int b0 = 4 * t + g, b1 = b0 + 2;
  uint32_t s0 = rowp[min(b0, nb - 1)];
  uint32_t s1 = rowp[min(b1, nb - 1)];
  s0 = b0 < nb ? s0 : 127u;
  s1 = b1 < nb ? s1 : 127u;
  return s0 | (s1 << 16);
}

// Per-lane LDS addresses of the fragment halves: [kk][half] for A, then for B.  The
// 16-byte chunk c of tile row r sits at r*128 + 16*(c ^ (r & 7)); fragment row r of this
// lane is (wave row base) + 32*f + li, so (r & 7) = (li & 7) and f only adds 4096*f.
struct FragAddr {
  uint32_t a[2][2], b[2][2];
};

template <int FA, int FB>
__device__ __forceinline__ void compute_step(const FragAddr& fa, uint32_t so, const uint32_t (&sa)[4],
                                             const uint32_t (&sb)[4], v16f (&acc)[4][4]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    v8i a[4], b[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      v4i alo = lds16(fa.a[kk][0] + so, 4096 * f);
      v4i ahi = lds16(fa.a[kk][1] + so, 4096 * f);
      v4i blo = lds16(fa.b[kk][0] + so, 4096 * f);
      v4i bhi = lds16(fa.b[kk][1] + so, 4096 * f);
      a[f] = __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7);
      b[f] = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int fj = 0; fj < 4; ++fj) {
        if (kk == 0)
          acc[fi][fj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[fi], b[fj], acc[fi][fj], FA, FB, 0,
                                                                        (int)sa[fi], 0, (int)sb[fj]);
        else
          acc[fi][fj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[fi], b[fj], acc[fi][fj], FA, FB, 2,
                                                                        (int)sa[fi], 2, (int)sb[fj]);
      }
  }
}

// The four E8M0 bytes of K step t (blocks 4t..4t+3) of one row, byte b = block 4t+b;
// blocks past the end read as 127.
__device__ __forceinline__ uint32_t load_scale_quad(const uint8_t* rowp, int t, int nb) {
  uint32_t q = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int blk = 4 * t + b;
    uint32_t v = rowp[min(blk, nb - 1)];
    q |= (blk < nb ? v : 127u) << (8 * b);
  }
  return q;
}

// fp32 value 2^(byte-127) of an E8M0 byte (byte 0 is the fp32 subnormal 2^-127; 255 NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t byte) {
  return __uint_as_float(byte == 0 ? 0x00400000u : (byte == 255 ? 0x7FC00000u : byte << 23));
}

// Eight codes (two dwords) -> eight bf16 values code * scale (exact while the product is
// inside bf16's range), with the gfx950 scaled conversion.
template <int F>
__device__ __forceinline__ v8bf codes_to_bf16(uint32_t w0, uint32_t w1, float s) {
  v2bf p0, p1, p2, p3;
  if (F == kE4M3) {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true);
  } else {
    p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, s, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, s, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, s, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, s, true);
  }
  typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
  v4bf lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  v4bf hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Exact-product accumulation: each lane decodes its codes with their block scale into
// bf16 (exact) and feeds v_mfma_f32_32x32x16_bf16, whose products are exact and whose
// sums are FP32.  Per 32-wide block, lane (i, g) holds k = 16g..16g+15 of the block:
// bytes 0..7 go to the first 16-wide MFMA, bytes 8..15 to the second (A and B lanes
// use the same assignment, so each MFMA contracts a matching set of 16 k).
template <int FA, int FB>
__device__ __forceinline__ void compute_step_exact(const FragAddr& fa, uint32_t so, const uint32_t (&sqa)[4],
                                                   const uint32_t (&sqb)[4], v16f (&acc)[4][4]) {
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    v4i ra[4], rb[4];
    float sa[4], sb[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      ra[f] = lds16(fa.a[blk >> 1][blk & 1] + so, 4096 * f);
      rb[f] = lds16(fa.b[blk >> 1][blk & 1] + so, 4096 * f);
      sa[f] = e8m0_to_f32((sqa[f] >> (8 * blk)) & 0xFFu);
      sb[f] = e8m0_to_f32((sqb[f] >> (8 * blk)) & 0xFFu);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8bf a[4], b[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        a[f] = codes_to_bf16<FA>((uint32_t)ra[f][2 * h], (uint32_t)ra[f][2 * h + 1], sa[f]);
        b[f] = codes_to_bf16<FB>((uint32_t)rb[f][2 * h], (uint32_t)rb[f][2 * h + 1], sb[f]);
      }
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int fj = 0; fj < 4; ++fj)
          acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fi], b[fj], acc[fi][fj], 0, 0, 0);
    }
  }
}

// Zero the code bytes at k >= krem of every row of both tiles of one stage (the last,
// partial K step), in place in LDS.  Thread t owns tile row t of A and of B.
__device__ __forceinline__ void mask_tail(uint32_t so, int krem) {
  const int r = threadIdx.x;
  const uint32_t x = r & 7;
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    uint8_t* row = smem + (op ? kOffB : 0) + so + r * BK;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int lim = krem - 16 * c;
      if (lim < 16) {
        v4i* p = reinterpret_cast<v4i*>(row + ((c ^ x) << 4));
        *p = mask_bytes(*p, lim);
      }
    }
  }
}

template <int MODE, int FA, int FB>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(int M, int N, int K, int tiles_m, int tiles_n,
                                                     const uint8_t* __restrict__ xc, int64_t ld_x,
                                                     const uint8_t* __restrict__ xs, int64_t ld_xs,
                                                     const uint8_t* __restrict__ wc, int64_t ld_w,
                                                     const uint8_t* __restrict__ ws, int64_t ld_ws,
                                                     const GemmEpilogue ep) {
  // ---- tile selection: XCD-first, then grouped rows
  const int ntiles = tiles_m * tiles_n;
  const int wg = blockIdx.x;
  int t;
  {
    const int xcd = wg % kXcds, local = wg / kXcds;
    const int q = ntiles / kXcds, r = ntiles % kXcds;
    t = xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  }
  const int per_group = kGroupM * tiles_n;
  const int group = t / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (t % per_group) % gsize;
  const int tn = (t % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int li = lane & 31, lg = lane >> 5;
  const int Kp = 32 * ((K + 31) / 32);
  const int nb = Kp / 32;
  const int nsteps = (K + BK - 1) / BK;
  const int krem_last = K - (nsteps - 1) * BK;     // valid bytes in the last step
  const bool tail = (K % BK) != 0;

  // ---- global -> LDS: buffer descriptors over the valid bytes of this tile's rows
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const uint8_t* a_base = xc + (int64_t)m0 * ld_x;
  const uint8_t* b_base = wc + (int64_t)n0 * ld_w;
  const uint32_t a_bytes = (uint32_t)((int64_t)(rows_a - 1) * ld_x + Kp);
  const uint32_t b_bytes = (uint32_t)((int64_t)(rows_b - 1) * ld_w + Kp);
  // load n of this wave fills LDS chunks (wid*8+n)*64 + lane: tile row 64*wid + 8n + lane/8,
  // physical chunk lane&7, logical chunk (lane&7) ^ (lane>>3)
  const int lrow = 64 * wid + (lane >> 3);
  const int lchunk = (lane & 7) ^ (lane >> 3);
  const uint32_t voff_a = (uint32_t)(lrow * ld_x + lchunk * 16);
  const uint32_t voff_b = (uint32_t)(lrow * ld_w + lchunk * 16);
  const uint32_t step_a = (uint32_t)(8 * ld_x), step_b = (uint32_t)(8 * ld_w);

  auto issue = [&](int step, int stage) {
    const uint32_t kb = (uint32_t)step * BK;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base + kb, a_bytes - kb);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base + kb, b_bytes - kb);
    uint8_t* la = smem + stage * kTileBytes + wid * 8 * 1024;
    uint8_t* lb = smem + kOffB + stage * kTileBytes + wid * 8 * 1024;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(la + n * 1024), 16, voff_a + n * step_a, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(lb + n * 1024), 16, voff_b + n * step_b, 0, 0, 0);
    }
  };

  // ---- fragment addresses in LDS
  FragAddr fa;
  {
    const uint32_t x = li & 7;
    const uint32_t ra = (uint32_t)(wm * 128 + li) * BK, rb = (uint32_t)(wn * 128 + li) * BK + kOffB;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t c = (uint32_t)(4 * kk + 2 * h + lg);
        fa.a[kk][h] = ra + ((c ^ x) << 4);
        fa.b[kk][h] = rb + ((c ^ x) << 4);
      }
  }

  // ---- scale bytes of this lane's fragment rows (rows past the edge clamped in range;
  //      their results are never stored)
  const uint8_t* xs_tile = xs + (int64_t)m0 * ld_xs;
  const uint8_t* ws_tile = ws + (int64_t)n0 * ld_ws;
  uint32_t xs_off[4], ws_off[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    xs_off[f] = (uint32_t)(min(wm * 128 + 32 * f + li, rows_a - 1) * ld_xs);
    ws_off[f] = (uint32_t)(min(wn * 128 + 32 * f + li, rows_b - 1) * ld_ws);
  }

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // scale operands of the current step: MODE 0 holds blocks (4t+g, 4t+2+g) for the
  // scaled MFMA, MODE 1 the four bytes of the step
  auto scales_of = [&](const uint8_t* rowp, int t_) {
    return MODE == 0 ? load_scale_pair(rowp, t_, lg, nb) : load_scale_quad(rowp, t_, nb);
  };
  uint32_t sa[4], sb[4];
  if (nsteps > 0) {
    issue(0, 0);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      sa[f] = scales_of(xs_tile + xs_off[f], 0);
      sb[f] = scales_of(ws_tile + ws_off[f], 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // K loop: step s lives in stage s & 1 while step s+1 streams into the other stage
  for (int s = 0; s < nsteps; ++s) {
    const uint32_t so = (uint32_t)(s & 1) * kTileBytes;
    if (s + 1 < nsteps) issue(s + 1, (s + 1) & 1);
    const int tn_ = min(s + 1, nsteps - 1);
    uint32_t na[4], nbx[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      na[f] = scales_of(xs_tile + xs_off[f], tn_);
      nbx[f] = scales_of(ws_tile + ws_off[f], tn_);
    }
    if (tail && s == nsteps - 1) {
      mask_tail(so, krem_last);
      __syncthreads();
    }
    if (MODE == 0)
      compute_step<FA, FB>(fa, so, sa, sb, acc);
    else
      compute_step_exact<FA, FB>(fa, so, sa, sb, acc);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int f = 0; f < 4; ++f) { sa[f] = na[f]; sb[f] = nbx[f]; }
  }

  // ---- epilogue: v = act(alpha * acc + bias[col]) in place (lane (g, i) holds column
  //      32 fj + i, row 32 fi + 8 (r / 4) + 4 g + r % 4 of the wave's 128x128 block); y = v
  //      rounded once to its type; the MX codes of bf16(v) along rows
  {
    const bool has_bias = ep.bias != nullptr;
#pragma unroll
    for (int fj = 0; fj < 4; ++fj) {
      const int col = n0 + wn * 128 + 32 * fj + li;
      const float bv = (has_bias && col < N) ? ep.bias[col] : 0.0f;
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[fi][fj][r] = has_bias ? __builtin_fmaf(ep.alpha, acc[fi][fj][r], bv) : ep.alpha * acc[fi][fj][r];
    }
    if (ep.act) {
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int fj = 0; fj < 4; ++fj)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[fi][fj][r] = silu(acc[fi][fj][r]);
    }
  }
  if (ep.y) {
#pragma unroll
    for (int fj = 0; fj < 4; ++fj) {
      const int col = n0 + wn * 128 + 32 * fj + li;
#pragma unroll
      for (int fi = 0; fi < 4; ++fi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 128 + 32 * fi + 8 * (r >> 2) + 4 * lg + (r & 3);
          if (row < M && col < N) {
            if (ep.y_bf16)
              reinterpret_cast<uint16_t*>(ep.y)[(int64_t)row * ep.ld_y + col] =
                  (uint16_t)f32_to_bf16_rne(acc[fi][fj][r]);
            else
              reinterpret_cast<float*>(ep.y)[(int64_t)row * ep.ld_y + col] = acc[fi][fj][r];
          }
        }
      }
    }
  }
  if (ep.qc) {
    // the loop's last barrier has retired every LDS read and DMA of the main loop; each
    // wave stages bf16(v) of its block in its own 32 KiB, columns >= N as +0
    const uint32_t wbase = (uint32_t)wid * 32768u;
#pragma unroll
    for (int fj = 0; fj < 4; ++fj) {
      const int cw = 32 * fj + li;
      const bool in = n0 + wn * 128 + cw < N;
#pragma unroll
      for (int fi = 0; fi < 4; ++fi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rw = 32 * fi + 8 * (r >> 2) + 4 * lg + (r & 3);
          const uint32_t addr = wbase + (uint32_t)(rw * 256) + ((uint32_t)((cw >> 3) ^ (rw & 7)) << 4) +
                                (uint32_t)((2 * cw) & 15);
          *reinterpret_cast<uint16_t*>(smem + addr) = in ? (uint16_t)f32_to_bf16_rne(acc[fi][fj][r]) : (uint16_t)0;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    quantize_staged<4>(wbase, lane, m0 + wm * 128, M, (n0 + wn * 128) / 32, (N + 31) / 32, ep);
  }
}

// ---------------------------------------------------------------------------------------
// Ping-pong kernel (both accumulation modes; 16-byte aligned scale rows).
//
// 8 waves, 256x256 output tile, 64-byte K steps, 4 LDS code stages.  Waves w and w+4
// share a SIMD; waves 0-3 (group 0) own output rows 0-127 of the tile and waves 4-7
// (group 1) rows 128-255, each wave a 128x64 block (4x2 MFMA tiles, 128 accumulator
// registers).  The two groups alternate between a memory phase (issue the DMA of step
// t+3, read step t's fragments and scales from LDS) and a compute phase (8 scaled MFMAs),
// with one workgroup barrier between phases and group 1 shifted by one phase, so on every
// SIMD one wave feeds the matrix core while the other waits on LDS.
//
// A code stage holds both tiles of one step, 256 rows x 64 bytes each, 16-byte chunk c
// of row r stored at chunk c ^ ((r >> 2) & 3), which makes the ds_read_b128 fragment
// reads conflict free.  Scales travel separately, 16 bytes (8 steps) per row at a time,
// into a two-slot ring.  Tiles and scales move global -> LDS by buffer_load ... lds
// issued from inline assembly, their completion tracked by explicit vmcnt waits (the
// compiler would otherwise wait for every LDS DMA before each LDS read).  Bytes past a
// row's codes and rows past the edge read as zero through the buffer bound; in the last,
// partial step the code bytes at k >= K are zeroed in registers and the scale of a block
// >= nb is replaced by 127.  The MFMA takes W as its A operand and X as its B operand, so
// a lane ends up holding four consecutive output columns of one row; interior tiles are
// written through LDS as 16-byte row segments.  Requires 16-byte aligned scale rows
// (scale base and leading dimension).
//
// The exact-product mode (EXACT) splits each step into two half steps, one per 32-K block,
// decodes the codes to bf16 with their block scale in its memory phases and runs bf16 MFMAs
// in its compute phases (see memory_half / compute_half).  With K a multiple of 64 (!TAIL)
// every step runs through one loop; otherwise the matrix-core mode peels the last, masked
// step and the exact mode masks it inside the loop.
namespace pp {

constexpr int kThreads = 512;
constexpr int kStages = 4;
constexpr int kCodeBytes = 256 * 64;            // one operand's codes in one stage
constexpr int kOffB = kCodeBytes;
constexpr int kStageBytes = 2 * kCodeBytes;     // 32 KiB
constexpr int kOffScale = kStages * kStageBytes;
constexpr int kScaleSlot = 2 * 256 * 16;        // A then B: 256 rows x 16 bytes each
constexpr int kOffJunk = kOffScale + 2 * kScaleSlot;    // target of the idle scale loads
constexpr int kLdsBytes = kOffJunk + 1024;               // 145 KiB
constexpr int kEpiWaveBytes = 16384;            // per-wave epilogue staging (in the code stages)

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

struct Dma {
  uint64_t a_base, b_base, s_base;   // tile row 0 of X codes, W codes, this wave's scales
  uint32_t a_bytes, b_bytes, s_bytes;
  uint32_t voff_a0, voff_a1, voff_b0, voff_b1, voff_s;
  uint32_t lds_a, lds_b, lds_s;      // LDS destinations (code stage 0, scale slot 0)
  uint32_t lds_junk;
  int T;
};

// Every step's DMA is 5 loads per wave, so the waits below are constants: kLoadsPerStep.
// Step s (K bytes 64s..64s+63) goes into code stage s % 4: this wave's 32 rows of each
// code tile (two 16-row loads per operand); every 8th step the fifth load brings this
// wave's 64 scale rows of the next 8 steps (16 bytes per row) into scale slot (s / 8) % 2,
// the other steps it is an empty load into a junk area.  Steps s >= T get an empty buffer
// range: they only write zeros into a stage (or scale slot) that is never read again.
// Keeping every step's issue pattern identical and branch free also keeps each phase in
// one basic block, where the scheduling barriers hold the MFMAs in place.
constexpr int kLoadsPerStep = 5;
struct StepDma {
  v4i ra, rb;
  uint32_t so;
};

__device__ __forceinline__ StepDma step_dma(const Dma& d, int s) {
  const bool live = s < d.T;
  const uint32_t kb = live ? 64u * (uint32_t)s : 0u;
  return StepDma{rsrc_of(d.a_base + kb, live ? d.a_bytes - kb : 0u), rsrc_of(d.b_base + kb, live ? d.b_bytes - kb : 0u),
                 (uint32_t)(s & 3) * kStageBytes};
}

__device__ __forceinline__ void issue_code(const Dma& d, const StepDma& sd, int n) {
  if (n == 0) dma16(d.lds_a + sd.so, d.voff_a0, sd.ra);
  if (n == 1) dma16(d.lds_a + sd.so + 1024, d.voff_a1, sd.ra);
  if (n == 2) dma16(d.lds_b + sd.so, d.voff_b0, sd.rb);
  if (n == 3) dma16(d.lds_b + sd.so + 1024, d.voff_b1, sd.rb);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// dma16 placed between two MFMAs: it names `after` (an operand of the MFMAs before it)
// and `before` (an operand of the MFMAs after it) as read-write operands it never touches,
// which orders it after the last reader of `after` and before the first reader of
// `before` without any hardware dependency.  (Only operands are named: naming an MFMA
// result would make the compiler copy it while the MFMA is still writing it.)
template <typename V>
__device__ __forceinline__ void dma16_between(uint32_t lds, uint32_t voff, v4i rsrc, V& after, V& before) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %3, %4, 0 offen lds"
               : "+v"(after), "+v"(before)
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// The same after the last MFMA that reads `after`.
template <typename V>
__device__ __forceinline__ void dma16_after(uint32_t lds, uint32_t voff, v4i rsrc, V& after) {
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds"
               : "+v"(after)
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void issue_scales(const Dma& d, int s) {
  const bool real = (s & 7) == 0;
  const bool live = real && s < d.T;
  const uint32_t ub = live ? 2u * (uint32_t)s : 0u;    // 16 bytes per 8 steps
  const v4i rs = rsrc_of(d.s_base + ub, live ? d.s_bytes - ub : 0u);
  dma16(real ? d.lds_s + (uint32_t)((s >> 3) & 1) * kScaleSlot : d.lds_junk, d.voff_s, rs);
}

__device__ __forceinline__ void issue_step(const Dma& d, int s) {
  const StepDma sd = step_dma(d, s);
#pragma unroll
  for (int n = 0; n < 4; ++n) issue_code(d, sd, n);
  issue_scales(d, s);
}

// Round-to-nearest-even float -> bf16 bits of two values, packed (lo = a).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
}

template <int FA, int FB, bool EXACT, bool TAIL>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_pp(int M, int N, int K, int tiles_m, int tiles_n,
                                                        const uint8_t* __restrict__ xc, int64_t ld_x,
                                                        const uint8_t* __restrict__ xs, int64_t ld_xs,
                                                        const uint8_t* __restrict__ wc, int64_t ld_w,
                                                        const uint8_t* __restrict__ ws, int64_t ld_ws,
                                                        const GemmEpilogue ep) {
  // ---- tile selection: XCD-first, then grouped rows
  const int ntiles = tiles_m * tiles_n;
  const int wg = blockIdx.x;
  int t;
  {
    const int xcd = wg % kXcds, local = wg / kXcds;
    const int q = ntiles / kXcds, r = ntiles % kXcds;
    t = xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  }
  const int per_group = kGroupM * tiles_n;
  const int group = t / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (t % per_group) % gsize;
  const int tn = (t % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gp = wid >> 2, wq = wid & 3;
  const int li = lane & 31, lg = lane >> 5;
  const int Kp = 32 * ((K + 31) / 32);
  const int nb = Kp / 32;
  const int T = (K + 63) / 64;
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)smem;

  // ---- DMA set-up: wave w loads rows 32w..32w+31 of both code tiles; load n covers rows
  //      32w + 16n + lane/4, physical chunk lane & 3 holding logical chunk
  //      (lane & 3) ^ ((row >> 2) & 3).  Scales: waves 0-3 rows 64w + lane of X, waves 4-7
  //      rows 64(w-4) + lane of W.
  Dma d;
  {
    d.T = T;
    d.a_base = (uint64_t)(uintptr_t)(xc + (int64_t)m0 * ld_x);
    d.b_base = (uint64_t)(uintptr_t)(wc + (int64_t)n0 * ld_w);
    d.a_bytes = (uint32_t)((int64_t)(rows_a - 1) * ld_x + Kp);
    d.b_bytes = (uint32_t)((int64_t)(rows_b - 1) * ld_w + Kp);
    const int drow = 32 * wid + (lane >> 2);
    const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
    d.voff_a0 = (uint32_t)(drow * ld_x + 16 * dchunk);
    d.voff_a1 = d.voff_a0 + (uint32_t)(16 * ld_x);
    d.voff_b0 = (uint32_t)(drow * ld_w + 16 * dchunk);
    d.voff_b1 = d.voff_b0 + (uint32_t)(16 * ld_w);
    d.lds_a = lds0 + (uint32_t)(32 * wid) * 64;
    d.lds_b = lds0 + kOffB + (uint32_t)(32 * wid) * 64;
    d.lds_junk = lds0 + kOffJunk;
    const int nb16 = (nb + 15) & ~15;
    const int srow = 64 * (wid & 3) + lane;
    if (wid < 4) {
      d.s_base = (uint64_t)(uintptr_t)(xs + (int64_t)m0 * ld_xs);
      d.s_bytes = (uint32_t)((int64_t)(rows_a - 1) * ld_xs + nb16);
      d.voff_s = (uint32_t)(srow * ld_xs);
      d.lds_s = lds0 + kOffScale + (uint32_t)(64 * wid) * 16;
    } else {
      d.s_base = (uint64_t)(uintptr_t)(ws + (int64_t)n0 * ld_ws);
      d.s_bytes = (uint32_t)((int64_t)(rows_b - 1) * ld_ws + nb16);
      d.voff_s = (uint32_t)(srow * ld_ws);
      d.lds_s = lds0 + kOffScale + 4096 + (uint32_t)(64 * (wid - 4)) * 16;
    }
  }

  // ---- fragment read addresses (stage 0); tile f / fj adds 2048 bytes.  Scale read
  //      addresses (slot 0): row * 16, tile f / fj adds 512 bytes.
  const uint32_t xsw = (uint32_t)((li >> 2) & 3);
  uint32_t ra[2], rb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t c = (uint32_t)(2 * h + lg);
    ra[h] = (uint32_t)(gp * 128 + li) * 64 + ((c ^ xsw) << 4);
    rb[h] = kOffB + (uint32_t)(wq * 64 + li) * 64 + ((c ^ xsw) << 4);
  }
  const uint32_t rsa = kOffScale + (uint32_t)(gp * 128 + li) * 16;
  const uint32_t rsb = kOffScale + 4096 + (uint32_t)(wq * 64 + li) * 16;

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  v8i fa[4], fb[2];
  uint32_t sa[4], sb[2];
  // exact-product mode: bf16 operands of one half step (bits of v8bf), [fragment][MFMA]
  v4i ea[4][2], eb[2][2];

  // memory phase of step s: fragments and scales of step s, then wait for this wave's DMA
  // of step s+1 (its LDS reads complete at the barrier that follows); only the DMA of step
  // s+2 stays in flight (issued in the previous compute phase, or by the prologue)
  auto memory_phase = [&](int s, auto par, auto last) {
    const uint32_t so = (uint32_t)(s & 3) * kStageBytes;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const v4i lo = lds16(ra[0] + so, 2048 * f), hi = lds16(ra[1] + so, 2048 * f);
      fa[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const v4i lo = lds16(rb[0] + so, 2048 * f), hi = lds16(rb[1] + so, 2048 * f);
      fb[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // scale dword of blocks 4u..4u+3 (u = s/2) of each fragment row, read at even steps
    // and kept for the odd one; lane g uses block 2s+g, byte 2(s&1) after the shift
    if (decltype(par)::value == 0) {
      const uint32_t ss = (uint32_t)((s >> 3) & 1) * kScaleSlot + 4u * (uint32_t)((s & 7) >> 1);
#pragma unroll
      for (int f = 0; f < 4; ++f)
        sa[f] = *reinterpret_cast<const uint32_t*>(smem + rsa + ss + 512 * f) >> (8 * lg);
#pragma unroll
      for (int f = 0; f < 2; ++f)
        sb[f] = *reinterpret_cast<const uint32_t*>(smem + rsb + ss + 512 * f) >> (8 * lg);
    }
    if (decltype(last)::value) {
      if ((K & 63) != 0) {
        // dword e of a fragment holds k = 64s + 32(e/4) + 16g + 4(e%4) .. +3
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int keep = K - (64 * s + 32 * (e >> 2) + 16 * lg + 4 * (e & 3));
          const uint32_t m = keep >= 4 ? 0xFFFFFFFFu : (keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u));
#pragma unroll
          for (int f = 0; f < 4; ++f) fa[f][e] = (int)((uint32_t)fa[f][e] & m);
#pragma unroll
          for (int f = 0; f < 2; ++f) fb[f][e] = (int)((uint32_t)fb[f][e] & m);
        }
      }
      if (2 * s + lg >= nb) {
        const uint32_t sh = 16u * (uint32_t)(s & 1);
        const uint32_t keep = ~(0xFFu << sh), one = 127u << sh;
#pragma unroll
        for (int f = 0; f < 4; ++f) sa[f] = (sa[f] & keep) | one;
#pragma unroll
        for (int f = 0; f < 2; ++f) sb[f] = (sb[f] & keep) | one;
      }
    }
    if (decltype(last)::value)
      wait_vm<0>();    // also the empty loads of steps T and T+1
    else
      wait_vm<kLoadsPerStep>();
  };

  // Compute phase of step s: 8 MFMAs, with this wave's DMA of step s+3 (whose stage was
  // last read in the phase before) issued between them, one load after every second MFMA,
  // so the address unit sees a steady stream instead of a burst; the last step issues none.
  // The empty volatile asm statements make the MFMAs take their operands only after the
  // barrier that opens the phase.  (Results are never routed through such statements:
  // the compiler would then miss the MFMA result latency when it reads them.)
  auto compute_phase = [&](int s, auto par, auto with_dma) {
    constexpr int OPS = 2 * decltype(par)::value;
    constexpr bool DMA = decltype(with_dma)::value;
    StepDma sd;
    if (DMA) {
      sd = step_dma(d, s + 3);
      issue_scales(d, s + 3);
    }
    asm volatile("" : "+v"(fa[0]), "+v"(fa[1]), "+v"(fa[2]), "+v"(fa[3]), "+v"(fb[0]), "+v"(fb[1]));
    asm volatile("" : "+v"(sa[0]), "+v"(sa[1]), "+v"(sa[2]), "+v"(sa[3]), "+v"(sb[0]), "+v"(sb[1]));
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int fj = 0; fj < 2; ++fj) {
        acc[fi][fj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[fj], fa[fi], acc[fi][fj], FB, FA, OPS,
                                                                      (int)sb[fj], OPS, (int)sa[fi]);
        if (DMA && fj == 1 && fi < 3) {
          // load fi of the step's DMA, between MFMA (fi, 1) and MFMA (fi + 1, 0)
          const uint32_t lds = fi == 0 ? d.lds_a + sd.so : fi == 1 ? d.lds_a + sd.so + 1024 : d.lds_b + sd.so;
          const uint32_t voff = fi == 0 ? d.voff_a0 : fi == 1 ? d.voff_a1 : d.voff_b0;
          dma16_between(lds, voff, fi < 2 ? sd.ra : sd.rb, fa[fi], fa[fi + 1]);
        }
        if (DMA && fj == 1 && fi == 3) dma16_after(d.lds_b + sd.so + 1024, d.voff_b1, sd.rb, fa[3]);
      }
  };

  // Exact-product mode.  A step is split into two halves: half h holds the 16-byte half h
  // of every fragment row, i.e. block 2s + h of the step (lane g's half h covers k = 32h +
  // 16g .. +15 of the 64-byte step).  Its memory phase reads those halves, decodes them
  // with the block's scale to bf16 (exact while code * 2^(s-127) lies in bf16's range) and
  // its compute phase runs 16 v_mfma_f32_32x32x16_bf16: MFMA m of a fragment takes bytes
  // 8m..8m+7 of every lane, the same k for W and X, so each MFMA contracts 16 matching k
  // of one block with exact products and FP32 sums.  The DMA and the waits are those of
  // the matrix-core mode (issued in half 0, waited in half 0).
  auto memory_half = [&](int s, auto h_c, auto par, auto last) __attribute__((always_inline)) {
    constexpr int h = decltype(h_c)::value;
    const uint32_t so = (uint32_t)(s & 3) * kStageBytes;
    v4i ca[4], cb[2];
#pragma unroll
    for (int f = 0; f < 4; ++f) ca[f] = lds16(ra[h] + so, 2048 * f);
#pragma unroll
    for (int f = 0; f < 2; ++f) cb[f] = lds16(rb[h] + so, 2048 * f);
    // scale dwords of blocks 4u..4u+3 (u = s/2) of each fragment row, read at the first half
    // of even steps and kept for the odd one; block 2s + h is byte 2(s&1) + h
    if (h == 0 && decltype(par)::value == 0) {
      const uint32_t ss = (uint32_t)((s >> 3) & 1) * kScaleSlot + 4u * (uint32_t)((s & 7) >> 1);
#pragma unroll
      for (int f = 0; f < 4; ++f) sa[f] = *reinterpret_cast<const uint32_t*>(smem + rsa + ss + 512 * f);
#pragma unroll
      for (int f = 0; f < 2; ++f) sb[f] = *reinterpret_cast<const uint32_t*>(smem + rsb + ss + 512 * f);
    }
    bool dead_block = false;
    if (decltype(last)::value || (TAIL && s == T - 1)) {
      if ((K & 63) != 0) {
        // dword e of this half holds k = 64s + 32h + 16g + 4e .. +3
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int keep = K - (64 * s + 32 * h + 16 * lg + 4 * e);
          const uint32_t m = keep >= 4 ? 0xFFFFFFFFu : (keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u));
#pragma unroll
          for (int f = 0; f < 4; ++f) ca[f][e] = (int)((uint32_t)ca[f][e] & m);
#pragma unroll
          for (int f = 0; f < 2; ++f) cb[f][e] = (int)((uint32_t)cb[f][e] & m);
        }
      }
      dead_block = 2 * s + h >= nb;   // its bytes are zero; its scale byte is not read
    }
    const uint32_t sh = 8u * (uint32_t)(2 * (s & 1) + h);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const float sc = e8m0_to_f32(dead_block ? 127u : (sa[f] >> sh) & 0xFFu);
#pragma unroll
      for (int m = 0; m < 2; ++m)
        ea[f][m] = __builtin_bit_cast(v4i, codes_to_bf16<FA>((uint32_t)ca[f][2 * m], (uint32_t)ca[f][2 * m + 1], sc));
    }
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const float sc = e8m0_to_f32(dead_block ? 127u : (sb[f] >> sh) & 0xFFu);
#pragma unroll
      for (int m = 0; m < 2; ++m)
        eb[f][m] = __builtin_bit_cast(v4i, codes_to_bf16<FB>((uint32_t)cb[f][2 * m], (uint32_t)cb[f][2 * m + 1], sc));
    }
    if (h == 0) {
      if (decltype(last)::value)
        wait_vm<0>();
      else
        wait_vm<kLoadsPerStep>();
    }
  };

  // Compute phase of one half step: 16 bf16 MFMAs (both MFMAs of every tile, the first of
  // each tile before any second one), with the DMA of step s+3 issued between the first
  // eight in half 0 as in the matrix-core mode.
  auto compute_half = [&](int s, auto with_dma) __attribute__((always_inline)) {
    constexpr bool DMA = decltype(with_dma)::value;
    StepDma sd;
    if (DMA) {
      sd = step_dma(d, s + 3);
      issue_scales(d, s + 3);
    }
    asm volatile("" : "+v"(ea[0][0]), "+v"(ea[1][0]), "+v"(ea[2][0]), "+v"(ea[3][0]), "+v"(eb[0][0]), "+v"(eb[1][0]));
    asm volatile("" : "+v"(ea[0][1]), "+v"(ea[1][1]), "+v"(ea[2][1]), "+v"(ea[3][1]), "+v"(eb[0][1]), "+v"(eb[1][1]));
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int fj = 0; fj < 2; ++fj) {
          acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, eb[fj][m]),
                                                                __builtin_bit_cast(v8bf, ea[fi][m]), acc[fi][fj], 0, 0, 0);
          if (DMA && m == 0 && fj == 1 && fi < 3) {
            const uint32_t lds = fi == 0 ? d.lds_a + sd.so : fi == 1 ? d.lds_a + sd.so + 1024 : d.lds_b + sd.so;
            const uint32_t voff = fi == 0 ? d.voff_a0 : fi == 1 ? d.voff_a1 : d.voff_b0;
            dma16_between(lds, voff, fi < 2 ? sd.ra : sd.rb, ea[fi][0], ea[fi + 1][0]);
          }
          if (DMA && m == 0 && fj == 1 && fi == 3)
            dma16_after(d.lds_b + sd.so + 1024, d.voff_b1, sd.rb, ea[3][0]);
        }
  };

  // ---- prologue: steps 0..2 in flight, step 0 landed everywhere
#pragma unroll
  for (int s = 0; s < 3; ++s)
    issue_step(d, s);
  if (T > 0)
    wait_vm<2 * kLoadsPerStep>();
  else
    wait_vm<0>();   // K = 0: no step waits for the empty loads before the epilogue uses LDS
  lds_barrier();
  if (gp == 1) lds_barrier();   // group 1 runs one phase behind group 0

  // one K step: memory phase, barrier, compute phase, barrier
  auto step = [&](int s, auto par, auto last) {
    __builtin_amdgcn_sched_barrier(0);
    memory_phase(s, par, last);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    compute_phase(s, par, std::integral_constant<bool, !decltype(last)::value>());
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using No = std::false_type;
  using Yes = std::true_type;
  // exact-product mode: two half steps, each a memory phase and a compute phase
  auto step_exact = [&](int s, auto par, auto last) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    memory_half(s, C0(), par, last);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    compute_half(s, std::integral_constant<bool, !decltype(last)::value>());
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    memory_half(s, C1(), par, last);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    compute_half(s, No());
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
  };
  auto any_step = [&](int s, auto par, auto last) __attribute__((always_inline)) {
    if constexpr (EXACT)
      step_exact(s, par, last);
    else
      step(s, par, last);
  };
  // steps 0..T-2 in pairs (even step: opsel byte 0, odd: byte 2); the last step, which
  // may be partial, on its own
  int s = 0;
  if constexpr (TAIL && !EXACT) {
    // matrix-core mode, K not a multiple of 64: the last step is peeled (masked code bytes
    // at k >= K, blocks >= nb replaced), which keeps the masking out of the loop's registers
    for (; s + 2 <= T - 1; s += 2) {
      any_step(s, C0(), No());
      any_step(s + 1, C1(), No());
    }
    if (s < T - 1) {
      any_step(s, C0(), No());
      ++s;
    }
    if (T > 0) {
      if (s & 1)
        any_step(s, C1(), Yes());
      else
        any_step(s, C0(), Yes());
    }
  } else {
    // every step runs through the same loop: the last one's DMA of steps >= T reads empty
    // ranges, and in the exact mode with K not a multiple of 64 its memory phase masks code
    // bytes at k >= K and blocks >= nb behind a uniform branch.  The epilogue reuses the
    // code stages, so every wave's loads must have landed before any wave writes there.
    for (; s + 2 <= T; s += 2) {
      any_step(s, C0(), No());
      any_step(s + 1, C1(), No());
    }
    if (s < T) any_step(s, C0(), No());
    wait_vm<0>();
    lds_barrier();
  }
  if (gp == 0) lds_barrier();   // matches group 1's extra barrier: all LDS reads are done

  // ---- epilogue: v = act(alpha * acc + bias[col]) in place; y = v rounded once to its
  //      type; the MX codes of bf16(v) along rows.  Lane (g, i) holds Y[row 32 fi + i][col
  //      32 fj + 8 q + 4 g + e] in acc[fi][fj][4 q + e] (rows and columns relative to the
  //      wave's 128x64 block).
  const int wrow0 = m0 + gp * 128, wcol0 = n0 + wq * 64;
  {
    const bool has_bias = ep.bias != nullptr;
#pragma unroll
    for (int fj = 0; fj < 2; ++fj)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = wcol0 + 32 * fj + 8 * q + 4 * lg + e;
          const float bv = (has_bias && col < N) ? ep.bias[col] : 0.0f;
#pragma unroll
          for (int fi = 0; fi < 4; ++fi) {
            const float a = acc[fi][fj][4 * q + e];
            acc[fi][fj][4 * q + e] = has_bias ? __builtin_fmaf(ep.alpha, a, bv) : ep.alpha * a;
          }
        }
    if (ep.act) {
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int fj = 0; fj < 2; ++fj)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[fi][fj][r] = silu(acc[fi][fj][r]);
    }
  }
  // interior tile, aligned y: stage the block in this wave's LDS region as row-major rows
  // of 64 values with the 16-byte chunk index XOR (row & 7), then store whole 16-byte row
  // pieces (E = bytes per value)
  auto store_staged = [&](auto e_c) {
    constexpr int E = decltype(e_c)::value;
    constexpr int RB = 64 * E;                       // bytes per staged row
    constexpr int CPR = RB / 16;                     // 16-byte chunks per row
    constexpr int RP = kEpiWaveBytes / RB;           // rows per pass: 128 (bf16) or 64 (fp32)
    constexpr int FPP = RP / 32;                     // fragment rows per pass
    const uint32_t wbase = (uint32_t)wid * kEpiWaveBytes;
#pragma unroll
    for (int pass = 0; pass < 128 / RP; ++pass) {
#pragma unroll
      for (int fj = 0; fj < 2; ++fj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c0 = 32 * fj + 8 * q + 4 * lg;   // first of this lane's 4 columns
#pragma unroll
          for (int fl = 0; fl < FPP; ++fl) {
            const int fi = pass * FPP + fl;
            const int row = 32 * fl + li;
            const uint32_t byte = (uint32_t)(c0 * E);
            const uint32_t chunk = (byte >> 4) ^ (uint32_t)(row & (CPR - 1) & 7);
            const uint32_t addr = wbase + (uint32_t)row * RB + (chunk << 4) + (byte & 15);
            if (E == 2) {
              typedef uint32_t v2u __attribute__((ext_vector_type(2)));
              v2u p;
              p[0] = pack_bf16(acc[fi][fj][4 * q + 0], acc[fi][fj][4 * q + 1]);
              p[1] = pack_bf16(acc[fi][fj][4 * q + 2], acc[fi][fj][4 * q + 3]);
              *reinterpret_cast<v2u*>(smem + addr) = p;
            } else {
              typedef float v4f __attribute__((ext_vector_type(4)));
              v4f p;
#pragma unroll
              for (int e = 0; e < 4; ++e) p[e] = acc[fi][fj][4 * q + e];
              *reinterpret_cast<v4f*>(smem + addr) = p;
            }
          }
        }
      // read back 16 bytes per lane: 64 lanes cover 1024 bytes = 1024 / RB rows
      constexpr int RPI = 1024 / RB;
#pragma unroll
      for (int it = 0; it < RP / RPI; ++it) {
        const int row = it * RPI + lane / CPR;
        const int c = lane % CPR;
        const uint32_t addr = wbase + (uint32_t)row * RB + (uint32_t)((c ^ (row & (CPR - 1) & 7)) << 4);
        const v4i v = *reinterpret_cast<const v4i*>(smem + addr);
        uint8_t* dst = reinterpret_cast<uint8_t*>(ep.y) +
                       ((int64_t)(wrow0 + pass * RP + row) * ep.ld_y + wcol0) * E + 16 * c;
        *reinterpret_cast<v4i*>(dst) = v;
      }
    }
  };
  if (!ep.y) {
  } else if (ep.y_vec16 && m0 + BM <= M && n0 + BN <= N) {
    if (ep.y_bf16)
      store_staged(std::integral_constant<int, 2>());
    else
      store_staged(std::integral_constant<int, 4>());
  } else {
#pragma unroll
    for (int fj = 0; fj < 2; ++fj)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = wcol0 + 32 * fj + 8 * q + 4 * lg + e;
#pragma unroll
          for (int fi = 0; fi < 4; ++fi) {
            const int row = wrow0 + 32 * fi + li;
            if (row < M && col < N) {
              const float v = acc[fi][fj][4 * q + e];
              if (ep.y_bf16)
                reinterpret_cast<uint16_t*>(ep.y)[(int64_t)row * ep.ld_y + col] = (uint16_t)f32_to_bf16_rne(v);
              else
                reinterpret_cast<float*>(ep.y)[(int64_t)row * ep.ld_y + col] = v;
            }
          }
        }
  }
  if (ep.qc) {
    // bf16(v) of the wave's 128x64 block as 128 rows of 128 bytes in its own LDS region
    // (the same region and chunk swizzle as the bf16 staging above), columns >= N as +0
    const uint32_t wbase = (uint32_t)wid * kEpiWaveBytes;
#pragma unroll
    for (int fj = 0; fj < 2; ++fj)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c0 = 32 * fj + 8 * q + 4 * lg;
        bool in[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) in[e] = wcol0 + c0 + e < N;
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) {
          const int row = 32 * fi + li;
          const uint32_t chunk = (uint32_t)(((2 * c0) >> 4) ^ (row & 7));
          const uint32_t addr = wbase + (uint32_t)row * 128u + (chunk << 4) + (uint32_t)((2 * c0) & 15);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = in[e] ? acc[fi][fj][4 * q + e] : 0.0f;
          typedef uint32_t v2u __attribute__((ext_vector_type(2)));
          v2u p;
          p[0] = pack_bf16(v[0], v[1]);
          p[1] = pack_bf16(v[2], v[3]);
          *reinterpret_cast<v2u*>(smem + addr) = p;
        }
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    quantize_staged<2>(wbase, lane, wrow0, M, wcol0 / 32, (N + 31) / 32, ep);
  }
}

template <int FA, int FB, bool EXACT, bool TAIL>
hipError_t launch_t(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                    int64_t ld_xs, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws,
                    const GemmEpilogue& ep, hipStream_t stream) {
  static bool attr_set[64] = {false};
  auto kern = k_gemm_pp<FA, FB, EXACT, TAIL>;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!attr_set[dev]) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(kThreads), kLdsBytes, stream, (int)M, (int)N, (int)K, tiles_m,
                     tiles_n, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep);
  return hipGetLastError();
}

// K not a multiple of 64: the kernel with the masked last step
template <int FA, int FB, bool EXACT>
hipError_t launch_f(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                    int64_t ld_xs, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws,
                    const GemmEpilogue& ep, hipStream_t stream) {
  if (K % 64 != 0) return launch_t<FA, FB, EXACT, true>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
  return launch_t<FA, FB, EXACT, false>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
}

template <bool EXACT>
hipError_t launch_e(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs, int64_t ld_xs,
                    int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws, int w_fmt,
                    const GemmEpilogue& ep, hipStream_t stream) {
  if (x_fmt == kE4M3 && w_fmt == kE4M3)
    return launch_f<0, 0, EXACT>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
  if (x_fmt == kE4M3) return launch_f<0, 1, EXACT>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
  if (w_fmt == kE4M3) return launch_f<1, 0, EXACT>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
  return launch_f<1, 1, EXACT>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
}

hipError_t launch(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs, int64_t ld_xs,
                  int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws, int w_fmt,
                  const GemmEpilogue& ep, bool exact, hipStream_t stream) {
  if (exact) return launch_e<true>(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, stream);
  return launch_e<false>(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, stream);
}

}  // namespace pp

template <int MODE, int FA, int FB>
hipError_t gemm_f(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs, int64_t ld_xs,
                  const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws, const GemmEpilogue& ep,
                  hipStream_t stream) {
  static bool attr_set[64] = {false};
  auto kern = k_gemm<MODE, FA, FB>;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!attr_set[dev]) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  const int ntiles = tiles_m * tiles_n;
  hipLaunchKernelGGL(kern, dim3(ntiles), dim3(kThreads), kLdsBytes, stream, (int)M, (int)N, (int)K, tiles_m, tiles_n,
                     xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep);
  return hipGetLastError();
}

template <int MODE>
hipError_t gemm_m(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs, int64_t ld_xs,
                  int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws, int w_fmt,
                  const GemmEpilogue& ep, hipStream_t stream) {
  if (x_fmt == kE4M3 && w_fmt == kE4M3) return gemm_f<MODE, 0, 0>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
  if (x_fmt == kE4M3) return gemm_f<MODE, 0, 1>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
  if (w_fmt == kE4M3) return gemm_f<MODE, 1, 0>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
  return gemm_f<MODE, 1, 1>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
}

}  // namespace

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                       int64_t ld_xs, int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws,
                       int w_fmt, const GemmEpilogue& ep_in, int exact, hipStream_t stream) {
  GemmEpilogue ep = ep_in;
  const int64_t ey = ep.y_bf16 ? 2 : 4;
  ep.y_vec16 = ep.y && ((uintptr_t)ep.y % 16 == 0) && ((ep.ld_y * ey) % 16 == 0);
  const bool scales16 = ((uintptr_t)xs % 16 == 0) && ((uintptr_t)ws % 16 == 0) && ld_xs % 16 == 0 && ld_ws % 16 == 0;
  if (scales16)
    return pp::launch(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, exact != 0, stream);
  if (exact) return gemm_m<1>(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, stream);
  return gemm_m<0>(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, stream);
}

}  // namespace mxq

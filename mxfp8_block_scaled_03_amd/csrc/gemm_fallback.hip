// gemm_fallback.hip -- block-scaled FP8 GEMM for operands whose scale rows break the
// alignment the fast kernels need (both accumulation modes).
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
// Fallback kernel (scale rows that are not 16-byte aligned, both accumulation modes).
// Tiling: 256x256 output tile per workgroup of 4 waves (2x2 waves of 128x128), K step of
// 128 bytes.  Code tiles move global -> LDS with buffer_load ... lds (16 bytes per lane,
// no VGPR staging), double-buffered, with a 16-byte-chunk XOR swizzle so the fragment
// reads (ds_read_b128) are bank-conflict free.  Out-of-range rows and K positions past the
// row read as zero through the buffer descriptor's bound; code bytes at k >= K inside the
// last step are masked in registers and scale bytes of blocks >= nb are replaced by 127
// (a finite 1.0, so zero codes contribute exactly zero).  Workgroups are mapped to tiles
// XCD-first (consecutive tiles on the same XCD share its L2), then in groups of 4 tile rows.
#include "gemm_common.hpp"

namespace mxq {
namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kTileBytes = BM * BK;      // 32 KiB: one operand tile of one stage
constexpr int kOffB = 2 * kTileBytes;    // LDS: A stage 0 | A stage 1 | B stage 0 | B stage 1
constexpr int kLdsBytes = 4 * kTileBytes;

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
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
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

hipError_t launch_gemm_fallback(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                                int64_t ld_xs, int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws,
                                int64_t ld_ws, int w_fmt, const GemmEpilogue& ep, int exact, hipStream_t stream) {
  if (exact) return gemm_m<1>(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, stream);
  return gemm_m<0>(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, stream);
}

}  // namespace mxq

// gemm_exact.hip -- block-scaled FP8 GEMM with exact products and FP32 sums (accumulation
// mode MXQ_ACC_FP32) on gfx950.
//
// "Low-Precision GPU Programming", "Scale ownership and the GEMM dataflow": Y = X W; with
// 32-element blocks along K the product of the X-block and W-block scales stays inside the
// outer sum over blocks, a partial final block is zero-padded, and the consumer may apply
// the scales inside the contraction.  "Accumulator type isn't the whole arithmetic
// contract": a declared FP32 accumulator can hide reduced internal precision; here every
// product 2^(sx-127) x~ * 2^(sw-127) w~ is formed exactly and only the sums round (FP32).
// "Hardware support and kernel ABI contracts": X row-major (1x32 groups along K), W
// column-major (32x1 groups), E8M0 scales, epilogue scale (alpha), bias, activation, cast.
//
// How the products stay exact: a code times its block scale is decoded to bf16 in
// registers (v_cvt_scalef32_pk_bf16_{fp8,bf8}: exact whenever code * 2^(s-127) is a bf16
// value, which holds for scale bytes 3..246 (E4M3) and 10..239 (E5M2) and every code), and
// v_mfma_f32_32x32x16_bf16 multiplies bf16 pairs exactly and sums in FP32.
//
// Work split.  256x256 output tile per workgroup of 4 waves, one wave per SIMD; wave
// (wm, wn) owns the 128x128 block of X rows 128 wm.. and W rows 128 wn.. (4x4 MFMA tiles,
// 256 FP32 accumulators per lane).  A wave decodes each of its 256 fragment rows once per
// K element: two conversion instructions per MFMA, which the matrix core's 32-cycle issue
// interval hides.  A narrow variant (256x192 tile, 128x96 per wave, 4x3 MFMA tiles, 7/3
// conversions per MFMA) runs the same loop without the fourth W fragment column; the host
// picks it where its rounds fill the CUs better.  Full-width tiles may also run as several
// K ranges whose sums a fix-up adds (ExSplit below).
//
// K loop.  A stage is 64 bytes of K (two 32-element blocks) of 256 X rows and 256 W rows,
// 32 KiB in LDS, 16-byte chunk c of row r at chunk c ^ ((r >> 2) & 3) (conflict-free
// ds_read_b128 fragment reads).  Four stages rotate; stage s + 4 is fetched global -> LDS
// (buffer_load ... lds from inline assembly, completion tracked by explicit vmcnt waits)
// while stages s and s + 1 are read, so three stages of look-ahead hide the fetch latency.
// Scale bytes travel the same way, 4 bytes (4 blocks) per row into a four-slot ring.
// Each stage is four k16 steps; in step t the wave issues its 16 MFMAs on the bf16 operands
// of step t while, between them, it converts the codes of step t + 1 (two conversions per
// MFMA on average), reads the codes of the next block from LDS and issues its share of the
// DMA.  The program order puts two conversions after each MFMA; inside a step the compiler
// may regroup them (scheduling fences only at the step boundaries: it clusters up to seven
// conversions behind some MFMAs and none behind others, which measured ~2 % faster than
// the strict interleave; the narrow tile runs without the fences, 2.6 % faster there and
// no different for the full-width one).  One workgroup barrier per stage hands the stage
// ring over.
//
// Edges.  Rows past the matrix and K bytes past a row read as zero through the buffer
// descriptor's bound; in the last stage the code bytes at k >= K are zeroed in LDS once, and
// a block past nb gets scale byte 127 there (1.0: its zero codes then contribute exactly
// zero whatever byte the caller's array holds past the end).  Scale rows
// are read in 4-byte words; the last row of X or W, whose final word may end past the
// caller's array, has its last partial word read byte by byte instead.  The narrow tile
// keeps the stage layout of 256 W rows: its descriptor ends at its 192 rows, so the DMA of
// rows 192..255 lands zeros that no fragment reads.
#include <cstdlib>
#include <cstring>

#include "gemm_common.hpp"

namespace mxq {
namespace {
namespace ex {

constexpr int BM = 256, BN = 256;
constexpr int kThreads = 256;                        // 4 waves, one per SIMD
constexpr int kStages = 4;
constexpr int kOpBytes = 256 * 64;                   // one operand of one stage
constexpr int kStageBytes = 2 * kOpBytes;            // X rows then W rows: 32 KiB
constexpr int kOffScale = kStages * kStageBytes;     // 128 KiB
constexpr int kScaleSlotBytes = 512 * 4;             // X rows 0..255, W rows 256..511; 4 blocks each
constexpr int kScaleSlots = 4;
constexpr int kLdsBytes = kOffScale + kScaleSlots * kScaleSlotBytes;   // 136 KiB
constexpr int kEpiWaveBytes = 32768;                 // per-wave epilogue staging (in the code stages)
constexpr int kPartFloats = 4 * 64 * 256;            // one tile's FP32 accumulators (256 KiB)

// K split.  Items 0 .. full-1 are whole tiles (tile numbers 0 .. full-1); items full ..
// full+items-1 are the ks K ranges of tiles full ..: range r runs stages [r s_per,
// (r+1) s_per), the last range up to S.  Each range writes its FP32 sums, row-major
// 256 x 256, to part[(ks (t - full) + r) * kPartFloats ..] through the epilogue's own
// store path; a second launch adds the ranges of each split tile in range order and runs
// the epilogue on the total (k_gemm_ex_fix_ew, or this kernel with fix = 1 when MX codes
// are written).  No split: full = tiles, items = 0.
struct ExSplit {
  int full, items, ks, s_per;
  int fix;          // 1: the fix-up launch (one 64-thread workgroup per wave of a split tile)
  float* part;
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 4 bytes per lane from buffer offset voff into LDS at lds + 4 * lane.
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, v4i rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int FA, int FB, int BNT>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_ex(int M, int N, int K, int tiles_m, int tiles_n,
                                                        const uint8_t* __restrict__ xc, int64_t ld_x,
                                                        const uint8_t* __restrict__ xs, int64_t ld_xs,
                                                        const uint8_t* __restrict__ wc, int64_t ld_w,
                                                        const uint8_t* __restrict__ ws, int64_t ld_ws,
                                                        const GemmEpilogue ep, const ExSplit sp) {
  static_assert(BNT == 256 || BNT == 192, "tile width");
  constexpr int WN = BNT / 2;               // output columns (W rows) per wave
  constexpr int NFW = WN / 32;              // W fragments per wave
  // work item -> tile and K-stage range [s0, s0 + S); the fix-up launch takes tile
  // full + blockIdx.x and no stages
  const int S_all = (K + 63) / 64;          // stages of the whole K
  int t, rng = -1;                          // rng: the item's K range, -1 for a whole tile
  if (sp.fix) {
    t = sp.full + (int)(blockIdx.x >> 2);
  } else if ((int)blockIdx.x < sp.full) {
    t = xcd_order(blockIdx.x, sp.full);
  } else {
    const int k = xcd_order(blockIdx.x - sp.full, sp.items);
    t = sp.full + k / sp.ks;
    rng = k - (t - sp.full) * sp.ks;
  }
  int tm, tn;
  tile_at(t, tiles_m, tiles_n, tm, tn);
  const int s0 = rng > 0 ? rng * sp.s_per : 0;
  const bool last_range = rng < 0 || rng == sp.ks - 1;   // holds the last stage
  const int S = sp.fix ? 0 : (last_range ? S_all - s0 : sp.s_per);   // stages of this item
  const int P0 = s0 >> 1;                   // its first scale word (s_per is even)
  const int m0 = tm * BM, n0 = tn * BNT;
  const int lane = threadIdx.x & 63;
  // the fix-up launch runs one wave per workgroup (4 per tile): its wave index comes from
  // the workgroup index, and its epilogue staging uses LDS slot 0
  const int wid = sp.fix ? (int)(blockIdx.x & 3) : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wslot = sp.fix ? 0 : wid;
  const int wm = wid >> 1, wn = wid & 1;
  const int li = lane & 31, lg = lane >> 5;
  const int nb = (K + 31) / 32;             // blocks per line
  const int Kp = 32 * nb;
  const int nbf = nb / 4;                   // whole 4-block scale words per row
  const int rows_x = min(BM, M - m0), rows_w = min(BNT, N - n0);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)smem;

  // ---- code DMA: wave w loads rows 64w..64w+63 of both operands, 16 rows per load: lane
  //      l covers row 64w + 16n + l/4, physical chunk l & 3 holding logical chunk
  //      (l & 3) ^ ((row >> 2) & 3)
  const uint64_t x_base = (uint64_t)(uintptr_t)(xc + (int64_t)m0 * ld_x);
  const uint64_t w_base = (uint64_t)(uintptr_t)(wc + (int64_t)n0 * ld_w);
  const uint32_t x_bytes = (uint32_t)((int64_t)(rows_x - 1) * ld_x + Kp);
  const uint32_t w_bytes = (uint32_t)((int64_t)(rows_w - 1) * ld_w + Kp);
  uint32_t voff_x[4], voff_w[4];
  {
    const int drow = 64 * wid + (lane >> 2);
    const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      voff_x[n] = (uint32_t)((drow + 16 * n) * ld_x + 16 * dchunk + 64 * s0);
      voff_w[n] = (uint32_t)((drow + 16 * n) * ld_w + 16 * dchunk + 64 * s0);
    }
  }
  const uint32_t lds_cx = lds0 + (uint32_t)(64 * wid) * 64;   // + stage slot + 1024 n
  const uint32_t lds_cw = lds_cx + kOpBytes;

  // ---- scale DMA: the load of iteration j brings word P = (j + 6) / 2 (blocks 4P..4P+3)
  //      of scale rows 128w + 64h + lane (h = j & 1) of the 512 rows (X then W).  The last
  //      tile row of the matrix stops its descriptor before its partial last word; other
  //      tiles read their last row's word up to 4 * ceil(nb / 4) <= ld bytes.
  const bool s_is_x = wid < 2;
  const int s_rows = s_is_x ? rows_x : rows_w;
  const int64_t ld_s = s_is_x ? ld_xs : ld_ws;
  const bool s_last_tile = s_is_x ? (m0 + BM >= M) : (n0 + BNT >= N);
  const uint64_t s_base = (uint64_t)(uintptr_t)(s_is_x ? xs + (int64_t)m0 * ld_xs : ws + (int64_t)n0 * ld_ws);
  const uint32_t s_rowspan = (uint32_t)((int64_t)(s_rows - 1) * ld_s);
  const int s_words = s_last_tile ? nbf : (nb + 3) / 4;        // words of the descriptor's last row
  uint32_t voff_s[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) voff_s[h] = (uint32_t)((128 * (wid & 1) + 64 * h + lane) * ld_s + 4 * P0);
  const uint32_t lds_s = lds0 + kOffScale + (uint32_t)(128 * wid) * 4;   // + slot + 256 h

  // One descriptor per operand for the whole K loop, the K offset in the lane offset: a
  // byte is fetched only while its offset lies inside the tile's rows (rows * ld, the last
  // row up to Kp or its last scale word), so rows past the edge, K bytes past the last
  // row's end and stages or words past the end read as zero, and every byte read lies in
  // the caller's arrays.  (A stage past the end may read the following row's bytes in the
  // other rows; such stages are never multiplied.)
  const v4i rsrc_x = rsrc_of(x_base, x_bytes), rsrc_w = rsrc_of(w_base, w_bytes);
  const v4i rsrc_s = rsrc_of(s_base, s_rowspan + 4u * (uint32_t)s_words);
  auto issue_codes = [&](int c, int n) __attribute__((always_inline)) {
    // load n (0..3 X, 4..7 W) of stage c
    const uint32_t kb = 64u * (uint32_t)c;
    const uint32_t so = (uint32_t)(c & 3) * kStageBytes;
    if (n < 4)
      dma16(lds_cx + so + 1024u * (uint32_t)n, voff_x[n] + kb, rsrc_x);
    else
      dma16(lds_cw + so + 1024u * (uint32_t)(n - 4), voff_w[n - 4] + kb, rsrc_w);
  };
  auto issue_scale = [&](int j) __attribute__((always_inline)) {
    const int P = (j + 6) >> 1, h = j & 1;
    dma4(lds_s + (uint32_t)(P & 3) * kScaleSlotBytes + 256u * (uint32_t)h, voff_s[h] + 4u * (uint32_t)P, rsrc_s);
  };

  // ---- fragment reads: lane (li, lg) of frag f reads tile row 128 wm + 32 f + li (X) or
  //      128 wn + 32 f + li (W), 16 bytes of block e of the stage (chunk 2e + lg); frag f
  //      adds 2048 bytes.  Scale words: row r of the slot at 4 r, frag f adds 128 bytes.
  uint32_t fx[2], fw[2];
  {
    const uint32_t sw = (uint32_t)((li >> 2) & 3);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t c = (uint32_t)(2 * e + lg);
      fx[e] = (uint32_t)(128 * wm + li) * 64u + ((c ^ sw) << 4);
      fw[e] = (uint32_t)kOpBytes + (uint32_t)(WN * wn + li) * 64u + ((c ^ sw) << 4);
    }
  }
  const uint32_t sx_rd = (uint32_t)kOffScale + (uint32_t)(128 * wm + li) * 4u;
  const uint32_t sw_rd = (uint32_t)kOffScale + (uint32_t)(256 + WN * wn + li) * 4u;

  // ---- the last row's partial scale word (nb % 4 != 0), read byte by byte: of a lane's 4
  //      X (W) fragment rows, 32 apart, at most one is the last row of X (W)
  uint32_t tail_x = 0, tail_w = 0;
  int tail_fx = -1, tail_fw = -1;
  if ((nb & 3) != 0) {
    const int rx = M - 1 - (m0 + 128 * wm + li), rw = N - 1 - (n0 + WN * wn + li);
    if (rx >= 0 && rx < 128 && (rx & 31) == 0) tail_fx = rx >> 5;
    if (rw >= 0 && rw < WN && (rw & 31) == 0) tail_fw = rw >> 5;
    if (tail_fx >= 0) {
      const uint8_t* p = xs + (int64_t)(M - 1) * ld_xs + 4 * nbf;
      for (int t = 0; t < (nb & 3); ++t) tail_x |= (uint32_t)p[t] << (8 * t);
    }
    if (tail_fw >= 0) {
      const uint8_t* p = ws + (int64_t)(N - 1) * ld_ws + 4 * nbf;
      for (int t = 0; t < (nb & 3); ++t) tail_w |= (uint32_t)p[t] << (8 * t);
    }
  }
  asm volatile("" : "+v"(tail_x), "+v"(tail_w));   // loaded before any DMA is issued

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  v4i code[2][8];     // codes of one block [block parity][frag: X 0..3, W 4..7]
  v4i opd[2][8];      // bf16 operands of one k16 step [step parity][frag]
  uint32_t sdw[8];    // scale words (4 blocks) of the current word index
  float sf[2][8];     // scale values of one block [block parity][frag]

  auto read_codes = [&](int b, int f) __attribute__((always_inline)) {
    if (f >= 4 + NFW) return;
    const uint32_t so = (uint32_t)((b >> 1) & 3) * kStageBytes;
    const int e = b & 1;
    code[e][f] = f < 4 ? lds16(fx[e] + so, 2048 * f) : lds16(fw[e] + so, 2048 * (f - 4));
  };
  auto read_scale = [&](int P, int f) __attribute__((always_inline)) {
    if (f >= 4 + NFW) return;
    const uint32_t sl = (uint32_t)(P & 3) * kScaleSlotBytes;
    const uint32_t a = (f < 4 ? sx_rd + 128u * (uint32_t)f : sw_rd + 128u * (uint32_t)(f - 4)) + sl;
    sdw[f] = *reinterpret_cast<const uint32_t*>(smem + a);
  };
  // the last row's partial word replaces what the DMA left there (zeros); branch free, so
  // no conversion is moved across it
  auto fix_scale = [&](int P) __attribute__((always_inline)) {
    const bool last_word = P + P0 == nbf;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      sdw[f] = (last_word && tail_fx == f) ? tail_x : sdw[f];
      if (f < NFW) sdw[4 + f] = (last_word && tail_fw == f) ? tail_w : sdw[4 + f];
    }
  };
  auto make_sf = [&](int b, int f) __attribute__((always_inline)) {
    if (f >= 4 + NFW) return;
    sf[b & 1][f] = e8m0_to_f32((sdw[f] >> (8 * (b & 3))) & 0xFFu);
  };
  // conversion piece q (0..15) of a k16 step (block b, half h): frag q / 2, code dword
  // 2h + (q & 1) -> operand dwords 2(q & 1), 2(q & 1) + 1 of opd[o]
  auto convert = [&](int o, int b, int h, int q) __attribute__((always_inline)) {
    const int f = q >> 1, w = q & 1;
    if (f >= 4 + NFW) return;
    const uint32_t src = (uint32_t)code[b & 1][f][2 * h + w];
    const float s = sf[b & 1][f];
    int lo, hi;
    if (f < 4) {
      lo = (int)cvt_pk_bf16<FA>(src, s, false);
      hi = (int)cvt_pk_bf16<FA>(src, s, true);
    } else {
      lo = (int)cvt_pk_bf16<FB>(src, s, false);
      hi = (int)cvt_pk_bf16<FB>(src, s, true);
    }
    // keep the conversions in their slot (no pass may sink them towards their MFMAs)
    asm volatile("" : "+v"(lo), "+v"(hi));
    opd[o][f][2 * w] = lo;
    opd[o][f][2 * w + 1] = hi;
  };
  auto mfma = [&](int o, int m) __attribute__((always_inline)) {
    const int fi = m >> 2, fj = m & 3;
    if (fj >= NFW) return;
    acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, opd[o][4 + fj]),
                                                          __builtin_bit_cast(v8bf, opd[o][fi]), acc[fi][fj], 0, 0, 0);
  };
  // zero the code bytes at k >= K of the last stage and, when nb is odd, set the scale
  // byte of its second block (block nb, past the end) to 127 = 1.0, in place in LDS (thread
  // t owns row t of X and of W).  The stage's scale word is first read after this.
  auto mask_last_stage = [&]() __attribute__((always_inline)) {
    const int r = threadIdx.x;
    if (nb & 1) {
      const int P = (nb >> 2) - P0;
      const uint32_t a = (uint32_t)kOffScale + (uint32_t)(P & 3) * kScaleSlotBytes + (uint32_t)(nb & 3);
      smem[a + 4u * (uint32_t)r] = 127;
      smem[a + 4u * (uint32_t)(256 + r)] = 127;
    }
    const uint32_t so = (uint32_t)((S - 1) & 3) * kStageBytes;
#pragma unroll
    for (int op = 0; op < 2; ++op) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int lim = K - (64 * (s0 + S - 1) + 16 * c);
        if (lim < 16) {
          v4i* q = reinterpret_cast<v4i*>(smem + so + (uint32_t)(op * kOpBytes + r * 64) +
                                          (uint32_t)((c ^ ((r >> 2) & 3)) << 4));
          *q = mask_bytes(*q, lim);
        }
      }
    }
  };

  if (S > 0) {
    // ---- DMA schedule.  Load i (0..8) of iteration j: code loads 0..7 of stage j+4 (into
    //      the slot of stage j, freed at iteration j's barrier), then the scale load.  They
    //      are issued two per step over steps 4j+1 .. 4j+4 (the scale load last), so the four
    //      waves, which leave the barrier together, never queue their loads at once.
    auto dma_part = [&](int j, int i) __attribute__((always_inline)) {
      if (i < 8)
        issue_codes(j + 4, i);
      else
        issue_scale(j);
    };
    // ---- prologue: pseudo-iterations -6..-1 (scale words 0..2, stages 0..3); loads 6..8
    //      of iteration -1 come from iteration 0's first step, as in every iteration
    issue_scale(-6);
    issue_scale(-5);
#pragma unroll
    for (int j = -4; j < -1; ++j) {
#pragma unroll
      for (int n = 0; n < 8; ++n) issue_codes(j + 4, n);
      issue_scale(j);
    }
#pragma unroll
    for (int n = 0; n < 6; ++n) issue_codes(3, n);
    // stage 0 and scale word 0 landed: 25 loads were issued after stage 0's codes
    wait_vm<25>();
    lds_barrier();
    if (last_range && K < 64 * S_all) {
      if (S == 1) {
        mask_last_stage();
        lds_barrier();
      }
    }
#pragma unroll
    for (int f = 0; f < 8; ++f) read_codes(0, f);
#pragma unroll
    for (int f = 0; f < 8; ++f) read_codes(1, f);
#pragma unroll
    for (int f = 0; f < 8; ++f) read_scale(0, f);
    fix_scale(0);
#pragma unroll
    for (int f = 0; f < 8; ++f) make_sf(0, f);
#pragma unroll
    for (int q = 0; q < 16; ++q) convert(0, 0, 0, q);

    // ---- K loop: iteration s runs steps 4s..4s+3 (blocks 2s, 2s+1 of stage s).  Step t
    //      issues its 16 MFMAs on opd[t & 1] and, between them, converts the next step's
    //      codes into opd[(t + 1) & 1].  Block b's codes are read two steps before their
    //      first conversion (into code[b & 1]) and its scale values one step before (into
    //      sf[b & 1]).
    for (int s = 0; s < S; ++s) {
      // step 4s: convert block 2s half 1; scale values of block 2s+1; frags 4..7 of block
      // 2s+1 (frags 0..3 were read in step 4s-1; the prologue reads block 1 whole, and
      // iteration 0 reads its frags 4..7 again, from the same stage);
      // DMA loads 6..8 of iteration s-1
      if constexpr (BNT == 256) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        mfma(0, m);
        convert(1, 2 * s, 1, m);
        if (m >= 8) make_sf(2 * s + 1, m - 8);
        if ((m & 3) == 1) read_codes(2 * s + 1, 4 + (m >> 2));
        if (m == 3 || m == 8 || m == 13) dma_part(s - 1, m == 3 ? 6 : (m == 8 ? 7 : 8));
      }
      // stage s+1 landed everywhere (19 loads were issued after its codes), and every wave
      // has finished reading stage s, whose slot the DMA of stage s+4 now reuses
      wait_vm<19>();
      lds_barrier();
      if (last_range && K < 64 * S_all) {
        if (s == S - 2) {
          mask_last_stage();
          lds_barrier();
        }
      }
      if constexpr (BNT == 256) __builtin_amdgcn_sched_barrier(0);
      // step 4s+1: convert block 2s+1 half 0; read the scale word of block 2s+2 and frags
      // 0..3 of block 2s+2 (stage s+1); DMA loads 0, 1 of iteration s
      const int Pn = (s + 1) >> 1;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        mfma(1, m);
        convert(0, 2 * s + 1, 0, m);
        if ((m & 1) == 0) read_scale(Pn, m >> 1);
        if ((m & 3) == 1) read_codes(2 * s + 2, m >> 2);
        if (m == 6 || m == 14) dma_part(s, m >> 3);
      }
      fix_scale(Pn);
      // step 4s+2: convert block 2s+1 half 1; scale values of block 2s+2; frags 4..7 of
      // block 2s+2; DMA loads 2, 3
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        mfma(0, m);
        convert(1, 2 * s + 1, 1, m);
        if (m >= 8) make_sf(2 * s + 2, m - 8);
        if ((m & 3) == 1) read_codes(2 * s + 2, 4 + (m >> 2));
        if (m == 6 || m == 14) dma_part(s, 2 + (m >> 3));
      }
      // step 4s+3: convert block 2s+2 half 0; frags 0..3 of block 2s+3 (stage s+1; frags
      // 4..7 follow in step 4s+4); DMA loads 4, 5
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        mfma(1, m);
        convert(0, 2 * s + 2, 0, m);
        if ((m & 3) == 1) read_codes(2 * s + 3, m >> 2);
        if (m == 6 || m == 14) dma_part(s, 4 + (m >> 3));
      }
    }
    // loads 6..8 of the last iteration
#pragma unroll
    for (int i = 6; i < 9; ++i) dma_part(S - 1, i);
    // every DMA landed and every wave is done with LDS before the epilogue stages there
    wait_vm<0>();
    lds_barrier();
  }
  if (BNT == 256 && sp.fix) {
    // the tile's first two range slots of the workspace, row-major 256 x 256 FP32, added:
    // ranges 0 and 1, or with more ranges the sum of all but the last and the last one
    // (k_gemm_ex_sum_ranges put them there), so the total is added in range order
    const float* p0 = sp.part + (int64_t)sp.ks * (t - sp.full) * kPartFloats;
    const float* p1 = p0 + kPartFloats;
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int fj = 0; fj < 4; ++fj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          typedef float v4f __attribute__((ext_vector_type(4)));
          const int off = (128 * wm + 32 * fi + li) * 256 + 128 * wn + 32 * fj + 8 * q + 4 * lg;
          const v4f a = *reinterpret_cast<const v4f*>(p0 + off), b = *reinterpret_cast<const v4f*>(p1 + off);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[fi][fj][4 * q + e] = a[e] + b[e];
        }
  }
  // a K range writes its FP32 sums through the epilogue's own store path: alpha 1 (exact),
  // no bias, activation or codes, fp32 rows of 256 into its slot of the workspace
  GemmEpilogue epx = ep;
  int Mx = M, Nx = N, m0x = m0, n0x = n0;
  if (BNT == 256 && rng >= 0) {
    epx.alpha = 1.0f;
    epx.bias = nullptr;
    epx.act = 0;
    epx.y = sp.part + ((int64_t)sp.ks * (t - sp.full) + rng) * kPartFloats;
    epx.y_bf16 = 0;
    epx.ld_y = 256;
    epx.y_vec16 = 1;
    epx.qc = nullptr;
    epx.qs = nullptr;
    Mx = Nx = 256;
    m0x = n0x = 0;
  }

  // ---- epilogue: v = act(alpha * acc + bias[col]) in place.  Lane (g, i) holds
  //      Y[row 32 fi + i][col 32 fj + 8 q + 4 g + e] in acc[fi][fj][4 q + e], rows and
  //      columns relative to the wave's 128x128 block.
  const int wrow0 = m0x + 128 * wm, wcol0 = n0x + WN * wn;
  {
    // branch free: the lane's 64 bias values, four consecutive columns per (fj, q), come
    // through the bias descriptor; the addend is -0 without a bias or past N (x + -0 == x
    // for every x, -0 included)
    const bool has_bias = epx.bias != nullptr;
    const __amdgpu_buffer_rsrc_t brs = bias_rsrc(epx.bias, Nx);
    typedef float v4f __attribute__((ext_vector_type(4)));
    v4f bq[NFW][4];
#pragma unroll
    for (int fj = 0; fj < NFW; ++fj)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        bq[fj][q] = __builtin_bit_cast(
            v4f, __builtin_amdgcn_raw_buffer_load_b128(brs, 4 * (wcol0 + 32 * fj + 8 * q + 4 * lg), 0, 0));
#pragma unroll
    for (int fj = 0; fj < NFW; ++fj)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = wcol0 + 32 * fj + 8 * q + 4 * lg + e;
          const float bv = (has_bias && col < Nx) ? bq[fj][q][e] : -0.0f;
#pragma unroll
          for (int fi = 0; fi < 4; ++fi)
            acc[fi][fj][4 * q + e] = __builtin_fmaf(epx.alpha, acc[fi][fj][4 * q + e], bv);
        }
    if (epx.act) {
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int fj = 0; fj < NFW; ++fj)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[fi][fj][r] = silu(acc[fi][fj][r]);
    }
  }
  const uint32_t wbase = (uint32_t)wslot * kEpiWaveBytes;
  auto wave_lds_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };
  // stage columns of the wave's block as 128 rows of 256 bytes, 16-byte chunk c of row r at
  // chunk c ^ (r & 7); bf16 (E = 2, all WN columns) or fp32 (E = 4, columns 64 P .. 64 P + 63
  // of pass P); columns >= N are staged as +0 when zero_past_n
  auto stage_rows = [&](auto e_c, int pass, bool zero_past_n) __attribute__((always_inline)) {
    constexpr int E = decltype(e_c)::value;
    constexpr int FJN = E == 2 ? NFW : 2;
#pragma unroll
    for (int fjl = 0; fjl < FJN; ++fjl)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int fj = pass * FJN + fjl;
        if (fj >= NFW) continue;
        const int c0 = 32 * fjl + 8 * q + 4 * lg;           // first of this lane's 4 staged columns
        bool in[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) in[e] = !zero_past_n || wcol0 + 32 * fj + 8 * q + 4 * lg + e < Nx;
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) {
          const int row = 32 * fi + li;
          const uint32_t byte = (uint32_t)(c0 * E);
          const uint32_t addr = wbase + (uint32_t)row * 256u + ((((byte >> 4) ^ (uint32_t)(row & 7))) << 4) + (byte & 15);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = in[e] ? acc[fi][fj][4 * q + e] : 0.0f;
          if (E == 2) {
            typedef uint32_t v2u __attribute__((ext_vector_type(2)));
            v2u pk;
            pk[0] = pack_bf16(v[0], v[1]);
            pk[1] = pack_bf16(v[2], v[3]);
            *reinterpret_cast<v2u*>(smem + addr) = pk;
          } else {
            typedef float v4f __attribute__((ext_vector_type(4)));
            v4f pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) pk[e] = v[e];
            *reinterpret_cast<v4f*>(smem + addr) = pk;
          }
        }
      }
  };
  if (!epx.y) {
  } else if (epx.y_vec16 && m0x + BM <= Mx && n0x + BNT <= Nx) {
    // interior tile, aligned y: staged rows stored as whole 16-byte pieces
    auto store_pass = [&](auto e_c, int pass) __attribute__((always_inline)) {
      constexpr int E = decltype(e_c)::value;
      // 16-byte chunks per staged row in this pass
      const int chunks = E == 2 ? WN / 8 : (min(64, WN - 64 * pass) * 4) / 16;
      stage_rows(e_c, pass, false);
      wave_lds_sync();
#pragma unroll
      for (int it = 0; it < 32; ++it) {
        const int row = 4 * it + (lane >> 4), c = lane & 15;
        if (c < chunks) {
          const v4i v = *reinterpret_cast<const v4i*>(smem + wbase + (uint32_t)row * 256u +
                                                      ((uint32_t)(c ^ (row & 7)) << 4));
          uint8_t* dst = reinterpret_cast<uint8_t*>(epx.y) +
                         ((int64_t)(wrow0 + row) * epx.ld_y + wcol0 + (E == 2 ? 0 : 64 * pass)) * E + 16 * c;
          *reinterpret_cast<v4i*>(dst) = v;
        }
      }
      wave_lds_sync();
    };
    if (epx.y_bf16) {
      store_pass(std::integral_constant<int, 2>(), 0);
    } else {
      store_pass(std::integral_constant<int, 4>(), 0);
      store_pass(std::integral_constant<int, 4>(), 1);
    }
  } else {
#pragma unroll
    for (int fj = 0; fj < NFW; ++fj)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = wcol0 + 32 * fj + 8 * q + 4 * lg + e;
#pragma unroll
          for (int fi = 0; fi < 4; ++fi) {
            const int row = wrow0 + 32 * fi + li;
            if (row < Mx && col < Nx) {
              const float v = acc[fi][fj][4 * q + e];
              if (epx.y_bf16)
                reinterpret_cast<uint16_t*>(epx.y)[(int64_t)row * epx.ld_y + col] = (uint16_t)f32_to_bf16_rne(v);
              else
                reinterpret_cast<float*>(epx.y)[(int64_t)row * epx.ld_y + col] = v;
            }
          }
        }
  }
  if (epx.qc) {
    // bf16(v) of the wave's block staged as 128 rows of 128 values, columns >= N as +0,
    // then quantized along the rows in 32-column blocks
    stage_rows(std::integral_constant<int, 2>(), 0, true);
    wave_lds_sync();
    quantize_staged<NFW, 256>(wbase, lane, wrow0, Mx, wcol0 / 32, (Nx + 31) / 32, epx);
  }
}

// Fix-up of the split tiles when no MX codes are written: elementwise over the tiles'
// 256 x 256 outputs, 4 consecutive columns per thread, 64 workgroups per tile.
// v = act(alpha * (((h0 + h1) + h2) + ...) + bias[col]) over the tile's K ranges, rounded
// and stored as the epilogue of k_gemm_ex does it (the same FP32 operations in the same
// order, so the same bits).
__global__ __launch_bounds__(256) void k_gemm_ex_fix_ew(int M, int N, int tiles_m, int tiles_n, const GemmEpilogue ep,
                                                       const ExSplit sp) {
  const int j = (int)(blockIdx.x >> 6);                 // split tile
  const int e0 = (int)((blockIdx.x & 63) * 1024 + 4 * threadIdx.x);   // element of the tile
  const int r = e0 >> 8, c = e0 & 255;
  int tm, tn;
  tile_at(sp.full + j, tiles_m, tiles_n, tm, tn);
  const int row = tm * BM + r, col0 = tn * BN + c;
  if (row >= M || col0 >= N) return;
  typedef float v4f __attribute__((ext_vector_type(4)));
  const float* p0 = sp.part + (int64_t)sp.ks * j * kPartFloats + e0;
  v4f a = *reinterpret_cast<const v4f*>(p0);
  for (int k = 1; k < sp.ks; ++k) a += *reinterpret_cast<const v4f*>(p0 + (int64_t)k * kPartFloats);
  const bool has_bias = ep.bias != nullptr;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int col = col0 + e;
    if (col >= N) break;
    const float acc = a[e];
    float v = has_bias ? __builtin_fmaf(ep.alpha, acc, ep.bias[col]) : ep.alpha * acc;
    if (ep.act) v = silu(v);
    if (ep.y_bf16)
      reinterpret_cast<uint16_t*>(ep.y)[(int64_t)row * ep.ld_y + col] = (uint16_t)f32_to_bf16_rne(v);
    else
      reinterpret_cast<float*>(ep.y)[(int64_t)row * ep.ld_y + col] = v;
  }
}

// Before the fix-up through the kernel's own epilogue (MX codes written) of tiles split
// into more than two K ranges: ranges 0 .. ks-2 added in range order into the tile's
// first slot and the last range copied into the second, so that the kernel's sum of the
// two slots is the fix-up's ((h0 + h1) + ...) + h_{ks-1} (a fix path that reads one slot
// made the register allocator spill twice as many values in the main kernel).  4
// consecutive values per thread, 64 workgroups per tile.
__global__ __launch_bounds__(256) void k_gemm_ex_sum_ranges(const ExSplit sp) {
  const int j = (int)(blockIdx.x >> 6);                 // split tile
  const int e0 = (int)((blockIdx.x & 63) * 1024 + 4 * threadIdx.x);
  typedef float v4f __attribute__((ext_vector_type(4)));
  float* p0 = sp.part + (int64_t)sp.ks * j * kPartFloats + e0;
  v4f a = *reinterpret_cast<const v4f*>(p0);
  for (int k = 1; k < sp.ks - 1; ++k) a += *reinterpret_cast<const v4f*>(p0 + (int64_t)k * kPartFloats);
  const v4f last = *reinterpret_cast<const v4f*>(p0 + (int64_t)(sp.ks - 1) * kPartFloats);
  *reinterpret_cast<v4f*>(p0) = a;
  *reinterpret_cast<v4f*>(p0 + kPartFloats) = last;
}

// K split, with P workgroups resident at once (one per CU) and T tiles of S stages.
// Last round: when there is more than one round and the last holds R = T mod P <= P / 2
// tiles, those tiles run as 2R K halves, so the last round takes half a tile's time
// instead of a whole one.  Under-filled grid: when T <= P / 2, every tile runs as ks K
// ranges of s_per stages (the last one the rest, at most s_per), s_per even (whole scale
// words) and ks <= min(P / T, 16), so that up to P workgroups share the work, if that
// shortens the longest item by more than the split costs: about 16 stage times for the
// per-call workspace, the fix-up launch and the wider partial stores, plus the read of the
// partial sums, one stage time per 16 ranges.  Measured, whole against split: 256 x 256 x
// 512 20 against 34 us (kept whole), x 1000 29 against 28 (kept whole), x 2048 45
// against 38; 1024 x 1024 x 4096 79 against 48; 2048 x 2048 x 8192 151 against 88.  At
// most P ranges in all, so the workspace stays within P tiles of FP32.
constexpr int kMaxRanges = 16;

ExSplit plan_split(int64_t tiles, int64_t K, int cus) {
  ExSplit sp;
  sp.full = (int)tiles;
  sp.items = 0;
  sp.ks = 1;
  sp.s_per = 0;
  sp.fix = 0;
  sp.part = nullptr;
  const int64_t S = (K + 63) / 64, R = cus > 0 ? tiles % cus : 0;
  if (tiles > cus && R > 0 && 2 * R <= cus && S >= 8) {
    sp.full = (int)(tiles - R);
    sp.ks = 2;
    sp.items = (int)(2 * R);
    sp.s_per = (int)(2 * (S / 4));           // even: a whole number of scale words
  } else if (cus > 0 && tiles >= 1 && 2 * tiles <= cus && S >= 8) {
    const int64_t ks_max = cus / tiles < kMaxRanges ? cus / tiles : kMaxRanges;
    const int64_t s_per = 2 * ((S + 2 * ks_max - 1) / (2 * ks_max));
    const int64_t ks = (S + s_per - 1) / s_per;
    if (ks >= 2 && S - s_per >= 16 + ks * tiles / 16) {
      sp.full = 0;
      sp.ks = (int)ks;
      sp.items = (int)(ks * tiles);
      sp.s_per = (int)s_per;
    }
  }
  return sp;
}

// Tile width for an M x N x K problem on `cus` CUs, from an estimate of each plan's time in
// stage times of a full-width tile: a round of full-width tiles costs the S stages of K
// plus a fixed part (prologue, epilogue, launch: about 8.5 stage times); the K split makes
// a last round at most half full cost half a round plus a fix-up launch and a workspace; a
// round of 256 x 192 tiles (3/4 of the work) measured 0.83 of a full-width round.  The
// narrow tile wins where it fills its rounds better (4096 x 6144: 512 narrow tiles in two
// full rounds against 384 wide ones in one and a half).  Problems of one round keep the
// full width: there the fixed part dominates, and a narrow tile column of the edge would
// take the per-element epilogue.  MXQ_EXACT_TILE_N=256 or 192 in the environment forces a
// width.
constexpr double kRoundFixed = 8.5, kNarrowCost = 0.83, kSplitFixed = 5.0, kFixupPerTile = 0.1;

// MXQ_EXACT_KSPLIT=0 in the environment turns the K split off (every tile whole).
bool ksplit_enabled() {
  const char* e = getenv("MXQ_EXACT_KSPLIT");
  return !(e != nullptr && strcmp(e, "0") == 0);
}

int choose_tile_n(int64_t M, int64_t N, int64_t K, int cus) {
  if (const char* e = getenv("MXQ_EXACT_TILE_N")) {
    if (strcmp(e, "192") == 0) return 192;
    if (strcmp(e, "256") == 0) return 256;
  }
  const int64_t P = cus > 0 ? cus : 1, S = (K + 63) / 64, tm = (M + BM - 1) / BM;
  const int64_t T256 = tm * ((N + 255) / 256), T192 = tm * ((N + 191) / 192);
  if (T256 <= P) return 256;
  const double round = (double)S + kRoundFixed;
  const ExSplit sp = plan_split(T256, K, ksplit_enabled() ? cus : 0);
  const double wide = sp.items > 0 ? (double)(sp.full / P) * round + (double)(S / 2) + kRoundFixed + kSplitFixed +
                                         kFixupPerTile * (double)(sp.items / 2)
                                    : (double)((T256 + P - 1) / P) * round;
  const double narrow = (double)((T192 + P - 1) / P) * kNarrowCost * round;
  return narrow < wide ? 192 : 256;
}

template <int FA, int FB, int BNT>
hipError_t launch_f(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                    int64_t ld_xs, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws,
                    const GemmEpilogue& ep, const ExSplit& sp, hipStream_t stream) {
  static bool attr_set[64] = {false};
  auto kern = k_gemm_ex<FA, FB, BNT>;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!attr_set[dev]) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BNT - 1) / BNT);
  hipLaunchKernelGGL(kern, dim3(sp.full + sp.items), dim3(kThreads), kLdsBytes, stream, (int)M, (int)N, (int)K,
                     tiles_m, tiles_n, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp.items == 0) return e;
  const int split_tiles = sp.items / sp.ks;
  if (!ep.qc) {
    // plain outputs: the elementwise fix-up (64 workgroups per split tile)
    hipLaunchKernelGGL(k_gemm_ex_fix_ew, dim3(64 * split_tiles), dim3(256), 0, stream, (int)M, (int)N, tiles_m, tiles_n,
                       ep, sp);
    return hipGetLastError();
  }
  // with MX codes: the kernel's own epilogue, one wave per workgroup, four per split tile,
  // 32 KiB of LDS each, so every CU takes part (one 4-wave workgroup per tile left half
  // the CUs idle)
  if (sp.ks > 2) {
    hipLaunchKernelGGL(k_gemm_ex_sum_ranges, dim3(64 * split_tiles), dim3(256), 0, stream, sp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ExSplit fx = sp;
  fx.fix = 1;
  hipLaunchKernelGGL(kern, dim3(4 * split_tiles), dim3(64), kEpiWaveBytes, stream, (int)M, (int)N, (int)K, tiles_m,
                     tiles_n, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, fx);
  return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch_w(int bn, int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                    int64_t ld_xs, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws,
                    const GemmEpilogue& ep, const ExSplit& sp, hipStream_t stream) {
  if (bn == 192) return launch_f<FA, FB, 192>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, sp, stream);
  return launch_f<FA, FB, 256>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, sp, stream);
}

// The split plan of the chosen width: the K split exists for full-width tiles only.
ExSplit plan_for(int bn, int64_t M, int64_t N, int64_t K, int cus) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + bn - 1) / bn);
  return plan_split(tiles, K, bn == 256 && ksplit_enabled() ? cus : 0);
}

}  // namespace ex
}  // namespace

void gemm_exact_plan(int64_t M, int64_t N, int64_t K, int cus, int* tile_n, int* ranges, int* split_tiles,
                     int* whole_tiles, int64_t* workspace_bytes) {
  const int bn = ex::choose_tile_n(M, N, K, cus);
  const ex::ExSplit sp = ex::plan_for(bn, M, N, K, cus);
  *tile_n = bn;
  *ranges = sp.items > 0 ? sp.ks : 1;
  *split_tiles = sp.items > 0 ? sp.items / sp.ks : 0;
  *whole_tiles = sp.full;
  *workspace_bytes = (int64_t)sp.items * ex::kPartFloats * (int64_t)sizeof(float);
}

int64_t gemm_exact_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  int bn, ks, split, whole;
  int64_t bytes;
  gemm_exact_plan(M, N, K, device_cu_count(), &bn, &ks, &split, &whole, &bytes);
  return bytes;
}

hipError_t launch_gemm_exact(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                             int64_t ld_xs, int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws,
                             int64_t ld_ws, int w_fmt, const GemmEpilogue& ep, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream) {
  const int cus = device_cu_count();
  const int bn = ex::choose_tile_n(M, N, K, cus);
  ex::ExSplit sp = ex::plan_for(bn, M, N, K, cus);
  if (sp.items > 0) {
    if (workspace == nullptr || workspace_bytes < (int64_t)sp.items * ex::kPartFloats * (int64_t)sizeof(float))
      sp = ex::plan_for(bn, M, N, K, 0);      // no room: the whole tiles only
    else
      sp.part = static_cast<float*>(workspace);
  }
  if (x_fmt == kE4M3 && w_fmt == kE4M3)
    return ex::launch_w<0, 0>(bn, M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, sp, stream);
  if (x_fmt == kE4M3) return ex::launch_w<0, 1>(bn, M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, sp, stream);
  if (w_fmt == kE4M3) return ex::launch_w<1, 0>(bn, M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, sp, stream);
  return ex::launch_w<1, 1>(bn, M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, sp, stream);
}

}  // namespace mxq

// gemm_fp8.hip -- block-scaled FP8 GEMM on the gfx950 scaled FP8 matrix cores
// (accumulation mode MXQ_ACC_FP8_MFMA).
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
// Ping-pong kernel (FP8 matrix-core accumulation; 16-byte aligned scale rows).
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
#include "gemm_common.hpp"

namespace mxq {
namespace {

constexpr int BM = 256, BN = 256;

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


template <int FA, int FB, bool TAIL>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_pp(int M, int N, int K, int tiles_m, int tiles_n,
                                                        const uint8_t* __restrict__ xc, int64_t ld_x,
                                                        const uint8_t* __restrict__ xs, int64_t ld_xs,
                                                        const uint8_t* __restrict__ wc, int64_t ld_w,
                                                        const uint8_t* __restrict__ ws, int64_t ld_ws,
                                                        const GemmEpilogue ep) {
  // ---- tile selection: XCD-first, then grouped rows
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
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
  auto any_step = [&](int s, auto par, auto last) __attribute__((always_inline)) { step(s, par, last); };
  // steps 0..T-2 in pairs (even step: opsel byte 0, odd: byte 2); the last step, which
  // may be partial, on its own
  int s = 0;
  if constexpr (TAIL) {
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
    // ranges.  The epilogue reuses the code stages, so every wave's loads must have landed
    // before any wave writes there.
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
    // branch free: the lane's 32 bias values, four consecutive columns per (fj, q), come
    // through the bias descriptor; the addend is -0 without a bias or past N (x + -0 == x
    // for every x, -0 included)
    const bool has_bias = ep.bias != nullptr;
    const __amdgpu_buffer_rsrc_t brs = bias_rsrc(ep.bias, N);
    typedef float v4f __attribute__((ext_vector_type(4)));
    v4f bq[2][4];
#pragma unroll
    for (int fj = 0; fj < 2; ++fj)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        bq[fj][q] = __builtin_bit_cast(
            v4f, __builtin_amdgcn_raw_buffer_load_b128(brs, 4 * (wcol0 + 32 * fj + 8 * q + 4 * lg), 0, 0));
#pragma unroll
    for (int fj = 0; fj < 2; ++fj)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = wcol0 + 32 * fj + 8 * q + 4 * lg + e;
          const float bv = (has_bias && col < N) ? bq[fj][q][e] : -0.0f;
#pragma unroll
          for (int fi = 0; fi < 4; ++fi)
            acc[fi][fj][4 * q + e] = __builtin_fmaf(ep.alpha, acc[fi][fj][4 * q + e], bv);
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

template <int FA, int FB, bool TAIL>
hipError_t launch_t(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                    int64_t ld_xs, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws,
                    const GemmEpilogue& ep, hipStream_t stream) {
  static bool attr_set[64] = {false};
  auto kern = k_gemm_pp<FA, FB, TAIL>;
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

// K not a multiple of 64: the kernel with the peeled, masked last step
template <int FA, int FB>
hipError_t launch_f(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                    int64_t ld_xs, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws,
                    const GemmEpilogue& ep, hipStream_t stream) {
  if (K % 64 != 0) return launch_t<FA, FB, true>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
  return launch_t<FA, FB, false>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
}

}  // namespace pp
}  // namespace

hipError_t launch_gemm_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                           int64_t ld_xs, int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws,
                           int w_fmt, const GemmEpilogue& ep, hipStream_t stream) {
  if (x_fmt == kE4M3 && w_fmt == kE4M3)
    return pp::launch_f<0, 0>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
  if (x_fmt == kE4M3) return pp::launch_f<0, 1>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
  if (w_fmt == kE4M3) return pp::launch_f<1, 0>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
  return pp::launch_f<1, 1>(M, N, K, xc, ld_x, xs, ld_xs, wc, ld_w, ws, ld_ws, ep, stream);
}

}  // namespace mxq

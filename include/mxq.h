/*
 * mxq.h -- C ABI of the MI355X (gfx950) MXFP8 library: OCP-MX block-scaled FP8
 * quantize, dequantize and GEMM  Y = X W.
 *
 * Sources ("Low-Precision GPU Programming", leetllm.com):
 *   - "Scale ownership and the GEMM dataflow": Y = X W with X in R^{M x K}, W in R^{K x N};
 *     every element is a positive scale times a low-precision code; with 32-element
 *     microscaling along K the product of the two block scales stays inside the sum
 *     over blocks, and a partial final block is zero-padded.  A consumer may apply the
 *     scales inside the GEMM; standalone dequantization is kept for debugging/fallback.
 *   - "Microscaling: the two-row experiment": 32-element blocks, one E8M0 scale byte per
 *     block (byte c means 2^(c-127), 255 is NaN); the block scale is the power of two
 *     obtained by rounding amax/fmax upward, clamped at 2^-127, and 1 for a zero block.
 *   - "Numerical hazards": round-to-nearest-even, saturating conversion to +-448 (E4M3)
 *     or +-57,344 (E5M2); subnormal codes are kept (no flush to zero).
 *   - "Hardware support and kernel ABI contracts": the kernel contract record -- X
 *     row-major with 1x32 groups along K, W column-major ("col_major_packed") with 32x1
 *     groups along K, E8M0 scales, FP32 accumulation, scales applied inside the block
 *     contraction, epilogue bias (FP32) then output cast, RNE, saturate; dtype tags,
 *     scales, orientation and padding are passed together.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library never
 *     synchronizes; work is enqueued on `stream` (a hipStream_t passed as void*; NULL
 *     means the default stream) and runs asynchronously.  Nothing is allocated, except
 *     the workspace of mxq_gemm / mxq_gemm_ex in the MXQ_ACC_FP32 mode when it splits
 *     tiles along K (see mxq_gemm_ex), which is taken from and given back
 *     to the device's stream-ordered memory pool on `stream` (hipMallocAsync /
 *     hipFreeAsync); mxq_gemm_ex_noalloc allocates nothing.
 *   - Sizes and leading dimensions are in ELEMENTS of the pointed-to type (bytes for
 *     code and scale arrays).  K is the contraction (block) axis, Kp = 32*ceil(K/32)
 *     and nb = Kp/32 is the number of blocks per line.
 *   - Return value: MXQ_OK (0) or a negative mxq_status.  All argument validation runs
 *     on the host before anything is enqueued; an invalid call enqueues nothing and
 *     never aborts.  A HIP launch error is reported as MXQ_ERR_HIP; a device fault
 *     surfaces at the caller's next synchronization.
 *   - A call with an empty problem (a zero dimension) validates its arguments and
 *     returns MXQ_OK without enqueuing work (mxq_gemm with K = 0 still writes
 *     Y = bias, or zeros).
 *   - Codes are raw OCP bytes (never the FNUZ encoding): E4M3 bias 7, NaN 0x7F/0xFF;
 *     E5M2 bias 15.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXQ_OK = 0,
  MXQ_ERR_NULL = -1,   /* a required pointer is NULL                              */
  MXQ_ERR_SHAPE = -2,  /* a negative dimension, or a size that overflows int64     */
  MXQ_ERR_LD = -3,     /* a leading dimension smaller than the row it must hold    */
  MXQ_ERR_ALIGN = -4,  /* a pointer or leading dimension breaks the stated alignment */
  MXQ_ERR_DTYPE = -5,  /* a dtype tag that the entry point does not accept         */
  MXQ_ERR_ARG = -6,    /* any other invalid argument (axis, non-finite alpha)      */
  MXQ_ERR_HIP = -7,    /* the HIP runtime reported an error when enqueuing          */
  MXQ_ERR_SCRATCH = -8 /* mxq_gemm_ex_noalloc: more workspace than its static scratch */
} mxq_status;

typedef enum {
  MXQ_F32 = 0,   /* IEEE binary32                                       */
  MXQ_BF16 = 1,  /* bfloat16 (upper half of binary32), stored as 2 bytes */
  MXQ_E4M3 = 2,  /* OCP FP8 E4M3 element code (forward operands)        */
  MXQ_E5M2 = 3   /* OCP FP8 E5M2 element code (gradients)               */
} mxq_dtype;

typedef enum {
  MXQ_ROWWISE = 0, /* 1x32 groups along each row: lines = rows, K = cols             */
  MXQ_COLWISE = 1  /* 32x1 groups down each column, output transposed: lines = cols,
                      K = rows (requantized from the wide source, not byte-transposed) */
} mxq_axis;

/*
 * Accumulation contract of mxq_gemm ("Accumulator type isn't the whole arithmetic
 * contract": a declared FP32 accumulator can hide reduced internal precision, so the
 * mode is an explicit argument).  Both modes accumulate in FP32 across the K loop.
 *
 * MXQ_ACC_FP8_MFMA  the block-scaled FP8 matrix-core instruction
 *                   (v_mfma_scale_f32_32x32x64_f8f6f4) consumes codes and E8M0 scales
 *                   directly.  Measured behaviour on gfx950: every product is exact, but
 *                   inside each group of 8 consecutive k of a block the products are
 *                   aligned to the group's largest one and truncated toward zero about 13
 *                   bits below it before the group sum; group sums, scales and the
 *                   accumulator then combine in FP32.  Error per output element
 *                   <= sum over groups g of 7 * 2^-12 * S_g * max_{k in g} |binade
 *                   products| + FP32 summation error.  Full MXFP8 matrix-core rate.
 * MXQ_ACC_FP32      exact products, FP32 sums.  Each code is decoded with its block scale
 *                   to bfloat16, x~ = bf16(dec(code) * 2^(s-127)) (round to nearest even,
 *                   bf16 subnormals kept; scale byte 255 gives NaN), and
 *                   acc = sum_k x~ * w~ is formed by v_mfma_f32_32x32x16_bf16, whose
 *                   products are exact (while they lie in FP32's normal range) and whose
 *                   sums are FP32.  x~ is exactly dec(code) * 2^(s-127) for every code when
 *                   3 <= s <= 246 (E4M3) or 10 <= s <= 239 (E5M2): the finest code bit
 *                   (2^-9, 2^-16) times the scale reaches bf16's subnormal spacing 2^-133
 *                   and the largest code (448, 57,344) times the scale stays below bf16's
 *                   maximum.  The scale rule puts every block whose amax lies in
 *                   [2^-116.2, 2^127.8] (E4M3) or [2^-102.2, 2^127.8] (E5M2) inside that
 *                   window, so for such data the result meets |y - y_exact| <= 1e-5 *
 *                   sum_k |scaled products| (plus the epilogue roundings).  Outside it the
 *                   result is the exact-product FP32 sum of the bf16-rounded operands
 *                   above.  Half the FP8 matrix-core rate at best.
 */
typedef enum { MXQ_ACC_FP8_MFMA = 0, MXQ_ACC_FP32 = 1 } mxq_accum;

/*
 * mxq_quantize -- MX block quantization of a 2-D bf16/fp32 matrix.
 *
 * src      [rows][ld_src] row-major, src_type MXQ_F32 or MXQ_BF16, ld_src >= cols.
 *          Any element alignment is accepted; 16-byte aligned rows take the fast path.
 * axis     MXQ_ROWWISE: line l = row l, K = cols.
 *          MXQ_COLWISE: line l = column l, K = rows.
 * elem     MXQ_E4M3 or MXQ_E5M2 (fmax 448 or 57,344).
 * codes    [L][ld_codes] bytes, ld_codes >= Kp, ld_codes % 16 == 0, pointer 16-byte
 *          aligned.  For each line, codes[l][0..Kp) are written; positions K..Kp-1 of
 *          the last block get 0x00 (zero padding); codes[l][Kp..ld_codes) are untouched.
 * scales   [L][ld_scales] bytes, ld_scales >= nb; scales[l][b] is the E8M0 byte of block b.
 *
 * Per block b of a line (elements 32b .. min(32b+32, K)-1):
 *   amax = max |x|;  scale byte = 127 if amax == 0, else e + 127 with e the smallest
 *   integer >= -127 such that amax <= fmax * 2^e;  code = RNE-satfinite(x * 2^-e), the
 *   sign copied from x (so -0 and negative underflow give 0x80).
 *   A block holding NaN or Inf gets scale byte 255 and every code 0x7F.
 * The result is bit-exact; it does not depend on the launch configuration.
 */
int mxq_quantize(const void* src, int src_type, int64_t rows, int64_t cols, int64_t ld_src,
                 int axis, int elem, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                 int64_t ld_scales, void* stream);

/*
 * mxq_scale_rule -- how a block's E8M0 scale is chosen from its amax.
 * MXQ_SCALE_CEIL  the rule of "Low-Precision GPU Programming", "Microscaling: the two-row
 *                 experiment": e is the smallest integer >= -127 with amax <= fmax * 2^e
 *                 (amax / fmax rounded up to a power of two), so no code saturates.  The
 *                 rule mxq_quantize and every other quantizing entry point use.
 * MXQ_SCALE_OCP   the scale-selection algorithm of the OCP Microscaling Formats (MX)
 *                 Specification v1.0, which the same section names as the alternative:
 *                 e = floor(log2 amax) - emax_elem (emax_elem = 8 for E4M3, 15 for E5M2,
 *                 the exponent of fmax), clamped at -127.  It is one below the CEIL
 *                 exponent exactly when amax's significand exceeds 1.75, and then the
 *                 codes of values above fmax * 2^e saturate to +-fmax (RNE-satfinite).
 * Both: a zero block takes scale byte 127, a block holding NaN or Inf byte 255 (codes 0x7F).
 */
typedef enum { MXQ_SCALE_CEIL = 0, MXQ_SCALE_OCP = 1 } mxq_scale_rule;

/*
 * mxq_quantize_rule -- mxq_quantize with the scale rule chosen.
 * All arguments as for mxq_quantize, plus rule (mxq_scale_rule; MXQ_ERR_ARG for any other
 * value).  rule = MXQ_SCALE_CEIL is mxq_quantize itself.  Per block: scale byte from the
 * rule above, code = RNE-satfinite(x * 2^-e) with the sign copied; bit-exact and
 * independent of the launch configuration, like mxq_quantize.
 */
int mxq_quantize_rule(const void* src, int src_type, int64_t rows, int64_t cols, int64_t ld_src,
                      int axis, int elem, int rule, uint8_t* codes, int64_t ld_codes,
                      uint8_t* scales, int64_t ld_scales, void* stream);

/*
 * mxq_quantize_sr -- mxq_quantize with stochastically rounded codes (gradients).
 * ("Rounding: RNE versus stochastic rounding": between the neighbouring representable
 * values l <= x < u, round up with probability (x - l) / (u - l), so E[SR(x)] = x and
 * representable values stay; applied to gradients, not every tensor.)
 *
 * Arguments, layouts, validation and scale bytes exactly as mxq_quantize (the scale rule
 * is unchanged, so x / S never exceeds fmax and nothing is clipped); only the codes
 * differ.  Random numbers: the element at index n = line * Kp + k of the padded code
 * array (line = row for MXQ_ROWWISE, column for MXQ_COLWISE) draws word n % 4 of
 * Philox4x32-10 (Salmon et al., SC 2011) with counter (n / 4 mod 2^32, n / 4 >> 32, 0, 0)
 * and key (seed mod 2^32, seed >> 32), and keeps its top 24 bits r; the code rounds up
 * iff r < 2^24 * (|x/S| - l) / (u - l), decided exactly.  Same seed and shape -> the same
 * bytes, independent of the launch configuration.  Pad codes are 0x00; a NaN/Inf block
 * is 0x7F throughout, as for mxq_quantize.
 */
int mxq_quantize_sr(const void* src, int src_type, int64_t rows, int64_t cols, int64_t ld_src,
                    int axis, int elem, uint64_t seed, uint8_t* codes, int64_t ld_codes,
                    uint8_t* scales, int64_t ld_scales, void* stream);

/*
 * mxq_quantize_scaled -- quantize with caller-owned scale bytes, plus diagnostics.
 * ("Worked failure: stale delayed scale": a scale taken from an earlier amax saturates a
 * later spike into a finite, wrong value; "Delayed scaling in Transformer Engine": the
 * quantization pass also records the current amax for the next scale update.)
 *
 * src, axis, elem, codes, ld_codes: as mxq_quantize.  scales [L][ld_scales] (ld >= nb) are
 * INPUT E8M0 bytes chosen by the caller (delayed, stale or any other policy).  Codes are
 * RNE-satfinite(x / S): |x / S| > fmax saturates to +-fmax (a clip), +-Inf too, NaN gives
 * 0x7F, a scale byte of 255 makes the whole block 0x7F, pad codes are 0x00.  Optional
 * per-block outputs (NULL = not written):
 *   amax    [L][ld_amax] FP32 (4-byte aligned): max |x| over the block's real elements
 *           (NaN if one is NaN) -- the value a delayed-scaling history records;
 *   clipped [L][ld_diag] uint8: elements with |x / S| > fmax;
 *   flushed [L][ld_diag] uint8: nonzero finite elements whose code is +-0.
 * With the scale bytes mxq_quantize would choose, the codes equal mxq_quantize's and
 * nothing is clipped.
 */
int mxq_quantize_scaled(const void* src, int src_type, int64_t rows, int64_t cols, int64_t ld_src,
                        int axis, int elem, const uint8_t* scales, int64_t ld_scales,
                        uint8_t* codes, int64_t ld_codes, float* amax, int64_t ld_amax,
                        uint8_t* clipped, uint8_t* flushed, int64_t ld_diag, void* stream);

/*
 * mxq_quantize_dual -- both orientations of one matrix from a single read of it.
 * ("Microscaling: the two-row experiment", closing paragraph: moving from 1x32 to 32x1
 * groups changes which values share a scale, so the second orientation is derived from
 * the wide data, not by transposing the first one's bytes.)
 *
 * Equivalent to mxq_quantize(..., MXQ_ROWWISE, elem, row_codes, ...) followed by
 * mxq_quantize(..., MXQ_COLWISE, elem, col_codes, ...) on the same src, bit for bit,
 * with the same argument rules for each output:
 *   row_codes [rows][ld_row_codes], ld >= 32*ceil(cols/32), row_scales [rows][>= ceil(cols/32)];
 *   col_codes [cols][ld_col_codes], ld >= 32*ceil(rows/32), col_scales [cols][>= ceil(rows/32)].
 * Code pointers 16-byte aligned, their leading dimensions multiples of 16.  One elem
 * (MXQ_E4M3 or MXQ_E5M2) for both.  Reads src once: 4.0625 B per bf16 element instead of
 * 2 x 3.03125 for the two separate calls.
 */
int mxq_quantize_dual(const void* src, int src_type, int64_t rows, int64_t cols, int64_t ld_src, int elem,
                      uint8_t* row_codes, int64_t ld_row_codes, uint8_t* row_scales, int64_t ld_row_scales,
                      uint8_t* col_codes, int64_t ld_col_codes, uint8_t* col_scales, int64_t ld_col_scales,
                      void* stream);

/*
 * mxq_dequantize -- reconstruction x_hat = dec(code) * 2^(s-127) (debug / fallback path).
 *
 * codes    [L][ld_codes] bytes (ld_codes >= K), scales [L][ld_scales] (ld_scales >= nb).
 * elem     MXQ_E4M3 or MXQ_E5M2.
 * dst      [L][ld_dst] of dst_type MXQ_F32 (exact; values at or beyond 2^128 become Inf)
 *          or MXQ_BF16 (round-to-nearest-even), ld_dst >= K, pointer aligned to its
 *          element size.  Scale byte 255 and NaN codes give NaN.
 */
int mxq_dequantize(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                   int64_t ld_scales, int elem, int64_t L, int64_t K, void* dst, int dst_type,
                   int64_t ld_dst, void* stream);

/*
 * mxq_gemm -- block-scaled FP8 GEMM  Y = alpha * (X W) + bias.
 *
 * X        x_codes [M][ld_x] (row-major, K contiguous), x_scales [M][ld_xs] E8M0,
 *          x_elem MXQ_E4M3 or MXQ_E5M2.
 * W        w_codes [N][ld_w]: W stored column-major, i.e. column j of the K x N matrix
 *          is the contiguous row w_codes[j][0..K) (this is what mxq_quantize gives for
 *          an [N][K] weight with MXQ_ROWWISE, or a [K][N] weight with MXQ_COLWISE);
 *          w_scales [N][ld_ws], w_elem MXQ_E4M3 or MXQ_E5M2 (mixed formats allowed).
 *          ld_x, ld_w >= Kp and multiples of 16; code pointers 16-byte aligned;
 *          ld_xs, ld_ws >= nb.  Bytes past nb of a scale row are ignored, but may be
 *          read: the MXQ_ACC_FP32 kernel reads rows other than the last in 4-byte words
 *          (never past ld), and with MXQ_ACC_FP8_MFMA and 16-byte aligned scale rows
 *          every row, the last included, is read in 16-byte units, so the last scale
 *          row must then be addressable up to 16 * ceil(nb / 16) bytes (mxq_quantize's
 *          torch wrapper allocates scale rows padded to 16 bytes).
 *          Performance: scale arrays whose base and leading dimension are multiples of
 *          4 bytes (MXQ_ACC_FP32) or 16 bytes (MXQ_ACC_FP8_MFMA) take the fastest
 *          kernel of their mode (other layouts a slower one); a 16-byte aligned y with
 *          a 16-byte multiple row pitch gets full-row stores.
 * Result   acc[i][j] = sum_b 2^(sx[i][b] + sw[j][b] - 254) * sum_{k in b, k < K}
 *                        dec(x[i][k]) * dec(w[j][k])
 *          accumulated as `accum` states (see mxq_accum; summation order is
 *          implementation-defined); code positions k >= K and scale bytes of blocks
 *          >= nb are ignored.  Epilogue: y = alpha * acc (+ bias[j] if bias != NULL, one
 *          FP32 fma), rounded once to y_type.
 * bias     [N] FP32 device array or NULL.
 * y        [M][ld_y] row-major, y_type MXQ_F32 or MXQ_BF16 (RNE), ld_y >= N, pointer
 *          aligned to its element size.
 * alpha    must be finite.
 * accum    MXQ_ACC_FP8_MFMA (fast) or MXQ_ACC_FP32 (exact products), see mxq_accum.
 * Limits   M, N < 2^31, K < 2^24, ld_x and ld_w < 2^24, ld_xs and ld_ws < 2^23.
 */
int mxq_gemm(int64_t M, int64_t N, int64_t K,
             const uint8_t* x_codes, int64_t ld_x, const uint8_t* x_scales, int64_t ld_xs, int x_elem,
             const uint8_t* w_codes, int64_t ld_w, const uint8_t* w_scales, int64_t ld_ws, int w_elem,
             float alpha, const float* bias, void* y, int y_type, int64_t ld_y, int accum, void* stream);

/*
 * Activation applied in the GEMM epilogue ("Hardware support and kernel ABI contracts":
 * the kernel contract's epilogue names an FP32 bias, a SiLU activation and the output
 * dtype; "Scale ownership and the GEMM dataflow": the epilogue may pipe the result into
 * a fused bias and activation).
 * MXQ_ACT_SILU  silu(v) = v / (1 + e^-v), evaluated in FP32 as v / (1 + t) for v >= 0 and
 *               v * t / (1 + t) for v < 0 with t = e^-|v| (no intermediate overflows;
 *               within 8 FP32 ulp of the exact value, plus 2^-126 absolute below).
 */
typedef enum { MXQ_ACT_NONE = 0, MXQ_ACT_SILU = 1 } mxq_act;

/*
 * mxq_gemm_ex -- mxq_gemm with an activation and a producer-fused quantized output.
 * ("Scale ownership and the GEMM dataflow": a preceding epilogue can itself produce the
 * codes and scales the next GEMM consumes -- producer fusion -- instead of a separate
 * conversion kernel reading the wide tensor back.)
 *
 * Operands, accum, alpha, bias and limits as for mxq_gemm.  Per output element
 *   v = act(alpha * acc + bias[j])          (FP32; act = MXQ_ACT_NONE or MXQ_ACT_SILU)
 * y        [M][ld_y] of y_type (F32 or BF16, RNE) receives v, as in mxq_gemm; may be NULL.
 * q_codes  [M][ld_q_codes] and q_scales [M][ld_q_scales] (may be NULL together) receive
 *          the MX quantization of bf16(v) along each row, 32-column blocks, element
 *          format q_elem (MXQ_E4M3 / MXQ_E5M2): byte for byte what
 *          mxq_quantize(Y_bf16, MXQ_ROWWISE, q_elem) gives for the bf16 Y this call
 *          writes with y_type = MXQ_BF16 -- i.e. rows ready to be the X operand of the
 *          next GEMM (K' = N).  ld_q_codes >= Np = 32*ceil(N/32) and a multiple of 16,
 *          q_codes 16-byte aligned, ld_q_scales >= Np/32; codes of columns N..Np-1 are 0.
 * At least one of y and q_codes must be given (MXQ_ERR_NULL otherwise).  Writing only
 * the codes saves the wide output's write and the quantize pass's read of it.
 *
 * Tile rounds (MXQ_ACC_FP32 with 4-byte aligned scale rows).  The output is computed in
 * 256 x 256 or 256 x 192 tiles, one per CU at a time; the width is chosen per call from
 * an estimate of the rounds each needs (the environment variable MXQ_EXACT_TILE_N = 256
 * or 192 forces it).  Tiles computed whole give identical bits at either width.  With
 * 256 x 256 tiles the K range of a tile may be split: when there are more tiles than
 * CUs and the last round holds at most half as many tiles as there are CUs, each of
 * those tiles is computed as two halves of K; when there are at most half as many tiles
 * as CUs, every tile is computed as up to 16 K ranges.  The ranges' FP32 sums are added
 * (FP32, in range order) before the epilogue: the result stays within the same bound and
 * is deterministic for a given device, but its rounding differs from the unsplit order.
 * The ranges' sums go to a workspace of 256 KiB per range, taken from the stream-ordered
 * pool for the call; if that allocation fails the tiles run whole.  MXQ_EXACT_KSPLIT=0
 * in the environment turns the split off.
 */
int mxq_gemm_ex(int64_t M, int64_t N, int64_t K,
                const uint8_t* x_codes, int64_t ld_x, const uint8_t* x_scales, int64_t ld_xs, int x_elem,
                const uint8_t* w_codes, int64_t ld_w, const uint8_t* w_scales, int64_t ld_ws, int w_elem,
                float alpha, const float* bias, int act,
                void* y, int y_type, int64_t ld_y,
                int q_elem, uint8_t* q_codes, int64_t ld_q_codes, uint8_t* q_scales, int64_t ld_q_scales,
                int accum, void* stream);

/*
 * mxq_gemm_ex_noalloc -- mxq_gemm_ex that allocates nothing, for callers that cannot call
 * hipMalloc or hipMallocAsync: work recorded under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.
 *
 * Arguments, results and errors as for mxq_gemm_ex, bit for bit.  The K split's workspace
 * (256 KiB per K range, at most one range per CU) is a file-scope device array of 64 MiB
 * (enough for a device of up to 256 CUs) that
 * every device the library runs on holds from load until the process ends; a problem
 * that would need more returns MXQ_ERR_SCRATCH.  All calls on one device share that
 * array: calls that may overlap on one device (different streams, no ordering between
 * them) race and must not be made.  No part of the array has to start at any value.
 */
int mxq_gemm_ex_noalloc(int64_t M, int64_t N, int64_t K,
                        const uint8_t* x_codes, int64_t ld_x, const uint8_t* x_scales, int64_t ld_xs, int x_elem,
                        const uint8_t* w_codes, int64_t ld_w, const uint8_t* w_scales, int64_t ld_ws, int w_elem,
                        float alpha, const float* bias, int act,
                        void* y, int y_type, int64_t ld_y,
                        int q_elem, uint8_t* q_codes, int64_t ld_q_codes, uint8_t* q_scales, int64_t ld_q_scales,
                        int accum, void* stream);

/*
 * mxq_gemm_exact_plan -- how mxq_gemm / mxq_gemm_ex in the MXQ_ACC_FP32 mode with 4-byte
 * aligned scale rows would run an M x N x K problem on a device of `cus` compute units
 * (host logic only: no device is touched, so it also answers for other CU counts), under
 * the environment overrides described at mxq_gemm_ex.  For tuning and tests; launches
 * nothing.
 *
 * Outputs (host pointers, all required): tile_n -- the tile width, 256 or 192 (tiles are
 * 256 rows tall); ranges_per_tile -- K ranges per split tile (1 when nothing is split);
 * split_tiles -- tiles computed as K ranges; whole_tiles -- tiles computed whole;
 * workspace_bytes -- the workspace the split needs (256 KiB per K range).
 * Returns MXQ_OK, MXQ_ERR_NULL, MXQ_ERR_SHAPE (M or N < 1, K < 0, or a size >= 2^31) or
 * MXQ_ERR_ARG (cus < 1).
 */
int mxq_gemm_exact_plan(int64_t M, int64_t N, int64_t K, int cus, int* tile_n, int* ranges_per_tile,
                        int* split_tiles, int* whole_tiles, int64_t* workspace_bytes);

/* Human-readable name of a status code (static storage, never NULL). */
const char* mxq_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int mxq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */

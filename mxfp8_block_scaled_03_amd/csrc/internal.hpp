// internal.hpp -- launchers shared between the C ABI layer and the kernel sources.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Rowwise quantize: line l = row l of src, K = cols.  flat: the whole problem is one
// dense run of blocks (ld_src == K == Kp, ld_codes == Kp, ld_scales == nb).
// vec: every 8-element chunk of src can be read with 16-byte loads.  rule: the scale
// rule, kRuleCeil (0, the pages') or kRuleOcp (1, the OCP MX specification's).
hipError_t launch_quant_rows(const void* src, int src_bf16, int64_t rows, int64_t K, int64_t ld_src,
                             int fmt, int rule, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                             int64_t ld_scales, bool flat, bool vec, hipStream_t stream);

// Columnwise quantize: line l = column l of src [rows][ld_src], K = rows, codes and
// scales stored [cols][ld].
hipError_t launch_quant_cols(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src,
                             int fmt, int rule, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                             int64_t ld_scales, hipStream_t stream);

// Both orientations in one pass: rowwise codes [rows][ld_rc] (K = cols) and columnwise
// codes [cols][ld_cc] (K = rows), with their scales.
hipError_t launch_quant_dual(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, int fmt,
                             uint8_t* rcodes, int64_t ld_rc, uint8_t* rscales, int64_t ld_rs, uint8_t* ccodes,
                             int64_t ld_cc, uint8_t* cscales, int64_t ld_cs, bool vec, hipStream_t stream);

// Quantize with stochastically rounded codes (rowwise, or colwise with transposed output);
// seed keys the Philox4x32-10 stream, element n of the padded code array draws word n % 4
// of counter n / 4.
hipError_t launch_quant_sr(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, bool colwise,
                           int fmt, uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool vec,
                           uint64_t seed, hipStream_t stream);

// Quantize with caller-owned scale bytes given [L][ld_given] (RNE-satfinite codes) and
// optional per-block diagnostics: amax (fp32), clipped and flushed counts (null = skip).
hipError_t launch_quant_scaled(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, bool colwise,
                               int fmt, const uint8_t* given, int64_t ld_given, uint8_t* codes, int64_t ld_codes,
                               float* amax, int64_t ld_amax, uint8_t* clipped, uint8_t* flushed, int64_t ld_diag,
                               bool vec, hipStream_t stream);

hipError_t launch_dequant(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales, int64_t ld_scales,
                          int fmt, int64_t L, int64_t K, void* dst, int dst_bf16, int64_t ld_dst,
                          bool vec, hipStream_t stream);

// What a GEMM launch writes: v = act(alpha * acc + bias[col]) (act 0: identity, 1: SiLU);
// y (may be null) receives v rounded to its type; qc/qs (qc may be null) receive the MX
// codes (format q_fmt) and E8M0 scales of bf16(v) in 32-column blocks along N, i.e. the
// bytes the rowwise quantize gives for a bf16 Y.  y_vec16: y and its rows are 16-byte
// aligned.
struct GemmEpilogue {
  float alpha;
  const float* bias;
  int act;
  void* y;
  int y_bf16;
  int64_t ld_y;
  int y_vec16;
  uint8_t* qc;
  int64_t ld_qc;
  uint8_t* qs;
  int64_t ld_qs;
  int q_fmt;
};

// The GEMM kernels (gemm_exact.hip, gemm_fp8.hip, gemm_fallback.hip); launch_gemm picks one.
// Exact-product GEMM.  workspace: device memory for the K split of the last round's tiles
// (gemm_exact_workspace_bytes(M, N, K) bytes; with less, or none, the tiles run whole).
int64_t gemm_exact_workspace_bytes(int64_t M, int64_t N, int64_t K);
// The exact GEMM's plan for `cus` CUs (host logic only): tile width, K ranges per split
// tile, split tiles, whole tiles and workspace bytes.
void gemm_exact_plan(int64_t M, int64_t N, int64_t K, int cus, int* tile_n, int* ranges, int* split_tiles,
                     int* whole_tiles, int64_t* workspace_bytes);
hipError_t launch_gemm_exact(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                             int64_t ld_xs, int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws,
                             int64_t ld_ws, int w_fmt, const GemmEpilogue& ep, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream);
hipError_t launch_gemm_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                           int64_t ld_xs, int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws,
                           int w_fmt, const GemmEpilogue& ep, hipStream_t stream);
hipError_t launch_gemm_fallback(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                                int64_t ld_xs, int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws,
                                int64_t ld_ws, int w_fmt, const GemmEpilogue& ep, int exact, hipStream_t stream);

// workspace / workspace_bytes: device memory the exact kernel may use for its K split;
// may_alloc: when it is too small, take one from the stream-ordered pool for the call.
hipError_t launch_gemm(int64_t M, int64_t N, int64_t K,
                       const uint8_t* x_codes, int64_t ld_x, const uint8_t* x_scales, int64_t ld_xs, int x_fmt,
                       const uint8_t* w_codes, int64_t ld_w, const uint8_t* w_scales, int64_t ld_ws, int w_fmt,
                       const GemmEpilogue& ep, int exact, void* workspace, int64_t workspace_bytes, bool may_alloc,
                       hipStream_t stream);

}  // namespace mxq

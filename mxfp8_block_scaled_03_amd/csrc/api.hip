// api.hip -- the C ABI declared in include/mxq.h: host-side argument validation and
// dispatch to the gfx950 kernels.  Nothing here synchronizes; the only allocation is the
// exact GEMM's split workspace (gemm.hip), which mxq_gemm_ex_noalloc takes from the
// static `scratch` array below instead.
#include "mxq.h"

#include <math.h>

#include "codec.hpp"
#include "internal.hpp"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;    // M, N, rows, cols, K below 2^31
constexpr int64_t kMaxCodeLd = (int64_t)1 << 24; // GEMM code leading dims (32-bit tile offsets)

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int to_fmt(int elem) { return elem == MXQ_E4M3 ? mxq::kE4M3 : mxq::kE5M2; }
int to_rule(int rule) { return rule == MXQ_SCALE_OCP ? mxq::kRuleOcp : mxq::kRuleCeil; }

bool is_elem(int t) { return t == MXQ_E4M3 || t == MXQ_E5M2; }
bool is_wide(int t) { return t == MXQ_F32 || t == MXQ_BF16; }

// a * b fits in int64 for non-negative a, b
bool mul_ok(int64_t a, int64_t b) { return a == 0 || b <= INT64_MAX / a; }

int hip_status(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_ERR_HIP; }

}  // namespace

extern "C" {

const char* mxq_status_string(int status) {
  switch (status) {
    case MXQ_OK: return "MXQ_OK";
    case MXQ_ERR_NULL: return "MXQ_ERR_NULL: a required pointer is NULL";
    case MXQ_ERR_SHAPE: return "MXQ_ERR_SHAPE: negative or too large dimension";
    case MXQ_ERR_LD: return "MXQ_ERR_LD: leading dimension too small or too large";
    case MXQ_ERR_ALIGN: return "MXQ_ERR_ALIGN: pointer or leading dimension misaligned";
    case MXQ_ERR_DTYPE: return "MXQ_ERR_DTYPE: dtype tag not accepted here";
    case MXQ_ERR_ARG: return "MXQ_ERR_ARG: invalid argument";
    case MXQ_ERR_HIP: return "MXQ_ERR_HIP: HIP runtime error while enqueuing";
    case MXQ_ERR_SCRATCH: return "MXQ_ERR_SCRATCH: the problem needs more workspace than the static scratch holds";
    default: return "unknown mxq status";
  }
}

int mxq_version(void) { return 102; }

int mxq_gemm_exact_plan(int64_t M, int64_t N, int64_t K, int cus, int* tile_n, int* ranges_per_tile,
                        int* split_tiles, int* whole_tiles, int64_t* workspace_bytes) {
  if (!tile_n || !ranges_per_tile || !split_tiles || !whole_tiles || !workspace_bytes) return MXQ_ERR_NULL;
  if (M < 1 || N < 1 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return MXQ_ERR_SHAPE;
  if (cus < 1) return MXQ_ERR_ARG;
  mxq::gemm_exact_plan(M, N, K, cus, tile_n, ranges_per_tile, split_tiles, whole_tiles, workspace_bytes);
  return MXQ_OK;
}

int mxq_quantize(const void* src, int src_type, int64_t rows, int64_t cols, int64_t ld_src, int axis, int elem,
                 uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, void* stream) {
  return mxq_quantize_rule(src, src_type, rows, cols, ld_src, axis, elem, MXQ_SCALE_CEIL, codes, ld_codes, scales,
                           ld_scales, stream);
}

int mxq_quantize_rule(const void* src, int src_type, int64_t rows, int64_t cols, int64_t ld_src, int axis, int elem,
                      int rule, uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, void* stream) {
  if (!is_wide(src_type) || !is_elem(elem)) return MXQ_ERR_DTYPE;
  if (axis != MXQ_ROWWISE && axis != MXQ_COLWISE) return MXQ_ERR_ARG;
  if (rule != MXQ_SCALE_CEIL && rule != MXQ_SCALE_OCP) return MXQ_ERR_ARG;
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim) return MXQ_ERR_SHAPE;
  const int64_t L = axis == MXQ_ROWWISE ? rows : cols;
  const int64_t K = axis == MXQ_ROWWISE ? cols : rows;
  const int64_t Kp = 32 * ((K + 31) / 32), nb = Kp / 32;
  if (L == 0 || K == 0) return MXQ_OK;
  if (!src || !codes || !scales) return MXQ_ERR_NULL;
  const int64_t es = src_type == MXQ_BF16 ? 2 : 4;
  if (ld_src < cols || ld_codes < Kp || ld_scales < nb) return MXQ_ERR_LD;
  if (!mul_ok(rows, ld_src * es) || !mul_ok(L, ld_codes) || !mul_ok(L, ld_scales)) return MXQ_ERR_SHAPE;
  if (!aligned(src, (uintptr_t)es) || !aligned(codes, 16) || ld_codes % 16 != 0) return MXQ_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const bool src16 = aligned(src, 16) && (ld_src * es) % 16 == 0;
  if (axis == MXQ_ROWWISE) {
    const bool vec = src16 && K % 8 == 0;
    const bool flat = vec && ld_src == K && K % 32 == 0 && ld_codes == Kp && ld_scales == nb;
    return hip_status(mxq::launch_quant_rows(src, src_type == MXQ_BF16, rows, K, ld_src, to_fmt(elem), to_rule(rule),
                                             codes, ld_codes, scales, ld_scales, flat, vec, st));
  }
  return hip_status(mxq::launch_quant_cols(src, src_type == MXQ_BF16, rows, cols, ld_src, to_fmt(elem), to_rule(rule),
                                           codes, ld_codes, scales, ld_scales, st));
}

int mxq_quantize_sr(const void* src, int src_type, int64_t rows, int64_t cols, int64_t ld_src, int axis, int elem,
                    uint64_t seed, uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                    void* stream) {
  if (!is_wide(src_type) || !is_elem(elem)) return MXQ_ERR_DTYPE;
  if (axis != MXQ_ROWWISE && axis != MXQ_COLWISE) return MXQ_ERR_ARG;
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim) return MXQ_ERR_SHAPE;
  const int64_t L = axis == MXQ_ROWWISE ? rows : cols;
  const int64_t K = axis == MXQ_ROWWISE ? cols : rows;
  const int64_t Kp = 32 * ((K + 31) / 32), nb = Kp / 32;
  if (L == 0 || K == 0) return MXQ_OK;
  if (!src || !codes || !scales) return MXQ_ERR_NULL;
  const int64_t es = src_type == MXQ_BF16 ? 2 : 4;
  if (ld_src < cols || ld_codes < Kp || ld_scales < nb) return MXQ_ERR_LD;
  if (!mul_ok(rows, ld_src * es) || !mul_ok(L, ld_codes) || !mul_ok(L, ld_scales) || !mul_ok(L, Kp))
    return MXQ_ERR_SHAPE;
  if (!aligned(src, (uintptr_t)es) || !aligned(codes, 16) || ld_codes % 16 != 0) return MXQ_ERR_ALIGN;
  const bool src16 = aligned(src, 16) && (ld_src * es) % 16 == 0;
  const bool vec = axis == MXQ_ROWWISE ? (src16 && K % 8 == 0) : src16;
  return hip_status(mxq::launch_quant_sr(src, src_type == MXQ_BF16, rows, cols, ld_src, axis == MXQ_COLWISE,
                                         to_fmt(elem), codes, ld_codes, scales, ld_scales, vec, seed,
                                         (hipStream_t)stream));
}

int mxq_quantize_scaled(const void* src, int src_type, int64_t rows, int64_t cols, int64_t ld_src, int axis,
                        int elem, const uint8_t* scales, int64_t ld_scales, uint8_t* codes, int64_t ld_codes,
                        float* amax, int64_t ld_amax, uint8_t* clipped, uint8_t* flushed, int64_t ld_diag,
                        void* stream) {
  if (!is_wide(src_type) || !is_elem(elem)) return MXQ_ERR_DTYPE;
  if (axis != MXQ_ROWWISE && axis != MXQ_COLWISE) return MXQ_ERR_ARG;
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim) return MXQ_ERR_SHAPE;
  const int64_t L = axis == MXQ_ROWWISE ? rows : cols;
  const int64_t K = axis == MXQ_ROWWISE ? cols : rows;
  const int64_t Kp = 32 * ((K + 31) / 32), nb = Kp / 32;
  if (L == 0 || K == 0) return MXQ_OK;
  if (!src || !codes || !scales) return MXQ_ERR_NULL;
  const int64_t es = src_type == MXQ_BF16 ? 2 : 4;
  if (ld_src < cols || ld_codes < Kp || ld_scales < nb) return MXQ_ERR_LD;
  if (amax && ld_amax < nb) return MXQ_ERR_LD;
  if ((clipped || flushed) && ld_diag < nb) return MXQ_ERR_LD;
  if (!mul_ok(rows, ld_src * es) || !mul_ok(L, ld_codes) || !mul_ok(L, ld_scales) ||
      (amax && !mul_ok(L, ld_amax * 4)) || ((clipped || flushed) && !mul_ok(L, ld_diag)))
    return MXQ_ERR_SHAPE;
  if (!aligned(src, (uintptr_t)es) || !aligned(codes, 16) || ld_codes % 16 != 0 || (amax && !aligned(amax, 4)))
    return MXQ_ERR_ALIGN;
  const bool src16 = aligned(src, 16) && (ld_src * es) % 16 == 0;
  const bool vec = axis == MXQ_ROWWISE ? (src16 && K % 8 == 0) : src16;
  return hip_status(mxq::launch_quant_scaled(src, src_type == MXQ_BF16, rows, cols, ld_src, axis == MXQ_COLWISE,
                                             to_fmt(elem), scales, ld_scales, codes, ld_codes, amax,
                                             amax ? ld_amax : 0, clipped, flushed, (clipped || flushed) ? ld_diag : 0,
                                             vec, (hipStream_t)stream));
}

int mxq_quantize_dual(const void* src, int src_type, int64_t rows, int64_t cols, int64_t ld_src, int elem,
                      uint8_t* row_codes, int64_t ld_row_codes, uint8_t* row_scales, int64_t ld_row_scales,
                      uint8_t* col_codes, int64_t ld_col_codes, uint8_t* col_scales, int64_t ld_col_scales,
                      void* stream) {
  if (!is_wide(src_type) || !is_elem(elem)) return MXQ_ERR_DTYPE;
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim) return MXQ_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MXQ_OK;
  if (!src || !row_codes || !row_scales || !col_codes || !col_scales) return MXQ_ERR_NULL;
  const int64_t kp_r = 32 * ((cols + 31) / 32), nb_r = kp_r / 32;
  const int64_t kp_c = 32 * ((rows + 31) / 32), nb_c = kp_c / 32;
  const int64_t es = src_type == MXQ_BF16 ? 2 : 4;
  if (ld_src < cols || ld_row_codes < kp_r || ld_row_scales < nb_r || ld_col_codes < kp_c || ld_col_scales < nb_c)
    return MXQ_ERR_LD;
  if (!mul_ok(rows, ld_src * es) || !mul_ok(rows, ld_row_codes) || !mul_ok(rows, ld_row_scales) ||
      !mul_ok(cols, ld_col_codes) || !mul_ok(cols, ld_col_scales))
    return MXQ_ERR_SHAPE;
  if (!aligned(src, (uintptr_t)es) || !aligned(row_codes, 16) || ld_row_codes % 16 != 0 || !aligned(col_codes, 16) ||
      ld_col_codes % 16 != 0)
    return MXQ_ERR_ALIGN;
  const bool vec = aligned(src, 16) && (ld_src * es) % 16 == 0 && cols % 8 == 0;
  return hip_status(mxq::launch_quant_dual(src, src_type == MXQ_BF16, rows, cols, ld_src, to_fmt(elem), row_codes,
                                           ld_row_codes, row_scales, ld_row_scales, col_codes, ld_col_codes,
                                           col_scales, ld_col_scales, vec, (hipStream_t)stream));
}

int mxq_dequantize(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales, int64_t ld_scales, int elem,
                   int64_t L, int64_t K, void* dst, int dst_type, int64_t ld_dst, void* stream) {
  if (!is_elem(elem) || !is_wide(dst_type)) return MXQ_ERR_DTYPE;
  if (L < 0 || K < 0 || L >= kMaxDim || K >= kMaxDim) return MXQ_ERR_SHAPE;
  if (L == 0 || K == 0) return MXQ_OK;
  if (!codes || !scales || !dst) return MXQ_ERR_NULL;
  const int64_t nb = (K + 31) / 32;
  const int64_t es = dst_type == MXQ_BF16 ? 2 : 4;
  if (ld_codes < K || ld_scales < nb || ld_dst < K) return MXQ_ERR_LD;
  if (!mul_ok(L, ld_codes) || !mul_ok(L, ld_dst * es) || !mul_ok(L, ld_scales)) return MXQ_ERR_SHAPE;
  if (!aligned(dst, (uintptr_t)es)) return MXQ_ERR_ALIGN;
  const bool vec = K % 8 == 0 && aligned(codes, 8) && ld_codes % 8 == 0 && aligned(dst, 16) && (ld_dst * es) % 16 == 0;
  return hip_status(mxq::launch_dequant(codes, ld_codes, scales, ld_scales, to_fmt(elem), L, K, dst,
                                        dst_type == MXQ_BF16, ld_dst, vec, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Static workspace for mxq_gemm_ex_noalloc: enough for the K split of the exact GEMM on a
// device of up to 256 CUs (at most 256 half tiles of 256 x 256 FP32 sums).  A file-scope
// device array: each device the library runs on holds its own copy from load to exit.
constexpr int64_t kScratchBytes = (int64_t)256 * 256 * 256 * 4;   // 64 MiB
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The device address of this device's copy of `scratch`, looked up once per device (the
// array's name in host code is not a device address).  nullptr if the lookup fails.
void* scratch_on_current_device() {
  static void* ptr[64] = {nullptr};
  static bool looked[64] = {false};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (!looked[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    ptr[dev] = p;
    looked[dev] = true;
  }
  return ptr[dev];
}

// mxq_gemm_ex's validation and dispatch; noalloc: the workspace is `scratch`, and nothing
// is allocated.
int gemm_ex_impl(int64_t M, int64_t N, int64_t K, const uint8_t* x_codes, int64_t ld_x, const uint8_t* x_scales,
                 int64_t ld_xs, int x_elem, const uint8_t* w_codes, int64_t ld_w, const uint8_t* w_scales,
                 int64_t ld_ws, int w_elem, float alpha, const float* bias, int act, void* y, int y_type,
                 int64_t ld_y, int q_elem, uint8_t* q_codes, int64_t ld_q_codes, uint8_t* q_scales,
                 int64_t ld_q_scales, int accum, void* stream, bool noalloc) {
  if (!is_elem(x_elem) || !is_elem(w_elem)) return MXQ_ERR_DTYPE;
  if (y && !is_wide(y_type)) return MXQ_ERR_DTYPE;
  if (q_codes && !is_elem(q_elem)) return MXQ_ERR_DTYPE;
  if (accum != MXQ_ACC_FP8_MFMA && accum != MXQ_ACC_FP32) return MXQ_ERR_ARG;
  if (act != MXQ_ACT_NONE && act != MXQ_ACT_SILU) return MXQ_ERR_ARG;
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxCodeLd) return MXQ_ERR_SHAPE;
  if (!isfinite(alpha)) return MXQ_ERR_ARG;
  if (M == 0 || N == 0) return MXQ_OK;
  const int64_t Kp = 32 * ((K + 31) / 32), nb = Kp / 32;
  if (!y && !q_codes) return MXQ_ERR_NULL;
  if (q_codes && !q_scales) return MXQ_ERR_NULL;
  if (K > 0 && (!x_codes || !x_scales || !w_codes || !w_scales)) return MXQ_ERR_NULL;
  if (K > 0) {
    if (ld_x < Kp || ld_w < Kp || ld_xs < nb || ld_ws < nb) return MXQ_ERR_LD;
    if (ld_x >= kMaxCodeLd || ld_w >= kMaxCodeLd || ld_xs >= kMaxCodeLd / 2 || ld_ws >= kMaxCodeLd / 2)
      return MXQ_ERR_LD;
    if (!aligned(x_codes, 16) || !aligned(w_codes, 16) || ld_x % 16 != 0 || ld_w % 16 != 0) return MXQ_ERR_ALIGN;
    if (!mul_ok(M, ld_x) || !mul_ok(N, ld_w) || !mul_ok(M, ld_xs) || !mul_ok(N, ld_ws)) return MXQ_ERR_SHAPE;
  }
  const int64_t ey = y_type == MXQ_BF16 ? 2 : 4;
  if (y) {
    if (ld_y < N) return MXQ_ERR_LD;
    if (!mul_ok(M, ld_y * ey)) return MXQ_ERR_SHAPE;
    if (!aligned(y, (uintptr_t)ey)) return MXQ_ERR_ALIGN;
  }
  if (q_codes) {
    const int64_t np = 32 * ((N + 31) / 32);
    if (ld_q_codes < np || ld_q_scales < np / 32) return MXQ_ERR_LD;
    if (!mul_ok(M, ld_q_codes) || !mul_ok(M, ld_q_scales)) return MXQ_ERR_SHAPE;
    if (!aligned(q_codes, 16) || ld_q_codes % 16 != 0) return MXQ_ERR_ALIGN;
  }
  if (bias && !aligned(bias, 4)) return MXQ_ERR_ALIGN;
  mxq::GemmEpilogue ep{};
  ep.alpha = alpha;
  ep.bias = bias;
  ep.act = act == MXQ_ACT_SILU ? 1 : 0;
  ep.y = y;
  ep.y_bf16 = y ? (y_type == MXQ_BF16) : 1;
  ep.ld_y = y ? ld_y : 0;
  ep.qc = q_codes;
  ep.ld_qc = q_codes ? ld_q_codes : 0;
  ep.qs = q_codes ? q_scales : nullptr;
  ep.ld_qs = q_codes ? ld_q_scales : 0;
  ep.q_fmt = q_codes ? to_fmt(q_elem) : 0;
  void* ws = nullptr;
  int64_t ws_bytes = 0;
  if (noalloc && accum == MXQ_ACC_FP32) {
    if (mxq::gemm_exact_workspace_bytes(M, N, K) > kScratchBytes) return MXQ_ERR_SCRATCH;
    ws = scratch_on_current_device();
    if (!ws) return MXQ_ERR_HIP;
    ws_bytes = kScratchBytes;
  }
  return hip_status(mxq::launch_gemm(M, N, K, x_codes, ld_x, x_scales, ld_xs, to_fmt(x_elem), w_codes, ld_w, w_scales,
                                     ld_ws, to_fmt(w_elem), ep, accum == MXQ_ACC_FP32, ws, ws_bytes, !noalloc,
                                     (hipStream_t)stream));
}

}  // namespace

extern "C" {

int mxq_gemm_ex(int64_t M, int64_t N, int64_t K, const uint8_t* x_codes, int64_t ld_x, const uint8_t* x_scales,
                int64_t ld_xs, int x_elem, const uint8_t* w_codes, int64_t ld_w, const uint8_t* w_scales,
                int64_t ld_ws, int w_elem, float alpha, const float* bias, int act, void* y, int y_type,
                int64_t ld_y, int q_elem, uint8_t* q_codes, int64_t ld_q_codes, uint8_t* q_scales,
                int64_t ld_q_scales, int accum, void* stream) {
  return gemm_ex_impl(M, N, K, x_codes, ld_x, x_scales, ld_xs, x_elem, w_codes, ld_w, w_scales, ld_ws, w_elem, alpha,
                      bias, act, y, y_type, ld_y, q_elem, q_codes, ld_q_codes, q_scales, ld_q_scales, accum, stream,
                      false);
}

int mxq_gemm_ex_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t* x_codes, int64_t ld_x,
                        const uint8_t* x_scales, int64_t ld_xs, int x_elem, const uint8_t* w_codes, int64_t ld_w,
                        const uint8_t* w_scales, int64_t ld_ws, int w_elem, float alpha, const float* bias, int act,
                        void* y, int y_type, int64_t ld_y, int q_elem, uint8_t* q_codes, int64_t ld_q_codes,
                        uint8_t* q_scales, int64_t ld_q_scales, int accum, void* stream) {
  return gemm_ex_impl(M, N, K, x_codes, ld_x, x_scales, ld_xs, x_elem, w_codes, ld_w, w_scales, ld_ws, w_elem, alpha,
                      bias, act, y, y_type, ld_y, q_elem, q_codes, ld_q_codes, q_scales, ld_q_scales, accum, stream,
                      true);
}

int mxq_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* x_codes, int64_t ld_x, const uint8_t* x_scales,
             int64_t ld_xs, int x_elem, const uint8_t* w_codes, int64_t ld_w, const uint8_t* w_scales, int64_t ld_ws,
             int w_elem, float alpha, const float* bias, void* y, int y_type, int64_t ld_y, int accum, void* stream) {
  if (!is_wide(y_type)) return MXQ_ERR_DTYPE;
  if (!y && M > 0 && N > 0 && M < kMaxDim && N < kMaxDim) {
    // the wide output is required here (mxq_gemm_ex also accepts a quantized one instead)
    if (!is_elem(x_elem) || !is_elem(w_elem)) return MXQ_ERR_DTYPE;
    if (accum != MXQ_ACC_FP8_MFMA && accum != MXQ_ACC_FP32) return MXQ_ERR_ARG;
    if (K < 0 || K >= kMaxCodeLd) return MXQ_ERR_SHAPE;
    if (!isfinite(alpha)) return MXQ_ERR_ARG;
    return MXQ_ERR_NULL;
  }
  return mxq_gemm_ex(M, N, K, x_codes, ld_x, x_scales, ld_xs, x_elem, w_codes, ld_w, w_scales, ld_ws, w_elem, alpha,
                     bias, MXQ_ACT_NONE, y, y_type, ld_y, MXQ_E4M3, nullptr, 0, nullptr, 0, accum, stream);
}

}  // extern "C"

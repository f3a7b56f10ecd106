// gemm.hip -- mx_gemm dispatch: the accumulation mode and the operands' scale layout pick
// the kernel.
//
//   exact products (MXQ_ACC_FP32), scale rows 4-byte aligned      -> gemm_exact.hip
//   FP8 matrix cores (MXQ_ACC_FP8_MFMA), scale rows 16-byte aligned -> gemm_fp8.hip
//   any other scale layout, either mode                            -> gemm_fallback.hip
#include "internal.hpp"

namespace mxq {

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                       int64_t ld_xs, int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws,
                       int w_fmt, const GemmEpilogue& ep_in, int exact, hipStream_t stream) {
  GemmEpilogue ep = ep_in;
  const int64_t ey = ep.y_bf16 ? 2 : 4;
  ep.y_vec16 = ep.y && ((uintptr_t)ep.y % 16 == 0) && ((ep.ld_y * ey) % 16 == 0);
  auto aligned = [&](uintptr_t a) {
    return ((uintptr_t)xs % a == 0) && ((uintptr_t)ws % a == 0) && ld_xs % (int64_t)a == 0 && ld_ws % (int64_t)a == 0;
  };
  if (exact) {
    if (aligned(4)) return launch_gemm_exact(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, stream);
  } else if (aligned(16)) {
    return launch_gemm_fp8(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, stream);
  }
  return launch_gemm_fallback(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, exact, stream);
}

}  // namespace mxq

// gemm.hip -- mx_gemm dispatch: the accumulation mode and the operands' scale layout pick
// the kernel.
//
//   exact products (MXQ_ACC_FP32), scale rows 4-byte aligned      -> gemm_exact.hip
//     (with a K split of the last round's tiles when that round is at most half full)
//   FP8 matrix cores (MXQ_ACC_FP8_MFMA), scale rows 16-byte aligned -> gemm_fp8.hip
//   any other scale layout, either mode                            -> gemm_fallback.hip
#include "internal.hpp"

namespace mxq {

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* xc, int64_t ld_x, const uint8_t* xs,
                       int64_t ld_xs, int x_fmt, const uint8_t* wc, int64_t ld_w, const uint8_t* ws, int64_t ld_ws,
                       int w_fmt, const GemmEpilogue& ep_in, int exact, void* workspace, int64_t workspace_bytes,
                       bool may_alloc, hipStream_t stream) {
  GemmEpilogue ep = ep_in;
  const int64_t ey = ep.y_bf16 ? 2 : 4;
  ep.y_vec16 = ep.y && ((uintptr_t)ep.y % 16 == 0) && ((ep.ld_y * ey) % 16 == 0);
  auto aligned = [&](uintptr_t a) {
    return ((uintptr_t)xs % a == 0) && ((uintptr_t)ws % a == 0) && ld_xs % (int64_t)a == 0 && ld_ws % (int64_t)a == 0;
  };
  if (exact) {
    if (aligned(4)) {
      // the K split of the last round needs a workspace: the caller's, or one taken from
      // the stream-ordered pool for this call (given back on the same stream after the
      // kernels); without one the tiles run whole
      const int64_t need = gemm_exact_workspace_bytes(M, N, K);
      void* wsp = workspace;
      int64_t wsb = workspace_bytes;
      bool own = false;
      if (need > 0 && wsb < need && may_alloc) {
        if (hipMallocAsync(&wsp, (size_t)need, stream) == hipSuccess) {
          own = true;
          wsb = need;
        } else {
          (void)hipGetLastError();           // not a launch error: run without the split
          wsp = nullptr;
          wsb = 0;
        }
      }
      const hipError_t e =
          launch_gemm_exact(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, wsp, wsb, stream);
      if (own) {
        const hipError_t f = hipFreeAsync(wsp, stream);
        if (e == hipSuccess && f != hipSuccess) return f;
      }
      return e;
    }
  } else if (aligned(16)) {
    return launch_gemm_fp8(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, stream);
  }
  return launch_gemm_fallback(M, N, K, xc, ld_x, xs, ld_xs, x_fmt, wc, ld_w, ws, ld_ws, w_fmt, ep, exact, stream);
}

}  // namespace mxq

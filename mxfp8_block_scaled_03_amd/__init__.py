"""MI355X (gfx950) MXFP8 library: OCP-MX block-scaled FP8 quantize, dequantize and GEMM.

The compute path is the HIP library ``libmxq.so`` built from ``csrc/`` (C ABI in
``include/mxq.h``).  This package only marshals arguments: the ``mxq_*`` functions
mirror the C entry points one to one (plain integers and device pointers), and
``quantize`` / ``dequantize`` / ``gemm`` are torch-tensor conveniences that allocate
outputs with torch and call them on torch's current stream.  There is no fallback:
if the library is missing, every call raises.

Sources: "Low-Precision GPU Programming" -- "Scale ownership and the GEMM dataflow"
(Y = XW, block scales inside the K sum), "Microscaling: the two-row experiment" (32-element
blocks, E8M0 scales, conservative power-of-two scale rule), "Hardware support and kernel
ABI contracts" (dtype tags, scales, orientation and padding travel together).
"""
from ._binding import (  # noqa: F401
    MXQ_ACC_FP32, MXQ_ACC_FP8_MFMA, MXQ_ACT_NONE, MXQ_ACT_SILU, MXQ_BF16, MXQ_COLWISE, MXQ_E4M3, MXQ_E5M2,
    MXQ_F32, MXQ_ROWWISE, MXQ_SCALE_CEIL, MXQ_SCALE_OCP, MxqError, dequantize, gemm, lib, library_path,
    mxq_dequantize, mxq_gemm, mxq_gemm_ex, mxq_gemm_ex_noalloc, mxq_quantize, mxq_quantize_dual, mxq_quantize_rule, mxq_quantize_scaled,
    mxq_gemm_exact_plan, mxq_quantize_sr, mxq_status_string, mxq_version,
    quantize, quantize_dual, quantize_scaled, quantize_sr,
)

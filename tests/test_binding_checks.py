"""The torch conveniences reject arguments the C ABI cannot see (host tensors, wrong
dtypes, undersized outputs or scale arrays) with ValueError before any library call.
CPU only: every check runs before the device is touched."""
import pytest
import torch

import mxfp8_block_scaled_03_amd as mxq


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def raises(fn, text):
    with pytest.raises(ValueError) as e:
        fn()
    assert text in str(e.value), str(e.value)


def test_quantize_rejections():
    raises(lambda: mxq.quantize(torch.zeros(4, 64, dtype=torch.float16)), "float32 or bfloat16")
    raises(lambda: mxq.quantize(bf(4, 64, 2)), "2-D")
    raises(lambda: mxq.quantize(bf(64, 4).t()), "unit stride")
    raises(lambda: mxq.quantize(bf(4, 64), axis="diag"), "axis")
    raises(lambda: mxq.quantize(bf(4, 64), codes=u8(3, 64)), "codes has 3 rows")
    raises(lambda: mxq.quantize(bf(4, 70), codes=u8(4, 70)), "codes has 70 columns, needs at least 96")
    raises(lambda: mxq.quantize(bf(4, 70), codes=u8(4, 96), scales=u8(4, 2)), "scales has 2 columns")
    raises(lambda: mxq.quantize(bf(4, 64), codes=torch.zeros(4, 64, dtype=torch.int8)), "codes must be torch.uint8")
    raises(lambda: mxq.quantize(bf(40, 4), axis="col", codes=u8(4, 32)), "needs at least 64")
    raises(lambda: mxq.quantize(bf(4, 64)), "CUDA")
    raises(lambda: mxq.quantize(bf(4, 64), rule="floor"), "rule")
    raises(lambda: mxq.quantize(bf(4, 64), rule="ocp"), "CUDA")


def test_other_quantizers_reject_host_tensors_and_bad_shapes():
    raises(lambda: mxq.quantize_sr(bf(4, 64), 1, codes=u8(4, 32)), "needs at least 64")
    raises(lambda: mxq.quantize_sr(bf(4, 64), 1), "CUDA")
    raises(lambda: mxq.quantize_scaled(bf(4, 64), u8(4, 3)), "[L][nb] = [4][2]")
    raises(lambda: mxq.quantize_scaled(bf(4, 64), torch.zeros(4, 2)), "scales must be torch.uint8")
    raises(lambda: mxq.quantize_scaled(bf(4, 64), u8(4, 2)), "CUDA")
    raises(lambda: mxq.quantize_dual(torch.zeros(4, 64, dtype=torch.int32)), "float32 or bfloat16")
    raises(lambda: mxq.quantize_dual(bf(4, 64)), "CUDA")


def test_dequantize_rejections():
    raises(lambda: mxq.dequantize(u8(4, 32), u8(4, 1), 33), "codes has 32 columns, needs at least 33")
    raises(lambda: mxq.dequantize(u8(4, 64), u8(4, 1), 33), "scales has 1 columns, needs at least 2")
    raises(lambda: mxq.dequantize(u8(4, 64), u8(3, 2), 64), "scales has 3 rows")
    raises(lambda: mxq.dequantize(u8(4, 64), u8(4, 2), 64, out_dtype=torch.float16), "out_dtype")
    raises(lambda: mxq.dequantize(u8(4, 64), u8(4, 2), 64), "CUDA")


def test_gemm_rejections():
    M, N, K = 8, 6, 40                     # Kp = 64, nb = 2
    ok = dict(x_codes=u8(M, 64), x_scales=u8(M, 2), w_codes=u8(N, 64), w_scales=u8(N, 2), K=K)

    def g(**kw):
        a = dict(ok)
        a.update(kw)
        return lambda: mxq.gemm(**a)
    raises(g(x_codes=u8(M, 48)), "x_codes has 48 columns, needs at least 64")
    raises(g(w_codes=u8(N, 32)), "w_codes has 32 columns")
    raises(g(x_scales=u8(M - 1, 2)), "x_scales has 7 rows, needs at least 8")
    raises(g(w_scales=u8(N, 1)), "w_scales has 1 columns, needs at least 2")
    raises(g(x_codes=torch.zeros(M, 64, dtype=torch.int16)), "x_codes must be torch.uint8")
    raises(g(bias=torch.zeros(N + 1)), "bias must be a contiguous 1-D float32 tensor of N = 6")
    raises(g(bias=torch.zeros(N, dtype=torch.float64)), "bias must be")
    raises(g(bias=torch.zeros(2 * N)[::2]), "bias must be")
    raises(g(out=torch.zeros(M, N + 1)), "out must have shape (M, N) = (8, 6)")
    raises(g(out=torch.zeros(N, M).t()), "unit stride")
    raises(g(out=torch.zeros(M, N, dtype=torch.float16)), "float32 or bfloat16")
    raises(g(accum="fp16"), "accum")
    raises(g(x_elem="e3m4"), "formats")
    raises(g(K=-1), "K must be >= 0")
    raises(g(), "CUDA")
    raises(g(bias=torch.zeros(N)), "CUDA")


def test_gemm_default_is_the_exact_mode():
    import inspect
    assert inspect.signature(mxq.gemm).parameters["accum"].default == "fp32"
    assert inspect.signature(mxq.mxq_gemm).parameters["accum"].default == mxq.MXQ_ACC_FP32
    assert inspect.signature(mxq.mxq_gemm_ex).parameters["accum"].default == mxq.MXQ_ACC_FP32

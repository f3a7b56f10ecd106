"""mxq_gemm_ex_noalloc (the allocation-free entry point, whose K-split workspace is a static
device array) against mxq_gemm_ex on the same operands: identical bytes, on two calls in a
row, the second with a smaller input (so the second call runs on scratch that still holds
the first call's sums); once with more tiles than CUs (the last round split into K
halves), once with an under-filled grid (every tile split into K ranges)."""
import ctypes

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_03_amd as mxq
from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def full_width_tiles(monkeypatch):
    """The K split exists for 256 x 256 tiles only: keep the library from picking the
    256 x 192 tile for these shapes."""
    monkeypatch.setenv("MXQ_EXACT_TILE_N", "256")

DEV = "cuda:0"


def operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(DEV)
    w = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)).to(DEV)
    xc, xs = mxq.quantize(x, "e4m3", "row")
    wc, ws = mxq.quantize(w, "e4m3", "row")
    b = torch.from_numpy(rng.standard_normal(N).astype(np.float32) * 0.5).to(DEV)
    return xc, xs, wc, ws, b


def run(fn, xc, xs, wc, ws, b, K, y):
    M, N = y.shape
    st = fn(M, N, K, xc.data_ptr(), xc.stride(0), xs.data_ptr(), xs.stride(0), mxq.MXQ_E4M3, wc.data_ptr(),
            wc.stride(0), ws.data_ptr(), ws.stride(0), mxq.MXQ_E4M3, ctypes.c_float(0.5), b.data_ptr(),
            mxq.MXQ_ACT_NONE, y.data_ptr(), mxq.MXQ_F32, y.stride(0), mxq.MXQ_E4M3, None, 0, None, 0,
            mxq.MXQ_ACC_FP32, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, mxq.mxq_status_string(st)


def test_noalloc_matches_gemm_ex_on_two_calls():
    P = torch.cuda.get_device_properties(0).multi_processor_count
    shapes = [(P * 256 + 3 * 256, 256, 1000),     # P + 3 tiles: 3 split
              (P * 256 + 100, 200, 640)]          # smaller: P + 1 tiles, 1 split
    for i, (M, N, K) in enumerate(shapes):
        say("no-alloc gemm call %d: %dx%dx%d" % (i, M, N, K))
        xc, xs, wc, ws, b = operands(M, N, K, 40 + i)
        y_ref = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        y_na = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        run(mxq.mxq_gemm_ex, xc, xs, wc, ws, b, K, y_ref)
        run(mxq.mxq_gemm_ex_noalloc, xc, xs, wc, ws, b, K, y_na)
        torch.cuda.synchronize()
        assert not torch.isnan(y_ref).any()
        assert torch.equal(y_ref.view(torch.int32), y_na.view(torch.int32)), "call %d differs" % i


def test_noalloc_matches_gemm_ex_k_ranges():
    """Under-filled grids split every tile into K ranges: 16 tiles x 16 ranges fill the
    whole static scratch (64 MiB), then a one-tile problem of 16 ranges runs on scratch
    that still holds the first call's sums; identical bytes to mxq_gemm_ex both times."""
    shapes = [(1024, 1024, 4096), (256, 256, 2048)]
    for i, (M, N, K) in enumerate(shapes):
        say("no-alloc gemm, K ranges, call %d: %dx%dx%d" % (i, M, N, K))
        xc, xs, wc, ws, b = operands(M, N, K, 50 + i)
        y_ref = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        y_na = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        run(mxq.mxq_gemm_ex, xc, xs, wc, ws, b, K, y_ref)
        run(mxq.mxq_gemm_ex_noalloc, xc, xs, wc, ws, b, K, y_na)
        torch.cuda.synchronize()
        assert not torch.isnan(y_ref).any()
        assert torch.equal(y_ref.view(torch.int32), y_na.view(torch.int32)), "call %d differs" % i

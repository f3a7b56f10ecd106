"""GPU parity of the exact-product GEMM's 256 x 192 tile (the width the library picks where
it fills the tile rounds better, e.g. 4096 x 6144 on 256 CUs).

MXQ_EXACT_TILE_N forces a width (MXQ_EXACT_KSPLIT=0 keeps every tile whole).  The two
widths run the same MFMAs over the same k16 steps for every output element, so whole tiles
must give identical bits; the narrow tile is also checked against the FP64 oracle within
1e-5 * sum_k |s x w| (every element of a ragged problem, a sample of the full-size ragged
workload), with bias, alpha, SiLU, bf16 and fp32 outputs, mixed E5M2 x E4M3 operands, and
the producer-fused MX output byte for byte against quantize of the bf16 Y."""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_block_scaled_03_amd as mxq
from gpu_helpers import check_gemm, full_check, host_src, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ENV = "MXQ_EXACT_TILE_N"
KSPLIT = "MXQ_EXACT_KSPLIT"


def operands(M, N, K, seed, fx="e4m3", fw="e4m3", xstd=1.0):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32) * np.float32(xstd)).to(DEV)
    w = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)).to(DEV)
    xc, xs = mxq.quantize(x, fx, "row")
    wc, ws = mxq.quantize(w, fw, "row")
    b = torch.from_numpy(rng.standard_normal(N).astype(np.float32) * 0.5).to(DEV)
    return xc, xs, wc, ws, b


def both_widths(monkeypatch, *args, **kw):
    """The call with each width forced and the K split off (a split changes the rounding
    order of the FP32 sums, so only whole tiles compare bit for bit)."""
    out = {}
    monkeypatch.setenv(KSPLIT, "0")
    for width in ("192", "256"):
        monkeypatch.setenv(ENV, width)
        out[width] = mxq.gemm(*args, **kw)
    monkeypatch.delenv(ENV)
    monkeypatch.delenv(KSPLIT)
    torch.cuda.synchronize()
    return out["192"], out["256"]


def same_bits(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


SHAPES = [(300, 200, 352),      # one tile row, N over one narrow tile, K ragged (11 blocks)
          (513, 385, 1000),     # three narrow tile columns, the last one column wide
          (256, 96, 64),        # N below one narrow tile, a single stage
          (1000, 1000, 4001)]   # odd block count, last stage one element


@pytest.mark.parametrize("shape", SHAPES)
def test_narrow_equals_wide_bitwise(monkeypatch, shape):
    M, N, K = shape
    say("narrow vs wide %dx%dx%d" % shape)
    xc, xs, wc, ws, b = operands(M, N, K, 50)
    y1, y2 = both_widths(monkeypatch, xc, xs, wc, ws, K, alpha=0.75, bias=b, out_dtype=torch.float32)
    assert same_bits(y1, y2)
    y1, y2 = both_widths(monkeypatch, xc, xs, wc, ws, K, out_dtype=torch.bfloat16, act="silu")
    assert same_bits(y1, y2)


def test_narrow_mixed_formats_bitwise(monkeypatch):
    M, N, K = 700, 450, 520
    xc, xs, wc, ws, _ = operands(M, N, K, 51, fx="e5m2", fw="e4m3")
    y1, y2 = both_widths(monkeypatch, xc, xs, wc, ws, K, x_elem="e5m2", w_elem="e4m3", out_dtype=torch.float32)
    assert same_bits(y1, y2)


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_narrow_every_element(monkeypatch, out):
    M, N, K = 513, 385, 1000
    say("narrow tile, every element %dx%dx%d %s" % (M, N, K, out))
    xc, xs, wc, ws, b = operands(M, N, K, 52)
    monkeypatch.setenv(ENV, "192")
    y = mxq.gemm(xc, xs, wc, ws, K, alpha=-0.5, bias=b, out_dtype=out)
    torch.cuda.synchronize()
    full_check(xc, xs, "e4m3", wc, ws, "e4m3", K, y, out, alpha=-0.5, bias=b, what="narrow tile", strict=True)


def test_narrow_ragged_workload_sampled():
    """The ragged workload's shape (4096 x 6144 x 4000), width as the library picks it: a
    sample, every tile-column edge of the narrow tiles and a whole output row."""
    M, N, K = 4096, 6144, 4000
    xc, xs, wc, ws, b = operands(M, N, K, 53)
    y = mxq.gemm(xc, xs, wc, ws, K, bias=b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    edges = np.concatenate([np.arange(0, N, 96), np.arange(95, N, 96)])
    ii = np.concatenate([rng.integers(0, M, 4000), rng.integers(0, M, edges.size), np.full(N, 4095)])
    jj = np.concatenate([rng.integers(0, N, 4000), edges, np.arange(N)])
    xc_h, xs_h, wc_h, ws_h = (a.cpu().numpy() for a in (xc, xs, wc, ws))
    y_ref, t = oracle.gemm_sampled(xc_h, xs_h, "e4m3", wc_h, ws_h, "e4m3", K, ii, jj, bias=b.cpu().numpy())
    check_gemm(y.cpu().numpy()[ii, jj], y_ref, t, torch.float32, True, "ragged workload")


def test_narrow_fused_codes(monkeypatch):
    """Producer-fused MX output from narrow tiles (three 32-column blocks per wave, the last
    block of N partial): codes and scales equal quantize of the bf16 Y of the same call."""
    M, N, K = 513, 385, 1000
    xc, xs, wc, ws, b = operands(M, N, K, 54, xstd=8.0)
    monkeypatch.setenv(ENV, "192")
    y, qc, qs = mxq.gemm(xc, xs, wc, ws, K, bias=b, out_dtype=torch.bfloat16, act="silu", quant_out="e4m3")
    monkeypatch.setenv(ENV, "256")
    monkeypatch.setenv(KSPLIT, "0")
    y2, qc2, qs2 = mxq.gemm(xc, xs, wc, ws, K, bias=b, out_dtype=torch.bfloat16, act="silu", quant_out="e4m3")
    torch.cuda.synchronize()
    rc, rs = oracle.quantize(host_src(y.cpu()), "e4m3")
    np_ = 32 * ((N + 31) // 32)
    assert np.array_equal(qc.cpu().numpy()[:, :np_], rc)
    assert np.array_equal(qs.cpu().numpy(), rs)
    assert same_bits(y, y2) and torch.equal(qc, qc2) and torch.equal(qs, qs2)

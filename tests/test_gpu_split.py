"""GPU parity of the exact-product GEMM when tiles run as K ranges: the last round of tiles
as K halves (more tiles than CUs, a last round at most half full), and every tile of an
under-filled grid (at most half as many tiles as CUs) as up to 16 ranges.  Every element of
split tiles and a sample of the rest against the FP64 oracle within 1e-5 * sum_k |s x w|,
with ragged M, N and K, a bias, alpha, bf16 and fp32 outputs and the SiLU epilogue; the
producer-fused MX output of split tiles byte for byte against quantize of the bf16 Y; and
determinism."""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_block_scaled_03_amd as mxq
from gpu_helpers import check_gemm, host_src, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def full_width_tiles(monkeypatch):
    """The K split exists for 256 x 256 tiles only: keep the library from picking the
    256 x 192 tile for these shapes."""
    monkeypatch.setenv("MXQ_EXACT_TILE_N", "256")

DEV = "cuda:0"
TILE = 256


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def splits(M, N, K):
    """Tiles that run as K halves, as the library plans them (one workgroup per CU)."""
    P = cus()
    T = ((M + TILE - 1) // TILE) * ((N + TILE - 1) // TILE)
    R = T % P
    return R if (T > P and 0 < R and 2 * R <= P and (K + 63) // 64 >= 8) else 0


def operands(M, N, K, seed, xstd=1.0):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32) * np.float32(xstd)).to(DEV)
    w = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)).to(DEV)
    xc, xs = mxq.quantize(x, "e4m3", "row")
    wc, ws = mxq.quantize(w, "e4m3", "row")
    b = torch.from_numpy(rng.standard_normal(N).astype(np.float32) * 0.5).to(DEV)
    return xc, xs, wc, ws, b


def check_at(xc, xs, wc, ws, K, y, ii, jj, out_dtype, alpha=1.0, bias=None, what=""):
    xc_h, xs_h, wc_h, ws_h = (a.cpu().numpy() for a in (xc, xs, wc, ws))
    y_ref, t = oracle.gemm_sampled(xc_h, xs_h, "e4m3", wc_h, ws_h, "e4m3", K, ii, jj, alpha=alpha,
                                   bias=None if bias is None else bias.cpu().numpy())
    yg = y.float().cpu().numpy()[ii, jj]
    return check_gemm(yg, y_ref, t, out_dtype, bias is not None or alpha != 1.0, what)


def one_tail_tile_shape():
    """P + 1 tiles in one tile column: the last (a ragged row tile) runs as two K halves."""
    P = cus()
    return P * TILE + 100, 200, 1000


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_split_tail_tile_every_element(out):
    M, N, K = one_tail_tile_shape()
    assert splits(M, N, K) == 1
    say("split tail tile %dx%dx%d %s" % (M, N, K, out))
    xc, xs, wc, ws, b = operands(M, N, K, 31)
    y = mxq.gemm(xc, xs, wc, ws, K, alpha=0.75, bias=b, out_dtype=out, accum="fp32")
    torch.cuda.synchronize()
    r0 = (M // TILE) * TILE                          # the split tile's rows
    ii, jj = np.meshgrid(np.arange(r0, M), np.arange(N), indexing="ij")
    rng = np.random.default_rng(1)
    si, sj = rng.integers(0, r0, 2000), rng.integers(0, N, 2000)
    ii = np.concatenate([ii.ravel(), si])
    jj = np.concatenate([jj.ravel(), sj])
    check_at(xc, xs, wc, ws, K, y, ii, jj, out, alpha=0.75, bias=b, what="split tail tile")


def test_split_half_full_last_round():
    """The largest split: T = 3P/2 tiles, the last P/2 of them as K halves (K = 520: odd
    block count, last stage partial, in the second half).  Every element of four split
    tiles (the first and last split, two between) and a sample of the rest."""
    P = cus()
    M, N, K = (P // 2) * TILE, 3 * TILE - 56, 520
    assert splits(M, N, K) == P // 2
    say("split half-full last round %dx%dx%d" % (M, N, K))
    xc, xs, wc, ws, _ = operands(M, N, K, 32)
    y = mxq.gemm(xc, xs, wc, ws, K, out_dtype=torch.float32, accum="fp32")
    torch.cuda.synchronize()
    # tiles are numbered in groups of 4 tile rows, column by column; the split ones are the
    # last P/2 numbers: tile rows M/256-... of the last tile columns -- check whole tile
    # rows of every tile column instead, which cover them
    rows = np.concatenate([np.arange(0, 8), np.arange(M - 300, M)])
    ii, jj = np.meshgrid(rows, np.arange(N), indexing="ij")
    rng = np.random.default_rng(2)
    ii = np.concatenate([ii.ravel(), rng.integers(0, M, 6000)])
    jj = np.concatenate([jj.ravel(), rng.integers(0, N, 6000)])
    check_at(xc, xs, wc, ws, K, y, ii, jj, torch.float32, what="split half-full round")


def test_split_silu_and_fused_codes():
    """SiLU epilogue and the producer-fused MX output on split tiles: the codes and scales
    equal quantize of the bf16 Y the same call writes, byte for byte."""
    M, N, K = one_tail_tile_shape()
    xc, xs, wc, ws, b = operands(M, N, K, 33, xstd=8.0)
    y, qc, qs = mxq.gemm(xc, xs, wc, ws, K, bias=b, out_dtype=torch.bfloat16, accum="fp32", act="silu",
                         quant_out="e4m3")
    torch.cuda.synchronize()
    rc, rs = oracle.quantize(host_src(y.cpu()), "e4m3")
    np_ = 32 * ((N + 31) // 32)
    assert np.array_equal(qc.cpu().numpy()[:, :np_], rc)
    assert np.array_equal(qs.cpu().numpy(), rs)
    # the pre-activation on the split tile within the strict bound
    v = mxq.gemm(xc, xs, wc, ws, K, bias=b, out_dtype=torch.float32, accum="fp32")
    r0 = (M // TILE) * TILE
    ii, jj = np.meshgrid(np.arange(r0, M), np.arange(N), indexing="ij")
    check_at(xc, xs, wc, ws, K, v, ii.ravel(), jj.ravel(), torch.float32, bias=b, what="split pre-activation")
    vv = v.cpu().numpy().astype(np.float64)
    s = oracle.silu(vv)
    yy = y.float().cpu().numpy().astype(np.float64)
    # bf16(silu_fp32(v)): within one bf16 rounding of the FP64 SiLU of the same v (+ the
    # FP32 SiLU's few ulp)
    tol = np.abs(s) * (2.0 ** -8 + 2.0 ** -20) + 2.0 ** -126
    assert np.all(np.abs(yy - s) <= tol)


def test_split_deterministic():
    M, N, K = one_tail_tile_shape()
    xc, xs, wc, ws, _ = operands(M, N, K, 34)
    y0 = mxq.gemm(xc, xs, wc, ws, K, out_dtype=torch.float32, accum="fp32")
    for _ in range(2):
        assert torch.equal(y0, mxq.gemm(xc, xs, wc, ws, K, out_dtype=torch.float32, accum="fp32"))


# ---- under-filled grids: every tile as ks K ranges (at most P / 2 tiles)

def ranges(M, N, K):
    """(ks, s_per) as the library plans an under-filled grid of 256 x 256 tiles, or None."""
    P = cus()
    T = ((M + TILE - 1) // TILE) * ((N + TILE - 1) // TILE)
    S = (K + 63) // 64
    if T < 1 or 2 * T > P or S < 8:
        return None
    ks_max = min(P // T, 16)
    s_per = 2 * ((S + 2 * ks_max - 1) // (2 * ks_max))
    ks = (S + s_per - 1) // s_per
    return (ks, s_per) if ks >= 2 and S - s_per >= 16 + ks * T // 16 else None


@pytest.mark.parametrize("M,N,K", [(256, 256, 2048), (200, 130, 4001), (256, 256, 1536)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_ranges_one_tile_every_element(M, N, K, out):
    """One tile split into K ranges (16 of 2 stages; 16 of 4 stages with the last one 3
    stages and a partial final block; 12 of 2 stages): every element within the strict
    bound, with bias and alpha."""
    assert ranges(M, N, K) is not None
    say("K ranges, one tile %dx%dx%d %s: %s" % (M, N, K, out, ranges(M, N, K)))
    xc, xs, wc, ws, b = operands(M, N, K, 35)
    y = mxq.gemm(xc, xs, wc, ws, K, alpha=-1.25, bias=b, out_dtype=out, accum="fp32")
    torch.cuda.synchronize()
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    check_at(xc, xs, wc, ws, K, y, ii.ravel(), jj.ravel(), out, alpha=-1.25, bias=b, what="K ranges one tile")


def test_ranges_sixteen_tiles_sampled():
    """16 tiles of a skinny problem with long K (1024 x 1024 x 4096: 16 ranges of 4 stages
    per tile, 256 items): a sample, whole rows at tile edges and a whole column."""
    M, N, K = 1024, 1024, 4096
    assert ranges(M, N, K) == (16, 4)
    xc, xs, wc, ws, b = operands(M, N, K, 36)
    y = mxq.gemm(xc, xs, wc, ws, K, bias=b, out_dtype=torch.float32, accum="fp32")
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    rows = np.array([0, 255, 256, 1023])
    ii = np.concatenate([rng.integers(0, M, 5000), np.repeat(rows, N), np.arange(M)])
    jj = np.concatenate([rng.integers(0, N, 5000), np.tile(np.arange(N), rows.size), np.full(M, 511)])
    check_at(xc, xs, wc, ws, K, y, ii, jj, torch.float32, bias=b, what="K ranges 16 tiles")


def test_ranges_fused_codes_and_determinism():
    """The producer-fused MX output of a split tile (the fix-up runs the kernel's own
    epilogue): codes and scales equal quantize of the bf16 Y of the same call; repeated
    calls give identical bytes."""
    M, N, K = 256, 256, 1536
    assert ranges(M, N, K) is not None
    xc, xs, wc, ws, b = operands(M, N, K, 37, xstd=8.0)
    y, qc, qs = mxq.gemm(xc, xs, wc, ws, K, bias=b, out_dtype=torch.bfloat16, accum="fp32", act="silu",
                         quant_out="e4m3")
    torch.cuda.synchronize()
    rc, rs = oracle.quantize(host_src(y.cpu()), "e4m3")
    assert np.array_equal(qc.cpu().numpy()[:, :N], rc)
    assert np.array_equal(qs.cpu().numpy(), rs)
    v = mxq.gemm(xc, xs, wc, ws, K, bias=b, out_dtype=torch.float32, accum="fp32")
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    check_at(xc, xs, wc, ws, K, v, ii.ravel(), jj.ravel(), torch.float32, bias=b, what="K ranges pre-activation")
    for _ in range(2):
        y2, qc2, qs2 = mxq.gemm(xc, xs, wc, ws, K, bias=b, out_dtype=torch.bfloat16, accum="fp32", act="silu",
                                quant_out="e4m3")
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)) and torch.equal(qc, qc2) and torch.equal(qs, qs2)
        assert torch.equal(v, mxq.gemm(xc, xs, wc, ws, K, bias=b, out_dtype=torch.float32, accum="fp32"))

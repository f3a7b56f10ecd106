"""GPU parity of mxq_gemm against the FP64 oracle evaluated on the GPU's own codes and
scales, in both accumulation modes:
  accum="fp32" (exact products, FP32 sums): every element within the strict bound
               |y - y_ref| <= 1e-5 * sum_k |S_X S_W Xq Wq| (+ epilogue roundings);
  accum="fp8"  (FP8 matrix cores): every element within the measured matrix-core
               contract bound; the fraction within the strict bound is reported.
See gpu_helpers for both bounds."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_03_amd as mxq
import oracle
from mxfp8_block_scaled_03_amd import workloads as wl
from gpu_helpers import full_check, sampled_check, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def quantized(rng, rows, K, std, fmt):
    x = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32) * np.float32(std)).to(DEV)
    return mxq.quantize(x, fmt, "row")


ACCS = ["fp8", "fp32"]


@pytest.fixture(params=["default", "192"], autouse=True)
def tile_width(request, monkeypatch):
    """Every exact-product test runs twice: with the tile width the library picks and with
    the 256 x 192 tile forced (the FP8 path has one width, so its second run is skipped)."""
    params = request.node.callspec.params if hasattr(request.node, "callspec") else {}
    if request.param == "192":
        if params.get("accum") == "fp8":
            pytest.skip("the tile width applies to the exact-product mode")
        monkeypatch.setenv("MXQ_EXACT_TILE_N", "192")
    return request.param


def run_case(M, N, K, fx="e4m3", fw="e4m3", out=torch.float32, alpha=1.0, bias=False, seed=0, xstd=1.0,
             what="", accum="fp8"):
    rng = np.random.default_rng(seed)
    xc, xs = quantized(rng, M, max(K, 1), xstd, fx)
    wc, ws = quantized(rng, N, max(K, 1), 0.02, fw)
    b = torch.from_numpy(rng.standard_normal(N).astype(np.float32) * 0.02).to(DEV) if bias else None
    y = mxq.gemm(xc, xs, wc, ws, K, fx, fw, alpha=alpha, bias=b, out_dtype=out, accum=accum)
    torch.cuda.synchronize()
    return full_check(xc, xs, fx, wc, ws, fw, K, y, out, alpha=alpha, bias=b, what="%s %s" % (accum, what),
                      strict=accum == "fp32")


SHAPES = [(1, 1, 1), (2, 1, 32), (5, 7, 33), (64, 64, 64), (300, 260, 200), (256, 256, 512), (257, 511, 128),
          (513, 257, 4001), (1, 300, 4096), (40, 30, 0)]


@pytest.mark.parametrize("accum", ACCS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_shapes_fp32(M, N, K, accum):
    say("gemm %dx%dx%d fp32 out, accum %s" % (M, N, K, accum))
    run_case(M, N, K, what="%dx%dx%d" % (M, N, K), accum=accum)


@pytest.mark.parametrize("accum", ACCS)
@pytest.mark.parametrize("fx,fw", [("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
def test_gemm_formats(fx, fw, accum):
    say("gemm formats %s x %s accum %s" % (fx, fw, accum))
    run_case(300, 260, 480, fx, fw, seed=1, what="%s x %s" % (fx, fw), accum=accum)


@pytest.mark.parametrize("accum", ACCS)
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("alpha,bias", [(1.0, True), (0.375, False), (-2.5, True)])
def test_gemm_epilogue(out, alpha, bias, accum):
    say("gemm epilogue %s alpha=%g bias=%s accum %s" % (out, alpha, bias, accum))
    run_case(270, 300, 352, out=out, alpha=alpha, bias=bias, seed=2, what="epilogue", accum=accum)


@pytest.mark.parametrize("accum", ACCS)
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_bias_view_unaligned(out, accum):
    """The epilogue reads the bias four columns at a time through a buffer descriptor: a
    bias starting one float into its buffer (4-byte, not 16-byte aligned) and N not a
    multiple of 4 give the same per-element parity."""
    say("gemm unaligned bias view %s accum %s" % (out, accum))
    M, N, K = 300, 301, 352
    rng = np.random.default_rng(21)
    xc, xs = quantized(rng, M, K, 1.0, "e4m3")
    wc, ws = quantized(rng, N, K, 0.02, "e4m3")
    big = torch.from_numpy(rng.standard_normal(N + 7).astype(np.float32) * 0.5).to(DEV)
    b = big[1:N + 1]
    assert b.data_ptr() % 16 == 4
    y = mxq.gemm(xc, xs, wc, ws, K, alpha=-0.75, bias=b, out_dtype=out, accum=accum)
    torch.cuda.synchronize()
    full_check(xc, xs, "e4m3", wc, ws, "e4m3", K, y, out, alpha=-0.75, bias=b, what="%s unaligned bias" % accum,
               strict=accum == "fp32")


def test_gemm_k_zero_writes_bias():
    rng = np.random.default_rng(3)
    b = torch.from_numpy(rng.standard_normal(50).astype(np.float32)).to(DEV)
    xc = torch.zeros((20, 32), dtype=torch.uint8, device=DEV)
    xs = torch.zeros((20, 1), dtype=torch.uint8, device=DEV)
    wc = torch.zeros((50, 32), dtype=torch.uint8, device=DEV)
    ws = torch.zeros((50, 1), dtype=torch.uint8, device=DEV)
    y = mxq.gemm(xc, xs, wc, ws, 0, bias=b, out_dtype=torch.float32).cpu()
    assert torch.equal(y, b.cpu().expand(20, 50))


@pytest.mark.parametrize("accum", ACCS)
def test_gemm_ignores_bytes_past_k(accum):
    """Codes at k >= K and scale bytes of blocks >= nb are never used: garbage there (even
    NaN scale bytes) must not change Y."""
    rng = np.random.default_rng(4)
    M, N, K = 70, 90, 100           # Kp = 128, nb = 4 but only ceil(100/32) = 4 blocks
    xc, xs = quantized(rng, M, K, 1.0, "e4m3")
    wc, ws = quantized(rng, N, K, 0.02, "e4m3")
    y0 = mxq.gemm(xc, xs, wc, ws, K, out_dtype=torch.float32, accum=accum)
    xg = torch.full((M, 160), 0x7E, dtype=torch.uint8, device=DEV)
    wg = torch.full((N, 160), 0x7E, dtype=torch.uint8, device=DEV)
    xg[:, :K] = xc[:, :K]
    wg[:, :K] = wc[:, :K]
    xsg = torch.full((M, 8), 255, dtype=torch.uint8, device=DEV)
    wsg = torch.full((N, 8), 255, dtype=torch.uint8, device=DEV)
    xsg[:, :4] = xs
    wsg[:, :4] = ws
    y1 = mxq.gemm(xg, xsg, wg, wsg, K, out_dtype=torch.float32, accum=accum)
    assert torch.equal(y0, y1)


def strided_scales(s, ld, offset=0):
    """Copy of a [rows][nb] scale array stored with leading dimension ld, starting `offset`
    bytes into its buffer (offset 1 makes every row start unaligned)."""
    rows, nb = s.shape
    buf = torch.full((rows * ld + offset + 8,), 255, dtype=torch.uint8, device=DEV)
    view = buf[offset:offset + rows * ld].view(rows, ld)[:, :nb]
    view.copy_(s)
    return view


@pytest.mark.parametrize("accum", ACCS)
@pytest.mark.parametrize("layout", ["ld%16", "ld%4", "ld odd", "unaligned"])
@pytest.mark.parametrize("M,N,K", [(300, 260, 4000), (257, 300, 96), (130, 70, 33), (64, 520, 4001)])
def test_gemm_scale_layouts(M, N, K, layout, accum):
    """Scale rows with a 16-byte aligned base and leading dimension take the ping-pong
    kernel, the others the 4-wave one; both must meet their accumulation mode's bound."""
    say("gemm scale layout %s %dx%dx%d accum %s" % (layout, M, N, K, accum))
    rng = np.random.default_rng(11)
    xc, xs = quantized(rng, M, K, 1.0, "e4m3")
    wc, ws = quantized(rng, N, K, 0.02, "e4m3")
    nb = xs.shape[1]
    ld = {"ld%16": (nb + 15) // 16 * 16 + 16, "ld%4": (nb + 3) // 4 * 4 + 4 + 8 * ((nb + 3) // 4 % 2 == 0),
          "ld odd": nb + 1 + (nb % 2), "unaligned": nb + 4}[layout]
    off = 1 if layout == "unaligned" else 0
    xs2, ws2 = strided_scales(xs, ld, off), strided_scales(ws, ld, off)
    y = mxq.gemm(xc, xs2, wc, ws2, K, out_dtype=torch.float32, accum=accum)
    y0 = mxq.gemm(xc, xs, wc, ws, K, out_dtype=torch.float32, accum=accum)
    torch.cuda.synchronize()
    strict = accum == "fp32"
    full_check(xc, xs, "e4m3", wc, ws, "e4m3", K, y, torch.float32, what="layout " + layout, strict=strict)
    full_check(xc, xs, "e4m3", wc, ws, "e4m3", K, y0, torch.float32, what="padded scales", strict=strict)


@pytest.mark.parametrize("accum", ACCS)
def test_gemm_two_row_fixture(accum):
    from conftest import load_golden
    g = load_golden("two_row_projection.json")
    x = torch.tensor([g["pattern_small"] * 4, g["pattern_large"] * 4], dtype=torch.float32, device=DEV)
    w_kn = torch.tensor(g["weight_pattern"] * 4, dtype=torch.float32, device=DEV).reshape(32, 1)
    xc, xs = mxq.quantize(x, "e4m3", "row")
    wc, ws = mxq.quantize(w_kn, "e4m3", "col")
    y = mxq.gemm(xc, xs, wc, ws, 32, out_dtype=torch.float32, accum=accum).cpu().numpy()[:, 0]
    assert ["%.6f" % v for v in y] == ["%.6f" % v for v in g["printed"]["mxfp8_y"]]
    sel = torch.zeros((32, 1), dtype=torch.float32, device=DEV)
    sel[3, 0] = 1.0
    sc, ss = mxq.quantize(sel, "e4m3", "col")
    ysel = mxq.gemm(xc, xs, sc, ss, 32, out_dtype=torch.float32, accum=accum).cpu().numpy()[:, 0]
    assert list(ysel) == g["selector"]["selected_mx"]


@pytest.mark.parametrize("accum", ACCS)
def test_gemm_deterministic(accum):
    rng = np.random.default_rng(5)
    xc, xs = quantized(rng, 600, 1000, 1.0, "e4m3")
    wc, ws = quantized(rng, 500, 1000, 0.02, "e4m3")
    y0 = mxq.gemm(xc, xs, wc, ws, 1000, out_dtype=torch.float32, accum=accum)
    for _ in range(3):
        assert torch.equal(y0, mxq.gemm(xc, xs, wc, ws, 1000, out_dtype=torch.float32, accum=accum))


# ----------------------------------------------------------------- full-size workloads (sampled)

@pytest.mark.parametrize("accum", ACCS)
def test_workload2_projection(accum):
    d = wl.workload2()
    xc, xs = mxq.quantize(d["x"].to(DEV), "e4m3", "row")
    wc, ws = mxq.quantize(d["w"].to(DEV), "e4m3", "row")
    for out in (torch.bfloat16, torch.float32):
        say("workload2 gemm %s accum %s" % (out, accum))
        y = mxq.gemm(xc, xs, wc, ws, d["K"], out_dtype=out, accum=accum)
        sampled_check(xc, xs, "e4m3", wc, ws, "e4m3", d["K"], y, out, what="workload2 %s %s" % (out, accum),
                      strict=accum == "fp32")


@pytest.mark.parametrize("accum", ACCS)
def test_workload4_dgrad_wgrad(accum):
    d = wl.workload4()
    dyc, dys = mxq.quantize(d["dy"].to(DEV), "e5m2", "row")
    wcc, wcs = mxq.quantize(d["w"].to(DEV), "e4m3", "col")       # W^T rows: [K][N] -> contraction over N
    say("workload4 dgrad")
    dx = mxq.gemm(dyc, dys, wcc, wcs, d["N"], "e5m2", "e4m3", out_dtype=torch.float32, accum=accum)
    sampled_check(dyc, dys, "e5m2", wcc, wcs, "e4m3", d["N"], dx, torch.float32, what="dgrad " + accum,
                  strict=accum == "fp32")
    dyt, dyts = mxq.quantize(d["dy"].to(DEV), "e5m2", "col")     # [N][M]
    xt, xts = mxq.quantize(d["x"].to(DEV), "e4m3", "col")        # [K][M]
    say("workload4 wgrad")
    dw = mxq.gemm(dyt, dyts, xt, xts, d["M"], "e5m2", "e4m3", out_dtype=torch.float32, accum=accum)
    sampled_check(dyt, dyts, "e5m2", xt, xts, "e4m3", d["M"], dw, torch.float32, what="wgrad " + accum,
                  strict=accum == "fp32")


@pytest.mark.parametrize("accum", ACCS)
@pytest.mark.parametrize("K", [4000, 4001, 4031])
def test_workload5_ragged(K, accum):
    d = wl.workload5(K=K)
    xc, xs = mxq.quantize(d["x"].to(DEV), "e4m3", "row")
    wc, ws = mxq.quantize(d["w"].to(DEV), "e4m3", "row")
    say("workload5 gemm K=%d" % K)
    y = mxq.gemm(xc, xs, wc, ws, K, out_dtype=torch.float32, accum=accum)
    sampled_check(xc, xs, "e4m3", wc, ws, "e4m3", K, y, torch.float32, what="workload5 K=%d %s" % (K, accum),
                  strict=accum == "fp32")


@pytest.mark.parametrize("accum", ACCS)
def test_workload1_full(accum):
    d = wl.workload1()
    xc, xs = mxq.quantize(d["x"].to(DEV), "e4m3", "row")
    wc, ws = mxq.quantize(d["w_kn"].to(DEV), "e4m3", "col")
    y = mxq.gemm(xc, xs, wc, ws, d["K"], out_dtype=torch.float32, accum=accum)
    full_check(xc, xs, "e4m3", wc, ws, "e4m3", d["K"], y, torch.float32, what="workload1 " + accum,
               strict=accum == "fp32")


# ----------------------------------------------------------------- exact mode at extreme scale bytes

# Scale-byte windows inside which every code * 2^(s-127) is a bfloat16 value (E4M3: the finest
# code bit 2^-9 must reach bf16's subnormal spacing 2^-133 and 448 * 2^(s-127) must stay below
# bf16's maximum; E5M2: finest bit 2^-16, maximum 57,344)
EXACT_WINDOW = {"e4m3": (3, 246), "e5m2": (10, 239)}


def quantized_fp32(rng, rows, K, scale, fmt, dist="normal"):
    v = rng.standard_normal((rows, K)) if dist == "normal" else rng.uniform(-1, 1, (rows, K))
    x = torch.from_numpy((v * scale).astype(np.float32)).to(DEV)
    return mxq.quantize(x, fmt, "row")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("case", ["huge", "tiny_inside", "tiny_outside"])
def test_exact_mode_at_extreme_scale_bytes(fmt, case):
    """The exact-product mode multiplies bf16 roundings of code * 2^(s-127).  Inside the
    window of EXACT_WINDOW those are the exact decoded values, so outputs meet the strict
    bound against the FP64 oracle: X near 1e36 (scale bytes ~233-240) and X near the small end
    of the window.  Outside it (X near 1e-36: scale bytes 0..2) the result is the exact-product
    FP32 sum of the bf16-rounded operands (the oracle's bf16 dequantization, bf16 subnormals
    kept), within 1e-5 of the sum of their absolute products.  W is scaled so that every
    product stays in FP32's normal range."""
    rng = np.random.default_rng(40 + len(case))
    M, N, K = 160, 144, 480
    lo, hi = EXACT_WINDOW[fmt]
    xmag = {"huge": 1e36, "tiny_inside": 2.0 ** (-104 if fmt == "e4m3" else -96), "tiny_outside": 1e-36}[case]
    wmag = {"huge": 0.02, "tiny_inside": 1.0, "tiny_outside": 2.0 ** 40}[case]
    xc, xs = quantized_fp32(rng, M, K, xmag, fmt)
    wc, ws = quantized_fp32(rng, N, K, wmag, "e4m3")
    xs_h = xs.cpu().numpy()
    inside = (xs_h >= lo) & (xs_h <= hi)
    say("extreme scales %s %s: X scale bytes %d..%d" % (fmt, case, xs_h.min(), xs_h.max()))
    y = mxq.gemm(xc, xs, wc, ws, K, fmt, "e4m3", out_dtype=torch.float32, accum="fp32")
    torch.cuda.synchronize()
    if case != "tiny_outside":
        assert inside.all(), "the inputs do not stay inside the exact window"
        full_check(xc, xs, fmt, wc, ws, "e4m3", K, y, torch.float32, what="exact %s %s" % (fmt, case), strict=True)
        return
    assert not inside.any(), "the inputs do not leave the exact window"
    xq = oracle.dequantize(xc.cpu().numpy(), xs_h, fmt, K, out="bf16").astype(np.uint32) << 16
    wq = oracle.dequantize(wc.cpu().numpy(), ws.cpu().numpy(), "e4m3", K, out="bf16").astype(np.uint32) << 16
    xb = xq.view(np.float32).astype(np.float64)
    wb = wq.view(np.float32).astype(np.float64)
    prod_min = np.min(np.abs(xb[xb != 0])) * np.min(np.abs(wb[wb != 0]))
    assert prod_min >= 2.0 ** -126, "a product leaves FP32's normal range"
    ref = xb @ wb.T
    t = np.abs(xb) @ np.abs(wb).T
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * t), "worst |err|/T = %g" % float(np.max(err / t))
    # the rounding is real: the exact decoded operands give a different sum somewhere
    y_exact, _ = oracle.gemm(xc.cpu().numpy(), xs_h, fmt, wc.cpu().numpy(), ws.cpu().numpy(), "e4m3", K)
    assert np.any(np.abs(ref - y_exact) > 0)


def test_exact_mode_nan_scale_gives_nan():
    """A block holding Inf quantizes to scale byte 255 with NaN codes; every output of that
    row is NaN in the exact-product mode, the others are finite and meet the strict bound."""
    rng = np.random.default_rng(47)
    M, N, K = 96, 80, 256
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(DEV)
    x[5, 70] = float("inf")
    xc, xs = mxq.quantize(x, "e4m3", "row")
    wc, ws = quantized_fp32(rng, N, K, 0.02, "e4m3")
    assert int(xs[5, 2]) == 255
    y = mxq.gemm(xc, xs, wc, ws, K, out_dtype=torch.float32, accum="fp32").cpu()
    assert torch.isnan(y[5]).all()
    keep = torch.ones(M, dtype=torch.bool)
    keep[5] = False
    assert torch.isfinite(y[keep]).all()

"""GPU parity of mxq_gemm_ex: the SiLU epilogue against the FP64 oracle's SiLU, and the
producer-fused MX output (codes and scales of bf16(Y) along N, written by the GEMM's
epilogue) against the oracle's quantize of the bf16 Y the same GEMM writes -- byte for
byte, in both kernels and both accumulation modes (16-byte aligned scale rows: the
ping-pong kernel; other layouts: the 4-wave kernel)."""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_block_scaled_03_amd as mxq
from mxfp8_block_scaled_03_amd import workloads as wl
from gpu_helpers import STRICT_REL, host_src, sampled_check, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# SiLU in FP32 (expf, one multiply, one IEEE division): within 8 FP32 ulp of the exact
# value, plus an absolute floor for results below the normal range
SILU_REL = 2.0 ** -20
SILU_ABS = 2.0 ** -126
PATHS = ["pingpong", "fallback", "pingpong_exact", "fallback_exact"]


def operands(M, N, K, seed, path, xstd=1.0, wstd=0.02, bias=True):
    rng = np.random.default_rng(seed)
    Kq = max(K, 1)
    x = torch.from_numpy(rng.standard_normal((M, Kq)).astype(np.float32) * np.float32(xstd)).to(DEV)
    w = torch.from_numpy(rng.standard_normal((N, Kq)).astype(np.float32) * np.float32(wstd)).to(DEV)
    xc, xs = mxq.quantize(x, "e4m3", "row")
    wc, ws = mxq.quantize(w, "e4m3", "row")
    if path.startswith("fallback"):             # odd scale pitch: the 4-wave kernel
        xs, ws = odd_pitch(xs), odd_pitch(ws)
    b = torch.from_numpy(rng.standard_normal(N).astype(np.float32) * 0.5).to(DEV) if bias else None
    return xc, xs, wc, ws, b


def odd_pitch(s):
    rows, nb = s.shape
    ld = nb + 1 + (nb % 2)
    buf = torch.full((rows * ld + 8,), 255, dtype=torch.uint8, device=DEV)
    v = buf[:rows * ld].view(rows, ld)[:, :nb]
    v.copy_(s)
    return v


def accum_of(path):
    return "fp32" if path.endswith("exact") else "fp8"


@pytest.fixture(params=["default", "192"], autouse=True)
def tile_width(request, monkeypatch):
    """Every exact-product test runs twice: with the tile width the library picks and with
    the 256 x 192 tile forced (the FP8 path has one width, so its second run is skipped)."""
    params = request.node.callspec.params if hasattr(request.node, "callspec") else {}
    if request.param == "192":
        fp8_only = request.node.originalname in ("test_fused_quant_respects_pitches_and_padding",
                                                 "test_ffn_pair_full_size_with_fused_quant")
        if fp8_only or (accum_of(params["path"]) if "path" in params else None) == "fp8":
            pytest.skip("the tile width applies to the exact-product mode")
        monkeypatch.setenv("MXQ_EXACT_TILE_N", "192")
    return request.param


@pytest.mark.parametrize("path", PATHS)
def test_silu_epilogue_matches_oracle_silu(path):
    """Same accumulation with and without the activation (the GEMM is deterministic):
    silu_gpu(v) against the FP64 SiLU of the GPU's own pre-activation v, over a range that
    reaches deep into both tails."""
    M, N, K = 300, 260, 480
    say("silu epilogue %s" % path)
    xc, xs, wc, ws, b = operands(M, N, K, 21, path, xstd=20.0)
    kw = dict(alpha=4.0, bias=b, out_dtype=torch.float32, accum=accum_of(path))
    v = mxq.gemm(xc, xs, wc, ws, K, **kw).cpu().numpy().astype(np.float64)
    s = mxq.gemm(xc, xs, wc, ws, K, act="silu", **kw).cpu().numpy().astype(np.float64)
    ref = oracle.silu(v)
    assert np.min(v) < -80 and np.max(v) > 80, "pre-activations do not span the tails"
    err = np.abs(s - ref)
    lim = SILU_REL * np.abs(ref) + SILU_ABS
    bad = np.argwhere(err > lim)
    assert bad.size == 0, "silu mismatch at %s: v=%r gpu=%r ref=%r" % (
        bad[0].tolist(), v[tuple(bad[0])], s[tuple(bad[0])], ref[tuple(bad[0])])


def test_silu_end_to_end_exact_accumulation():
    """Exact-product accumulation with the SiLU epilogue against silu(oracle GEMM): the
    strict 1e-5*T bound (plus the FP32 bias rounding) carried through SiLU, whose slope is
    at most 1.0998, plus the SiLU rounding."""
    M, N, K = 200, 300, 352
    xc, xs, wc, ws, b = operands(M, N, K, 22, "exact", xstd=3.0)
    s = mxq.gemm(xc, xs, wc, ws, K, alpha=1.5, bias=b, out_dtype=torch.float32, accum="fp32", act="silu")
    y_ref, t = oracle.gemm(xc.cpu().numpy(), xs.cpu().numpy(), "e4m3", wc.cpu().numpy(), ws.cpu().numpy(), "e4m3",
                           K, alpha=1.5, bias=b.cpu().numpy())
    ref = oracle.silu(y_ref)
    err = np.abs(s.cpu().numpy().astype(np.float64) - ref)
    lim = 1.1 * (STRICT_REL * t + 2.0 ** -23 * np.abs(y_ref)) + SILU_REL * np.abs(ref) + SILU_ABS
    assert np.all(err <= lim), "worst excess %g" % float(np.max(err - lim))


FUSED_SHAPES = [(1, 1, 1), (5, 7, 33), (64, 64, 64), (300, 260, 200), (257, 511, 128), (130, 70, 33),
                (256, 256, 512), (513, 257, 4001), (40, 30, 0)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("qfmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("act", [None, "silu"])
def test_fused_quant_output_equals_quantize_of_bf16_y(path, qfmt, act):
    for i, (M, N, K) in enumerate(FUSED_SHAPES):
        say("fused quant %s %s act=%s %dx%dx%d" % (path, qfmt, act, M, N, K))
        xc, xs, wc, ws, b = operands(M, N, K, 30 + i, path, xstd=2.0, bias=i % 2 == 0)
        kw = dict(alpha=0.75, bias=b, out_dtype=torch.bfloat16, accum=accum_of(path), act=act)
        y = mxq.gemm(xc, xs, wc, ws, K, **kw)
        y2, qc, qs = mxq.gemm(xc, xs, wc, ws, K, quant_out=qfmt, **kw)
        _, qc3, qs3 = mxq.gemm(xc, xs, wc, ws, K, quant_out=qfmt, wide_out=False, **kw)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), "the wide output changed when codes are also written"
        assert torch.equal(qc, qc3) and torch.equal(qs, qs3), "codes depend on whether y is written"
        oc, os_ = oracle.quantize(host_src(y.cpu()), qfmt, axis=0)
        gc, gs = qc.cpu().numpy(), qs.cpu().numpy()
        assert np.array_equal(gs, os_), "scale bytes differ from the oracle's quantize of Y"
        if not np.array_equal(gc, oc):
            j = np.argwhere(gc != oc)[0]
            raise AssertionError("code mismatch at %s: fused 0x%02x oracle 0x%02x"
                                 % (j.tolist(), gc[tuple(j)], oc[tuple(j)]))


def test_fused_quant_respects_pitches_and_padding():
    """Raw entry point into canary-filled outputs wider than needed: nothing is written past
    Np codes / Np/32 scales of a row, and the pad codes N..Np-1 are 0."""
    M, N, K = 300, 100, 96                # Np = 128
    xc, xs, wc, ws, b = operands(M, N, K, 40, "pingpong")
    qc = torch.full((M, 160), 0xCD, dtype=torch.uint8, device=DEV)
    qs = torch.full((M, 7), 0xCD, dtype=torch.uint8, device=DEV)
    st = mxq.mxq_gemm_ex(M, N, K, xc.data_ptr(), xc.stride(0), xs.data_ptr(), xs.stride(0), mxq.MXQ_E4M3,
                         wc.data_ptr(), wc.stride(0), ws.data_ptr(), ws.stride(0), mxq.MXQ_E4M3, 1.0, b.data_ptr(),
                         mxq.MXQ_ACT_SILU, None, mxq.MXQ_BF16, 0, mxq.MXQ_E5M2, qc.data_ptr(), qc.stride(0),
                         qs.data_ptr(), qs.stride(0), mxq.MXQ_ACC_FP8_MFMA, mxq._binding._stream_handle())
    assert st == 0, mxq.mxq_status_string(st)
    c, s = qc.cpu().numpy(), qs.cpu().numpy()
    assert np.all(c[:, 128:] == 0xCD) and np.all(s[:, 4:] == 0xCD)
    assert np.all(c[:, 100:128] == 0)
    y = mxq.gemm(xc, xs, wc, ws, K, bias=b, out_dtype=torch.bfloat16, act="silu", accum="fp8")
    oc, os_ = oracle.quantize(host_src(y.cpu()), "e5m2", axis=0)
    assert np.array_equal(c[:, :128], oc) and np.array_equal(s[:, :4], os_)


def test_ffn_pair_full_size_exact_accumulation():
    """The FFN pair T=16384, H=5120, I=8192 in the exact-product mode, at the strict bound
    |y - y_ref| <= 1e-5 * T (+ the epilogue roundings) on sampled outputs:
      - up projection with bias, FP32 and bf16 output;
      - up projection with bias and SiLU against silu(y_ref) of the FP64 oracle (the strict
        bound carried through SiLU, whose slope is at most 1.0998, plus the SiLU rounding);
      - the producer-fused MX codes of bf16(silu(...)) equal the GPU quantize of the unfused
        bf16 output everywhere and the oracle's quantize on sampled rows;
      - the down projection on the fused codes, bf16 and FP32 output."""
    d = wl.workload3()
    T, H, I = d["T"], d["H"], d["I"]
    say("ffn pair exact: quantize operands")
    xc, xs = mxq.quantize(d["x"].to(DEV), "e4m3", "row")
    w1c, w1s = mxq.quantize(d["w1"].to(DEV), "e4m3", "row")
    w2c, w2s = mxq.quantize(d["w2"].to(DEV), "e4m3", "row")
    b1, b2 = d["b1"].to(DEV), d["b2"].to(DEV)
    del d
    for out in (torch.float32, torch.bfloat16):
        say("ffn pair exact: up projection, bias, %s out" % out)
        v = mxq.gemm(xc, xs, w1c, w1s, H, bias=b1, out_dtype=out, accum="fp32")
        sampled_check(xc, xs, "e4m3", w1c, w1s, "e4m3", H, v, out, bias=b1, what="up exact %s" % out, n=2000,
                      strict=True)
        del v
    say("ffn pair exact: up projection with SiLU against the oracle")
    s32 = mxq.gemm(xc, xs, w1c, w1s, H, bias=b1, out_dtype=torch.float32, act="silu", accum="fp32")
    rng = np.random.default_rng(11)
    ii, jj = rng.integers(0, T, 2000), rng.integers(0, I, 2000)
    y_ref, t = oracle.gemm_sampled(xc.cpu().numpy(), xs.cpu().numpy(), "e4m3", w1c.cpu().numpy(), w1s.cpu().numpy(),
                                   "e4m3", H, ii, jj, bias=b1.cpu().numpy())
    ref = oracle.silu(y_ref)
    got = s32.cpu().numpy()[ii, jj].astype(np.float64)
    lim = 1.1 * (STRICT_REL * t + 2.0 ** -23 * np.abs(y_ref)) + SILU_REL * np.abs(ref) + SILU_ABS
    assert np.all(np.abs(got - ref) <= lim), "silu(up) worst excess %g" % float(np.max(np.abs(got - ref) - lim))
    del s32
    say("ffn pair exact: fused MX output of the up projection")
    y1 = mxq.gemm(xc, xs, w1c, w1s, H, bias=b1, out_dtype=torch.bfloat16, act="silu", accum="fp32")
    _, qc, qs = mxq.gemm(xc, xs, w1c, w1s, H, bias=b1, act="silu", quant_out="e4m3", wide_out=False, accum="fp32")
    gc, gs = mxq.quantize(y1, "e4m3", "row")
    torch.cuda.synchronize()
    assert torch.equal(qc, gc) and torch.equal(qs, gs), "fused codes differ from quantize(Y1)"
    rows = np.random.default_rng(8).choice(T, 256, replace=False)
    oc, os_ = oracle.quantize(host_src(y1[rows].cpu()), "e4m3", axis=0)
    assert np.array_equal(qc[rows].cpu().numpy(), oc) and np.array_equal(qs[rows].cpu().numpy(), os_)
    del y1, gc, gs
    for out in (torch.bfloat16, torch.float32):
        say("ffn pair exact: down projection on the fused codes, %s out" % out)
        y2 = mxq.gemm(qc, qs, w2c, w2s, I, bias=b2, out_dtype=out, accum="fp32")
        sampled_check(qc, qs, "e4m3", w2c, w2s, "e4m3", I, y2, out, bias=b2, what="down exact %s" % out, n=2000,
                      strict=True)
        del y2


def test_ffn_pair_full_size_with_fused_quant():
    """The FFN pair T=16384, H=5120, I=8192 on the FP8 matrix cores (accum="fp8"): the up
    projection with bias and SiLU writes the MX codes of its output directly, and the down
    projection consumes them.  Checks: up
    projection (no activation) sampled against the oracle under the matrix-core bound; the
    SiLU output against the FP64 SiLU of the GPU's own pre-activation on sampled rows; the
    fused codes equal the GPU quantize of the unfused bf16 output everywhere and the
    oracle's quantize on sampled rows; the down projection on the fused codes sampled
    against the oracle."""
    d = wl.workload3()
    T, H, I = d["T"], d["H"], d["I"]
    say("ffn pair: quantize operands")
    xc, xs = mxq.quantize(d["x"].to(DEV), "e4m3", "row")
    w1c, w1s = mxq.quantize(d["w1"].to(DEV), "e4m3", "row")
    w2c, w2s = mxq.quantize(d["w2"].to(DEV), "e4m3", "row")
    b1, b2 = d["b1"].to(DEV), d["b2"].to(DEV)
    del d
    say("ffn pair: up projection, pre-activation")
    v = mxq.gemm(xc, xs, w1c, w1s, H, bias=b1, out_dtype=torch.float32, accum="fp8")
    sampled_check(xc, xs, "e4m3", w1c, w1s, "e4m3", H, v, torch.float32, bias=b1, what="up", n=2000)
    say("ffn pair: up projection with SiLU, unfused and fused")
    y1 = mxq.gemm(xc, xs, w1c, w1s, H, bias=b1, out_dtype=torch.bfloat16, act="silu", accum="fp8")
    s32 = mxq.gemm(xc, xs, w1c, w1s, H, bias=b1, out_dtype=torch.float32, act="silu", accum="fp8")
    _, qc, qs = mxq.gemm(xc, xs, w1c, w1s, H, bias=b1, act="silu", quant_out="e4m3", wide_out=False, accum="fp8")
    gc, gs = mxq.quantize(y1, "e4m3", "row")
    torch.cuda.synchronize()
    assert torch.equal(qc, gc) and torch.equal(qs, gs), "fused codes differ from quantize(Y1)"
    rows = np.random.default_rng(7).choice(T, 384, replace=False)
    vr = v[rows].cpu().numpy().astype(np.float64)
    sr = s32[rows].cpu().numpy().astype(np.float64)
    ref = oracle.silu(vr)
    assert np.all(np.abs(sr - ref) <= SILU_REL * np.abs(ref) + SILU_ABS)
    oc, os_ = oracle.quantize(host_src(y1[rows].cpu()), "e4m3", axis=0)
    assert np.array_equal(qc[rows].cpu().numpy(), oc) and np.array_equal(qs[rows].cpu().numpy(), os_)
    del v, s32, y1, gc, gs
    say("ffn pair: down projection on the fused codes")
    y2 = mxq.gemm(qc, qs, w2c, w2s, I, bias=b2, out_dtype=torch.bfloat16, accum="fp8")
    sampled_check(qc, qs, "e4m3", w2c, w2s, "e4m3", I, y2, torch.bfloat16, bias=b2, what="down", n=2000)

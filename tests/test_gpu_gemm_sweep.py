"""Seeded random sweep of the exact-product GEMM (accum="fp32") against the FP64 oracle at
the strict bound |y - y_ref| <= 1e-5 * sum_k |s x w| (+ epilogue roundings): random M, N,
K (ragged, from one element to several tile rounds and long K), operand formats, value
scales, padded leading dimensions of codes, scales and output (scale rows that are not
4-byte aligned take the generic kernel), alpha, bias, bf16 / fp32 output, the SiLU
epilogue, and the tile plan (width as picked, 256 x 192 or 256 x 256 forced; K split on
or off).  Each case checks a random sample of outputs plus the corners and tile edges."""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_block_scaled_03_amd as mxq
from gpu_helpers import check_gemm, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CASES = 40


def padded_codes(c, pad):
    """The [L][Kp] codes stored with leading dimension Kp + pad (pad a multiple of 16)."""
    L, Kp = c.shape
    buf = torch.full((L, Kp + pad), 0xA5, dtype=torch.uint8, device=DEV)
    buf[:, :Kp].copy_(c)
    return buf[:, :Kp]


def padded_scales(s, pad, offset):
    """The [L][nb] scales stored with leading dimension nb + pad, `offset` bytes into a
    buffer filled with 0xFF (NaN scales) outside the view."""
    L, nb = s.shape
    ld = nb + pad
    buf = torch.full((L * ld + offset + 8,), 255, dtype=torch.uint8, device=DEV)
    view = buf[offset:offset + L * ld].view(L, ld)[:, :nb]
    view.copy_(s)
    return view


def plan(rng):
    width = str(rng.choice(["default", "192", "256"]))
    split = bool(rng.random() < 0.75)
    return width, split


@pytest.mark.parametrize("case", range(CASES))
def test_exact_gemm_random_sweep(monkeypatch, case):
    rng = np.random.default_rng(7000 + case)
    long_k = case % 3 == 0
    M = int(rng.integers(1, 1300))
    N = int(rng.integers(1, 1300))
    K = int(rng.integers(2000, 9000)) if long_k else int(rng.integers(1, 2100))
    fx, fw = (str(f) for f in rng.choice(["e4m3", "e5m2"], 2))
    out = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    act = "silu" if rng.random() < 0.3 else None
    bias = rng.random() < 0.6
    alpha = float(rng.choice([1.0, 0.5, -1.75]))
    xstd = float(10.0 ** rng.uniform(-3, 3))
    pad_x, pad_w = (16 * int(v) for v in rng.integers(0, 4, 2))
    nb = (K + 31) // 32
    if rng.random() < 0.8:      # 4-byte aligned scale rows: the main kernel and its plans
        pad_s, off_s = int((-nb) % 4 + 4 * rng.integers(0, 2)), 0
    else:                       # rows that are not: the generic kernel
        pad_s, off_s = int(rng.integers(0, 6)), int(rng.random() < 0.5)
    pad_y = int(rng.integers(0, 9))
    width, split = plan(rng)
    say("sweep %d: %dx%dx%d %sx%s %s act=%s bias=%s alpha=%g pads x%d w%d s%d+%d y%d width=%s split=%s"
        % (case, M, N, K, fx, fw, out, act, bias, alpha, pad_x, pad_w, pad_s, off_s, pad_y, width, split))

    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32) * np.float32(xstd)).to(DEV)
    w = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)).to(DEV)
    xc0, xs0 = mxq.quantize(x, fx, "row")
    wc0, ws0 = mxq.quantize(w, fw, "row")
    xc, wc = padded_codes(xc0, pad_x), padded_codes(wc0, pad_w)
    xs, ws = padded_scales(xs0, pad_s, off_s), padded_scales(ws0, pad_s, 0)
    b = torch.from_numpy(rng.standard_normal(N).astype(np.float32)).to(DEV) if bias else None

    if width != "default":
        monkeypatch.setenv("MXQ_EXACT_TILE_N", width)
    if not split:
        monkeypatch.setenv("MXQ_EXACT_KSPLIT", "0")
    ybuf = torch.full((M, N + pad_y), float("nan"), dtype=out, device=DEV)
    y = ybuf[:, :N]
    mxq.gemm(xc, xs, wc, ws, K, fx, fw, alpha=alpha, bias=b, out=y, accum="fp32", act=act)
    v = None
    if act is not None:
        v = mxq.gemm(xc, xs, wc, ws, K, fx, fw, alpha=alpha, bias=b, out_dtype=torch.float32, accum="fp32")
    torch.cuda.synchronize()

    n = 2500
    ei = np.unique(np.array([0, M - 1, min(255, M - 1), min(256, M - 1), M // 2]))
    ej = np.unique(np.array([0, N - 1, min(95, N - 1), min(96, N - 1), min(191, N - 1), min(192, N - 1),
                             min(255, N - 1), min(256, N - 1), N // 2]))
    ii = np.concatenate([rng.integers(0, M, n), np.repeat(ei, ej.size)])
    jj = np.concatenate([rng.integers(0, N, n), np.tile(ej, ei.size)])
    xc_h, xs_h, wc_h, ws_h = (t.cpu().numpy() for t in (xc, xs, wc, ws))
    y_ref, t = oracle.gemm_sampled(xc_h, xs_h, fx, wc_h, ws_h, fw, K, ii, jj, alpha=alpha,
                                   bias=None if b is None else b.cpu().numpy())
    yg = y.float().cpu().numpy()[ii, jj]
    assert torch.isnan(ybuf[:, N:].float()).all(), "sweep %d wrote past N" % case
    if act is None:
        check_gemm(yg, y_ref, t, out, bias or alpha != 1.0, "sweep %d" % case)
        return
    # SiLU: the pre-activation within the strict bound, and the activated output within one
    # rounding of the FP64 SiLU of that same pre-activation (+ the FP32 SiLU's few ulp)
    vg = v.cpu().numpy()[ii, jj]
    check_gemm(vg, y_ref, t, torch.float32, bias or alpha != 1.0, "sweep %d pre-activation" % case)
    s = oracle.silu(vg.astype(np.float64))
    rel = 2.0 ** -8 + 2.0 ** -20 if out == torch.bfloat16 else 2.0 ** -20
    assert np.all(np.abs(yg.astype(np.float64) - s) <= np.abs(s) * rel + 2.0 ** -126), "sweep %d SiLU" % case

"""Pins of the oracle's quantize / dequantize / block-scaled GEMM.

Sources: "Low-Precision GPU Programming" -- "Microscaling: the two-row experiment"
(two-row projection and spike selector, printed outputs), "Online scaling isn't
automatically fused into TMA" (block scales cannot be pulled out of the sum),
"Scale ownership and the GEMM dataflow" (per-row/per-column scaling factors out of a
single-block sum; block-K contraction keeps scales inside the sum over blocks).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import exact
from conftest import load_golden


def two_row_inputs():
    g = load_golden("two_row_projection.json")
    r = g["repeat"]
    x = np.array([g["pattern_small"] * r, g["pattern_large"] * r], dtype=np.float32)
    w_kn = np.array(g["weight_pattern"] * r, dtype=np.float32).reshape(32, 1)   # the page's K x N
    return g, x, w_kn


def test_two_row_projection(oracle_lib):
    g, x, w_kn = two_row_inputs()
    p = g["printed"]
    xc, xs = oracle.quantize(x, "e4m3", axis=0)
    wc, ws = oracle.quantize(w_kn, "e4m3", axis=1)      # 32x1 group down the column
    assert wc.shape == (1, 32) and ws.shape == (1, 1)
    assert [oracle.decode_e8m0(int(s)) for s in xs[:, 0]] == p["mxfp8_scales_x"]
    assert [hex(int(s)) for s in xs[:, 0]] == ["0x77", "0x80"]
    xh = oracle.dequantize(xc, xs, "e4m3", 32)
    assert "%.8f" % xh[0, 0] == "%.8f" % p["x00"]["mxfp8"]
    assert xh[1, 3] == p["x13"]["mxfp8"]
    y, t = oracle.gemm(xc, xs, "e4m3", wc, ws, "e4m3", 32)
    assert ["%.6f" % v for v in y[:, 0]] == ["%.6f" % v for v in p["mxfp8_y"]]
    assert y[1, 0] == 7.75
    # the unquantized projection of the fixture (pins the restated inputs); the page
    # printed an FP32 product, so compare at the printed precision plus FP32 rounding
    ref = (x.astype(np.float64) @ w_kn.astype(np.float64))[:, 0]
    assert np.all(np.abs(ref - np.array(p["reference_y"])) <= 5e-7 + 1e-7 * np.abs(ref))
    # codes are what the exact twin gives for each block
    for i in range(2):
        codes, sb = exact.quantize_block([Fraction(float(v)) for v in x[i]], "e4m3")
        assert list(xc[i]) == codes and xs[i, 0] == sb


def test_two_row_selector(oracle_lib):
    g, x, _ = two_row_inputs()
    sel = np.zeros((32, 1), dtype=np.float32)
    sel[3, 0] = 1.0
    xc, xs = oracle.quantize(x, "e4m3", axis=0)
    sc, ss = oracle.quantize(sel, "e4m3", axis=1)
    y, _ = oracle.gemm(xc, xs, "e4m3", sc, ss, "e4m3", 32)
    assert list(y[:, 0]) == g["selector"]["selected_mx"]
    assert abs(y[1, 0] - g["selector"]["selected_reference"][1]) == g["selector"]["spike_only_abs_error"]


def test_two_row_tensor_wide_codec_crosscheck(oracle_lib):
    """The page's per-tensor variant (FP32 scale amax/448, FP32 division) reproduced with
    the oracle's encoder: exercises the encoder on non-power-of-two scaled values."""
    g, x, w_kn = two_row_inputs()
    p = g["printed"]

    def roundtrip(v, s):
        q = (v / s).astype(np.float32)
        codes = np.array([oracle.encode(float(a), "e4m3") for a in q.ravel()])
        dec = np.array([oracle.decode(int(c), "e4m3") for c in codes], dtype=np.float32)
        return (dec.reshape(v.shape) * s).astype(np.float32)

    sx = np.float32(np.abs(x).max() / np.float32(448.0))
    sw = np.float32(np.abs(w_kn).max() / np.float32(448.0))
    assert "%.6f" % sx == "%.6f" % p["tensor_scale_x"]
    xt, wt = roundtrip(x, sx), roundtrip(w_kn, sw)
    assert xt[0, 0] == p["x00"]["tensor_fp8"] and xt[1, 3] == p["x13"]["tensor_fp8"]
    yt = (xt @ wt)[:, 0]
    assert ["%.6f" % v for v in yt] == ["%.6f" % v for v in p["tensor_fp8_y"]]


def test_block_scales_stay_inside_the_sum(oracle_lib):
    """The pages' arithmetic: partials 2, 3 under scale products 5, 8 give 34, and
    pulling one scale out gives 25.  5 is not a power of two, so the same point is
    made with E8M0-representable products 4 and 8: 2*4 + 3*8 = 32, not 4*(2+3) = 20."""
    g = load_golden("stale_scale.json")
    pa, sp = g["partials"], g["scale_products"]
    assert sum(a * b for a, b in zip(pa, sp)) == g["printed"]["block_scale_sum"]
    assert sp[0] * sum(pa) == g["printed"]["pulled_out_sum"]
    K = 64
    xc = np.zeros((1, K), np.uint8)
    wc = np.zeros((1, K), np.uint8)
    xc[0, 0] = oracle.encode(2.0, "e4m3")
    xc[0, 32] = oracle.encode(3.0, "e4m3")
    wc[0, 0] = wc[0, 32] = oracle.encode(1.0, "e4m3")
    xs = np.array([[127 + 2, 127 + 3]], np.uint8)      # 4, 8
    ws = np.array([[127, 127]], np.uint8)
    y, t = oracle.gemm(xc, xs, "e4m3", wc, ws, "e4m3", K)
    assert y[0, 0] == 32.0 and y[0, 0] != 4.0 * (2.0 + 3.0)
    assert t[0, 0] == 32.0


def rand_codes(rng, shape, fmt):
    n = oracle.num_finite_codes(fmt)
    mags = rng.integers(0, n, size=shape)
    sign = rng.integers(0, 2, size=shape) * 0x80
    return (mags | sign).astype(np.uint8)


def decoded(codes, fmt):
    table = np.array([oracle.decode(c, fmt) for c in range(256)])
    return table[codes]


@pytest.mark.parametrize("fmts", [("e4m3", "e4m3"), ("e5m2", "e4m3")])
def test_single_block_reduces_to_epilogue_scaling(oracle_lib, fmts):
    """K = 32: one block, so Y = S_X[i] * S_W[j] * (Xq Wq^T) -- the per-row/per-column
    factoring of the two-phase kernel."""
    fx, fw = fmts
    rng = np.random.default_rng(1)
    M, N, K = 7, 5, 32
    xc, wc = rand_codes(rng, (M, K), fx), rand_codes(rng, (N, K), fw)
    xs = rng.integers(120, 135, size=(M, 1)).astype(np.uint8)
    ws = rng.integers(120, 135, size=(N, 1)).astype(np.uint8)
    y, _ = oracle.gemm(xc, xs, fx, wc, ws, fw, K)
    core = decoded(xc, fx) @ decoded(wc, fw).T
    ref = np.exp2(xs.astype(np.float64) - 127) * core * np.exp2(ws.astype(np.float64).T - 127)
    assert np.array_equal(y, ref)


def test_unit_scales_reduce_to_plain_matmul(oracle_lib):
    rng = np.random.default_rng(2)
    M, N, K = 9, 6, 96
    xc, wc = rand_codes(rng, (M, K), "e4m3"), rand_codes(rng, (N, K), "e4m3")
    xs = np.full((M, 3), 127, np.uint8)
    ws = np.full((N, 3), 127, np.uint8)
    y, _ = oracle.gemm(xc, xs, "e4m3", wc, ws, "e4m3", K)
    assert np.array_equal(y, decoded(xc, "e4m3") @ decoded(wc, "e4m3").T)


@pytest.mark.parametrize("K", [1, 31, 32, 33, 64, 96])
def test_tiny_shapes_exact_brute_force(oracle_lib, K):
    """Oracle GEMM vs exact rational evaluation of the block sum, and the block sum ==
    (dequantized X)(dequantized W)^T exactly; the oracle's FP64 error stays within
    K * 2^-53 * T."""
    rng = np.random.default_rng(100 + K)
    nb = (K + 31) // 32
    for fx, fw in [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]:
        M, N = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        xc = rand_codes(rng, (M, 32 * nb), fx)
        wc = rand_codes(rng, (N, 32 * nb), fw)
        xs = rng.integers(100, 150, size=(M, nb)).astype(np.uint8)
        ws = rng.integers(100, 150, size=(N, nb)).astype(np.uint8)
        alpha = 0.75
        bias = rng.standard_normal(N).astype(np.float32)
        y, t = oracle.gemm(xc, xs, fx, wc, ws, fw, K, alpha=alpha, bias=bias)
        Y = exact.block_gemm(xc.tolist(), xs.tolist(), fx, wc.tolist(), ws.tolist(), fw, K,
                             alpha=Fraction(alpha), bias=[Fraction(float(b)) for b in bias])
        D = exact.dequant_then_matmul(xc.tolist(), xs.tolist(), fx, wc.tolist(), ws.tolist(), fw, K)
        for i in range(M):
            for j in range(N):
                assert Y[i][j] == Fraction(alpha) * D[i][j] + Fraction(float(bias[j]))
                err = abs(Fraction(float(y[i, j])) - Y[i][j])
                assert err <= Fraction(K + 2) * Fraction(2) ** -53 * (Fraction(float(t[i, j])) + abs(Y[i][j]))


def test_sampled_equals_full(oracle_lib):
    rng = np.random.default_rng(3)
    M, N, K = 13, 11, 70
    nb = 3
    xc, wc = rand_codes(rng, (M, 96), "e4m3"), rand_codes(rng, (N, 96), "e5m2")
    xs = rng.integers(110, 140, size=(M, nb)).astype(np.uint8)
    ws = rng.integers(110, 140, size=(N, nb)).astype(np.uint8)
    bias = rng.standard_normal(N).astype(np.float32)
    y, t = oracle.gemm(xc, xs, "e4m3", wc, ws, "e5m2", K, alpha=2.0, bias=bias)
    ii = rng.integers(0, M, 50)
    jj = rng.integers(0, N, 50)
    ys, ts = oracle.gemm_sampled(xc, xs, "e4m3", wc, ws, "e5m2", K, ii, jj, alpha=2.0, bias=bias)
    assert np.array_equal(ys, y[ii, jj]) and np.array_equal(ts, t[ii, jj])


# ----------------------------------------------------------------- quantize

@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("K", [1, 5, 32, 33, 70, 96])
def test_quantize_rows_vs_twin(oracle_lib, fmt, K):
    rng = np.random.default_rng(K)
    rows = 6
    x = (rng.standard_normal((rows, K)) * np.exp2(rng.integers(-30, 30, (rows, 1)))).astype(np.float32)
    x[0, :] = 0.0                                   # zero row -> scale byte 127
    x[1, 0] = -0.0
    if K > 3:
        x[2, 3] = 1e-30                             # far below the block's subnormal floor
        x[3, 1] = -1e-30                            # negative underflow -> signed zero
    xc, xs = oracle.quantize(x, fmt, axis=0)
    Kp = 32 * ((K + 31) // 32)
    assert xc.shape == (rows, Kp) and xs.shape == (rows, Kp // 32)
    for r in range(rows):
        for b in range(Kp // 32):
            vals = x[r, 32 * b:min(32 * b + 32, K)]
            codes, sb = exact.quantize_block([Fraction(float(v)) for v in vals], fmt,
                                             negzero=[math.copysign(1, v) < 0 for v in vals])
            assert xs[r, b] == sb
            assert list(xc[r, 32 * b:32 * b + 32]) == codes
    assert xs[0, 0] == 127 and np.all(xc[0] == 0)
    if K > 3:
        assert xc[3, 1] == 0x80


def test_quantize_bf16_input_matches_f32_input(oracle_lib):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    as_f32 = xb.float().numpy()
    a = oracle.quantize(bits, "e4m3")
    b = oracle.quantize(as_f32, "e4m3")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_colwise_is_rowwise_of_transpose(oracle_lib):
    rng = np.random.default_rng(6)
    w = rng.standard_normal((70, 9)).astype(np.float32) * 0.02
    c1, s1 = oracle.quantize(w, "e4m3", axis=1)
    c2, s2 = oracle.quantize(np.ascontiguousarray(w.T), "e4m3", axis=0)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_colwise_differs_from_transposed_bytes(oracle_lib):
    """Regrouping (rowwise 1x32 vs columnwise 32x1) changes scale membership: the
    columnwise codes are not the rowwise codes transposed."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((32, 32)).astype(np.float32) * np.exp2(np.arange(32, dtype=np.float32))[:, None]
    cr, _ = oracle.quantize(x, "e4m3", axis=0)
    cc, _ = oracle.quantize(x, "e4m3", axis=1)
    assert not np.array_equal(cc, cr.T)


def test_nonfinite_block_reading(oracle_lib):
    """Reading where the pages are silent: a block holding NaN/Inf gets scale byte 255
    (E8M0 NaN) and every code 0x7F; other blocks of the row are unaffected."""
    x = np.ones((2, 64), np.float32)
    x[0, 5] = np.nan
    x[1, 40] = -np.inf
    xc, xs = oracle.quantize(x, "e4m3")
    assert xs[0, 0] == 255 and np.all(xc[0, :32] == 0x7F)
    assert xs[0, 1] == 127 - 8 and xs[1, 0] == 127 - 8
    assert xs[1, 1] == 255 and np.all(xc[1, 32:] == 0x7F)


# ----------------------------------------------------------------- dequantize

@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_dequantize_exact_and_bf16(oracle_lib, fmt):
    rng = np.random.default_rng(8)
    L, K = 5, 70
    codes = rand_codes(rng, (L, 96), fmt)
    scales = rng.integers(0, 255, size=(L, 3)).astype(np.uint8)
    f32 = oracle.dequantize(codes, scales, fmt, K, "f32")
    b16 = oracle.dequantize(codes, scales, fmt, K, "bf16")
    for l in range(L):
        for k in range(K):
            v = Fraction(0)
            dv = exact.decode(int(codes[l, k]), fmt)
            v = dv * exact.e8m0_exact(int(scales[l, k // 32]))
            if v >= Fraction(2) ** 128 or v <= -Fraction(2) ** 128:
                assert math.isinf(f32[l, k])
            else:
                assert Fraction(float(f32[l, k])) == v
    # bf16 of an exactly-representable fp32 value is torch's fp32 -> bf16 RNE
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16, ref)
    # scale byte 255 reconstructs as NaN
    s2 = scales.copy()
    s2[0, 0] = 255
    assert np.all(np.isnan(oracle.dequantize(codes, s2, fmt, K, "f32")[0, :32]))

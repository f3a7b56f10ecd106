"""Pins of the oracle's second scale rule: the OCP Microscaling (MX) specification's, which
"Low-Precision GPU Programming", "Microscaling: the two-row experiment" names as the other
scale-selection algorithm (the page prints results only for its own rule, amax/448 rounded
up to a power of two).  The OCP rule: shared exponent = floor(log2(amax)) minus the exponent
of the element format's largest normal (E4M3 8, E5M2 15), elements RNE, clamped to the
largest normal.  Readings shared with the page's rule: exponent clamped at -127, zero block
S = 1, non-finite block byte 255.

Independent checks: the exact-rational twin (powers-of-two comparisons, brute-force nearest
code), the relation to the page's rule (pinned elsewhere against the page's printed scales),
and the two-row fixture's consequences derived by hand below."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact
from conftest import load_golden

FMTS = ["e4m3", "e5m2"]
EMAX = {"e4m3": 8, "e5m2": 15}
FMAX = {"e4m3": 448.0, "e5m2": 57344.0}


def all_positive_finite_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)          # +0 excluded, up to the largest finite
    return (bits << 16).view(np.float32)


def test_largest_normal_exponents_from_the_codes():
    # 448 = 1.75 * 2^8 and 57,344 = 1.75 * 2^15 ("Format taxonomy")
    assert exact.largest_normal_exponent("e4m3") == 8
    assert exact.largest_normal_exponent("e5m2") == 15


@pytest.mark.parametrize("fmt", FMTS)
def test_ocp_scale_rule_exhaustive_bf16(oracle_lib, fmt):
    """Every positive finite bf16 amax: the C oracle's byte equals the exact twin's; away
    from the -127 clamp, amax / S lies in [2^emax, 2^(emax+1)) (the block maximum keeps the
    largest normal's exponent); and against the page's rule (already pinned to the printed
    scales) the OCP exponent is one lower exactly when amax's significand exceeds 1.75, else
    equal."""
    vals = all_positive_finite_bf16()
    for v in vals[::7].tolist() + [float(vals[0]), float(vals[-1]), 1.0, 500.0, 448.0, 1.75, 1.7578125]:
        b = oracle.scale_byte_ocp(v, fmt)
        assert b == exact.scale_exponent_ocp(Fraction(v), fmt) + 127, v
    for v in vals.tolist():
        b_ocp = oracle.scale_byte_ocp(v, fmt)
        b_ceil = oracle.scale_byte(v, fmt)
        m, E = math.frexp(v)                    # v = m * 2^E, m in [0.5, 1)
        significand = 2.0 * m                   # in [1, 2)
        if b_ocp > 0:                           # not clamped
            q = v / 2.0 ** (b_ocp - 127)
            assert 2.0 ** EMAX[fmt] <= q < 2.0 ** (EMAX[fmt] + 1), (v, b_ocp)
            assert b_ceil - b_ocp == (1 if significand > 1.75 else 0), (v, b_ocp, b_ceil)
        else:
            assert b_ceil <= 1


def test_ocp_zero_and_nonfinite_blocks(oracle_lib):
    for fmt in FMTS:
        assert oracle.scale_byte_ocp(0.0, fmt) == 127
        assert oracle.scale_byte_ocp(math.inf, fmt) == 255
        assert oracle.scale_byte_ocp(math.nan, fmt) == 255
        assert oracle.scale_byte_ocp(2.0 ** -149, fmt) == 0        # clamped at 2^-127


def two_row_x():
    g = load_golden("two_row_projection.json")
    x = np.array([g["pattern_small"] * 4, g["pattern_large"] * 4], dtype=np.float32)
    w = np.array(g["weight_pattern"] * 4, dtype=np.float32).reshape(32, 1)
    return g, x, w


def test_ocp_rule_on_the_two_row_fixture(oracle_lib):
    """The page's two-row X under the OCP rule, derived by hand from the rule:
    row 0 (amax 1.0): floor(log2 1) - 8 = -8 -> S = 2^-8, the page's printed scale, so its
    codes and y[0] are unchanged (0.601562 printed);
    row 1 (amax 500): floor(log2 500) - 8 = 0 -> S = 1 (the page's rule gives 2): 500
    saturates to 448 (printed reconstruction under the page's rule: 512), -250 rounds to
    -256 as under the page's rule, the other values are exact;
    y[1] = 7.75 + 4 * (448 - 512) * (-0.0625) = 23.75."""
    g, x, w = two_row_x()
    xc, xs = oracle.quantize(x, "e4m3", rule="ocp")
    wc, ws = oracle.quantize(w, "e4m3", axis=1, rule="ocp")
    assert xs[:, 0].tolist() == [127 - 8, 127]
    assert [oracle.decode_e8m0(int(b)) for b in xs[:, 0]] == [g["printed"]["mxfp8_scales_x"][0], 1.0]
    xhat = oracle.dequantize(xc, xs, "e4m3", 32)
    assert xhat[1, 3] == 448.0
    assert "%.8f" % xhat[0, 0] == "%.8f" % g["printed"]["x00"]["mxfp8"]
    assert xhat[1, 7] == -256.0
    cc, cs = oracle.quantize(x, "e4m3")                    # the page's rule
    assert np.array_equal(xc[0], cc[0]) and not np.array_equal(xc[1], cc[1])
    y, _ = oracle.gemm(xc, xs, "e4m3", wc, ws, "e4m3", 32)
    assert "%.6f" % y[0, 0] == "%.6f" % g["printed"]["mxfp8_y"][0]
    assert y[1, 0] == 23.75
    # the one-hot selector column: [0.5, 448], absolute error 52 (12 under the page's rule)
    sel = np.zeros((32, 1), dtype=np.float32)
    sel[3, 0] = 1.0
    sc, ss = oracle.quantize(sel, "e4m3", axis=1, rule="ocp")
    ysel, _ = oracle.gemm(xc, xs, "e4m3", sc, ss, "e4m3", 32)
    assert ysel[:, 0].tolist() == [0.5, 448.0]
    assert abs(ysel[1, 0] - g["selector"]["selected_reference"][1]) == 52.0


@pytest.mark.parametrize("fmt", FMTS)
def test_ocp_quantize_blocks_vs_twin(oracle_lib, fmt):
    """Random blocks (ragged K, signed zeros, values whose block maximum saturates): codes
    and scale bytes equal the exact twin's RNE-satfinite quantization under the OCP rule."""
    rng = np.random.default_rng(61)
    K = 77
    x = (rng.standard_normal((24, K)) * np.exp2(rng.integers(-20, 20, (24, 1)))).astype(np.float32)
    x[3, :8] = -0.0
    x[4, 5] = 1.98 * 2.0 ** 10             # significand 1.98 > 1.75: the block maximum saturates
    x[5, 40] = -1.76 * 2.0 ** -3
    codes, scales = oracle.quantize(x, fmt, rule="ocp")
    saturated = 0
    for r in range(x.shape[0]):
        for b in range((K + 31) // 32):
            vals = [Fraction(float(v)) for v in x[r, 32 * b:min(32 * b + 32, K)]]
            nz = [math.copysign(1.0, float(v)) < 0 and float(v) == 0.0 for v in x[r, 32 * b:min(32 * b + 32, K)]]
            tc, ts = exact.quantize_block(vals, fmt, negzero=nz, rule="ocp")
            assert ts == scales[r, b], (r, b)
            assert list(codes[r, 32 * b:32 * b + 32]) == tc, (r, b)
            saturated += sum(1 for c in tc if c & 0x7F == {"e4m3": 0x7E, "e5m2": 0x7B}[fmt])
    assert saturated > 0


def test_ocp_planted_mistake_fails_a_pin(oracle_lib):
    """A plausible slip -- ceil instead of floor, i.e. the page's rule -- fails the two-row pin."""
    g, x, _ = two_row_x()
    b = oracle.scale_byte(500.0, "e4m3")      # the page's rule
    assert b != oracle.scale_byte_ocp(500.0, "e4m3")
    xhat_wrong = float(oracle.decode(oracle.encode(500.0 / 2.0 ** (b - 127), "e4m3"), "e4m3")) * 2.0 ** (b - 127)
    assert xhat_wrong != 448.0

"""Pins of the oracle's quantize with caller-owned (delayed / stale) scale bytes and its
per-block diagnostics ("Worked failure: stale delayed scale"; "Delayed scaling in
Transformer Engine": the pass also records the current amax)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact
from conftest import load_golden


def test_stale_scale_e8m0_analogue_of_the_pages_example():
    # the pages: a scale from old amax 10 meets a spike of 500; saturation to 448 leaves a
    # finite, positive, badly wrong value.  Their S = 10/448 is not an E8M0 value; the MX
    # rule's scale for amax 10 is 2^-5 (byte 122): 10 -> code 320 exactly, 500 -> 16000 ->
    # clipped to 448 -> reconstructed 14 (97.2 % error).
    g = load_golden("stale_scale.json")
    sb = oracle.scale_byte(g["old_amax"], "e4m3")
    assert sb == 122
    x = np.array([[g["old_amax"]] + [1.0] * 30 + [g["spike"]]], dtype=np.float32)
    codes, amax, clipped, flushed = oracle.quantize_scaled(x, "e4m3", np.array([[sb]], dtype=np.uint8))
    rec = oracle.dequantize(codes, np.array([[sb]], dtype=np.uint8), "e4m3", 32)[0]
    assert rec[0] == g["old_amax"]
    assert rec[31] == g["fp8_limit"] * 2.0 ** -5 == 14.0
    assert np.isfinite(rec).all() and rec[31] > 0
    assert abs(100 * (g["spike"] - rec[31]) / g["spike"] - 97.2) < 1e-9
    assert clipped[0, 0] == 1 and flushed[0, 0] == 0
    assert amax[0, 0] == g["spike"]          # the amax recorded for the next scale update


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_rule_scales_reproduce_quantize(fmt):
    rng = np.random.default_rng(60)
    x = (rng.standard_normal((40, 200)) * np.exp2(rng.integers(-30, 30, (40, 1)))).astype(np.float32)
    c0, s0 = oracle.quantize(x, fmt)
    c1, amax, clipped, flushed = oracle.quantize_scaled(x, fmt, s0)
    assert np.array_equal(c0, c1)
    assert not clipped.any()
    want = np.array([[np.max(np.abs(x[r, 32 * b:32 * b + 32])) for b in range(s0.shape[1])] for r in range(40)],
                    dtype=np.float32)
    assert np.array_equal(amax, want)
    # flushed counts what RNE sent to zero: nonzero x with a zero-magnitude code
    xp = np.zeros((40, c0.shape[1]), dtype=np.float32)
    xp[:, :200] = x
    fl = ((xp != 0) & ((c0 & 0x7F) == 0)).reshape(40, -1, 32).sum(axis=2)
    assert np.array_equal(flushed, fl)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_matches_exact_twin_with_clipping_and_flushing(fmt):
    """Scale bytes far from the rule's: the codes equal the exact twin's RNE-satfinite of
    the rational x / S, the counts equal the exact counts."""
    rng = np.random.default_rng(61)
    fmax = Fraction(exact.FORMATS[fmt][3])
    x = (rng.standard_normal((12, 64)) * 2.0 ** rng.integers(-8, 8, (12, 64))).astype(np.float32)
    x[0, 3] = 0.0
    x[1, 5] = -0.0
    given = rng.integers(100, 150, (12, 2)).astype(np.uint8)
    codes, amax, clipped, flushed = oracle.quantize_scaled(x, fmt, given)
    assert clipped.sum() > 0 and flushed.sum() > 0
    for r in range(12):
        for b in range(2):
            S = Fraction(2) ** (int(given[r, b]) - 127)
            nclip = nflush = 0
            for k in range(32 * b, 32 * b + 32):
                v = float(x[r, k])
                q = Fraction(v) / S
                want = exact.encode(q, fmt, negative_zero=np.signbit(x[r, k]))
                assert codes[r, k] == want, (r, k, v, int(given[r, b]))
                nclip += abs(q) > fmax
                nflush += v != 0 and (want & 0x7F) == 0
            assert clipped[r, b] == nclip and flushed[r, b] == nflush


def test_special_values_and_nan_scale():
    x = np.ones((3, 32), dtype=np.float32)
    x[0, 1] = np.nan
    x[0, 2] = np.inf
    x[0, 3] = -np.inf
    given = np.array([[127], [255], [127]], dtype=np.uint8)
    codes, amax, clipped, flushed = oracle.quantize_scaled(x, "e4m3", given)
    assert codes[0, 1] == 0x7F and codes[0, 2] == 0x7E and codes[0, 3] == 0xFE
    assert clipped[0, 0] == 2 and np.isnan(amax[0, 0])
    assert np.all(codes[1] == 0x7F) and clipped[1, 0] == 0
    assert np.all(codes[2] == 0x38) and amax[2, 0] == 1.0


def test_colwise_is_rowwise_of_transpose():
    rng = np.random.default_rng(62)
    x = rng.standard_normal((70, 40)).astype(np.float32)
    given = rng.integers(118, 130, (40, 3)).astype(np.uint8)
    a = oracle.quantize_scaled(x, "e5m2", given, axis=1)
    b = oracle.quantize_scaled(np.ascontiguousarray(x.T), "e5m2", given)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)

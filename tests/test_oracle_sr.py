"""Pins of the oracle's stochastic rounding ("Low-Precision GPU Programming", "Rounding: RNE
versus stochastic rounding": round up with probability (x - l) / (u - l) between the
neighbouring representable values l < x < u, so E[SR(x)] = x, representable values stay)
and of its random-number generator (Philox4x32-10, Salmon et al., SC 2011)."""
import math

import numpy as np
import pytest

import oracle
from oracle import exact


def test_philox_known_answers():
    # known-answer vectors published with the Random123 reference implementation of
    # Philox4x32-10 (counter, key -> output)
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        assert oracle.philox4x32_10(ctr, key) == want


def sr_codes(value, n, fmt="e4m3", seed=1):
    x = np.full((n // 32, 32), value, dtype=np.float32)
    codes, scales = oracle.quantize_sr(x, fmt, seed)
    return codes.ravel(), int(scales[0, 0])


def test_pages_example_upper_probability():
    # the pages' example: x = 1.01 between E4M3 neighbours 1 and 9/8, P(up) = 2/25.  The
    # block scale 2^-8 maps it to 258.56 between 256 (0x78) and 288 (0x79): the same p.
    n = 1 << 18
    codes, sb = sr_codes(1.01, n)
    assert sb == 127 - 8
    assert set(np.unique(codes)) == {0x78, 0x79}
    p = 2 / 25
    up = int(np.sum(codes == 0x79))
    assert abs(up - p * n) < 5 * math.sqrt(n * p * (1 - p))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_unbiased(fmt):
    # E[SR(x)] = x: the mean of the decoded codes of n copies of x approaches x
    rng = np.random.default_rng(5)
    for v in rng.uniform(0.3, 0.9, 6).astype(np.float32):
        n = 1 << 16
        codes, sb = sr_codes(v, n, fmt, seed=int(rng.integers(1 << 62)))
        dec = np.array([float(exact.decode(int(c), fmt)) for c in np.unique(codes)], dtype=np.float64)
        vals = dict(zip(np.unique(codes), dec))
        mean = np.mean([vals[c] for c in codes]) * 2.0 ** (sb - 127)
        lo, hi = sorted(vals.values())
        spread = (hi - lo) * 2.0 ** (sb - 127)
        assert abs(mean - float(v)) < 5 * spread * 0.5 / math.sqrt(n)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_only_neighbours_and_representables_fixed(fmt):
    mags = [float(v) for _, v in exact.finite_magnitudes(fmt)]
    rng = np.random.default_rng(6)
    # representable values stay put whatever the random number
    for m in mags:
        for r in (0, (1 << 24) - 1, 12345):
            c = oracle.encode_sr(m, fmt, r)
            assert float(exact.decode(c, fmt)) == m
    # any other value goes to one of its two neighbours; r = 0 always rounds up,
    # r = 2^24 - 1 rounds down unless p > 1 - 2^-24
    for _ in range(2000):
        i = int(rng.integers(0, len(mags) - 1))
        lo, hi = mags[i], mags[i + 1]
        x = lo + (hi - lo) * float(rng.uniform(0.001, 0.999))
        got = float(exact.decode(oracle.encode_sr(x, fmt, int(rng.integers(1 << 24))), fmt))
        assert got in (lo, hi)
        assert float(exact.decode(oracle.encode_sr(x, fmt, 0), fmt)) == hi
        assert float(exact.decode(oracle.encode_sr(x, fmt, (1 << 24) - 1), fmt)) == lo
        assert float(exact.decode(oracle.encode_sr(-x, fmt, 0), fmt)) == -hi


def test_scales_and_rne_agreement():
    # the scale bytes are the RNE quantizer's; codes differ from RNE's only by one step
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    c_sr, s_sr = oracle.quantize_sr(x, "e4m3", 99)
    c_rn, s_rn = oracle.quantize(x, "e4m3")
    assert np.array_equal(s_sr, s_rn)
    d = np.abs((c_sr & 0x7F).astype(int) - (c_rn & 0x7F).astype(int))
    assert d.max() <= 1 and np.array_equal(c_sr & 0x80, c_rn & 0x80)
    # colwise draws its random numbers by its own line index: colwise(x) == rowwise(x^T)
    cc, sc = oracle.quantize_sr(x, "e4m3", 99, axis=1)
    ct, st = oracle.quantize_sr(np.ascontiguousarray(x.T), "e4m3", 99)
    assert np.array_equal(cc, ct) and np.array_equal(sc, st)


def test_pins_reject_inverted_decision():
    """A planted mistake -- the comparison inverted, so the upper neighbour is taken with
    probability 1 - p -- fails the pages' example."""
    n = 1 << 16
    codes, _ = sr_codes(1.01, n)
    inverted = np.where(codes == 0x79, 0x78, 0x79)
    p = 2 / 25
    up = int(np.sum(inverted == 0x79))
    assert not abs(up - p * n) < 5 * math.sqrt(n * p * (1 - p))

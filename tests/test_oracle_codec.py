"""Pins of the oracle's FP8 / E8M0 codec and scale rule against what the pages fix.

Sources: "Low-Precision GPU Programming" -- "Format taxonomy", "Numerical hazards"
(subnormals, saturation), "Hands-on: auditing FP8 conversion boundaries",
"Microscaling: the two-row experiment" (E8M0 and the conservative scale rule).
Independent checks used: printed values (tests/golden), torch's own FP8 dtypes
(a library encoder/decoder, the method the audit section itself uses), and the
exact-rational twin ``oracle.exact`` (brute-force nearest code).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import exact
from conftest import load_golden

FMTS = ["e4m3", "e5m2"]
TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FMAX = {"e4m3": 448.0, "e5m2": 57344.0}


def all_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32)
    return (bits << 16).view(np.float32)


# ----------------------------------------------------------------- format facts

def test_e4m3_format_facts(oracle_lib):
    g = load_golden("format_facts.json")["e4m3"]
    dec = [oracle.decode(c, "e4m3") for c in range(256)]
    finite = [v for v in dec if not math.isnan(v)]
    assert max(finite) == g["max"] == oracle.decode(0x7E, "e4m3")
    assert [c for c in range(256) if math.isnan(dec[c])] == [0x7F, 0xFF]
    assert not any(math.isinf(v) for v in dec)                   # no infinities
    assert oracle.decode(0x08, "e4m3") == g["min_normal"] == 2.0 ** -6
    assert min(v for v in finite if v > 0) == 2.0 ** g["min_subnormal_log2"]
    in_12 = sorted(v for v in finite if 1.0 <= v < 2.0)
    assert np.all(np.diff(in_12) == g["spacing_1_2"]) and len(in_12) == 8
    top = sorted(v for v in finite if 256.0 <= v <= 448.0)
    assert np.all(np.diff(top) == g["spacing_256_448"]) and top[-1] == 448.0
    assert oracle.num_finite_codes("e4m3") == 127


def test_e5m2_format_facts(oracle_lib):
    g = load_golden("format_facts.json")["e5m2"]
    dec = [oracle.decode(c, "e5m2") for c in range(256)]
    finite = [v for v in dec if math.isfinite(v)]
    assert max(finite) == g["max"]
    assert min(v for v in finite if v > 0) == 2.0 ** g["min_subnormal_log2"]
    in_12 = sorted(v for v in finite if 1.0 <= v < 2.0)
    assert np.all(np.diff(in_12) == g["spacing_1_2"])
    assert oracle.encode(1e-7, "e5m2") == 0x00                    # below the floor
    assert math.isinf(dec[0x7C]) and math.isinf(dec[0xFC])
    assert oracle.num_finite_codes("e5m2") == 124


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_all_codes_matches_torch_and_twin(oracle_lib, fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()
    for c in range(256):
        v = oracle.decode(c, fmt)
        tw = exact.decode(c, fmt)
        if math.isnan(ref[c]):
            assert math.isnan(v) and tw == "nan"
        elif math.isinf(ref[c]):
            assert v == ref[c] and tw in ("+inf", "-inf")
        else:
            assert v == ref[c] and Fraction(v) == tw
            assert math.copysign(1.0, v) == math.copysign(1.0, ref[c])  # signed zero


# ----------------------------------------------------------------- audit casts

def test_audit_cast_values(oracle_lib):
    g = load_golden("audit_casts.json")
    d = 2.0 ** g["d_log2"]
    assert oracle.decode(oracle.encode(0.5 * d, "e4m3"), "e4m3") == 0.0
    assert oracle.encode(0.5 * d, "e4m3") == 0x00                 # tie -> even (zero)
    assert oracle.decode(oracle.encode(0.75 * d, "e4m3"), "e4m3") == d
    neg = oracle.encode(-0.5 * d, "e4m3")
    assert neg == 0x80 and math.copysign(1.0, oracle.decode(neg, "e4m3")) == -1.0
    assert oracle.decode(oracle.encode(1.0625, "e4m3"), "e4m3") == 1.0
    assert oracle.decode(oracle.encode(1.1875, "e4m3"), "e4m3") == 1.25
    for v, out in g["saturation_cliffs"]["e4m3"].items():
        assert oracle.decode(oracle.encode(float(v), "e4m3"), "e4m3") == out
        assert oracle.encode(-float(v), "e4m3") == 0xFE
    assert oracle.decode(oracle.encode(1e9, "e5m2"), "e5m2") == g["saturation_cliffs"]["e5m2_max"]
    # OCP reading of the bytes; the FNUZ reading of the same bytes must differ
    assert oracle.decode(0x38, "e4m3") == g["ocp_e4m3_bytes"]["0x38"]
    z = oracle.decode(0x80, "e4m3")
    assert z == 0.0 and math.copysign(1.0, z) == -1.0
    fnuz = torch.tensor([0x38, 0x80], dtype=torch.uint8).view(torch.float8_e4m3fnuz).float()
    assert fnuz[0].item() == g["fnuz_e4m3_bytes_same_codes"]["0x38"] and math.isnan(fnuz[1].item())
    assert oracle.decode(0x38, "e4m3") != fnuz[0].item()


# ----------------------------------------------------------------- exhaustive encode

@pytest.mark.parametrize("fmt", FMTS)
def test_encode_exhaustive_bf16_three_ways(oracle_lib, fmt):
    """Every bf16 value: C oracle == exact twin (brute force) == torch clamp-then-cast."""
    f = all_bf16_as_f32()
    fin = np.isfinite(f)
    ours = np.array([oracle.encode(float(v), fmt) for v in f], dtype=np.uint8)
    th = torch.from_numpy(f.copy()).clamp(-FMAX[fmt], FMAX[fmt]).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(ours[fin], th[fin])
    bits = np.arange(65536, dtype=np.uint32)
    for b in np.nonzero(fin)[0]:
        u = int(bits[b])
        neg = bool(u & 0x8000)
        E = (u >> 7) & 0xFF
        m = u & 0x7F
        if E == 0:
            num, dl = m, 133                      # m * 2^-133
        else:
            num, dl = (128 + m), 134 - E          # (1 + m/128) * 2^(E-127)
        if dl < 0:
            num, dl = num << (-dl), 0
        tw = exact.encode_int(num, dl, fmt, neg)
        assert tw == ours[b], (hex(u), hex(tw), hex(ours[b]))


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_midpoints_and_neighbours(oracle_lib, fmt):
    """Exact midpoints between adjacent codes tie to the even code; one fp64 ulp either
    side goes to the nearer code (covers the subnormal/normal seam)."""
    n = oracle.num_finite_codes(fmt)
    for c in range(n - 1):
        lo, hi = oracle.decode(c, fmt), oracle.decode(c + 1, fmt)
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.encode(mid, fmt) == even
        assert oracle.encode(np.nextafter(mid, -np.inf), fmt) == c
        assert oracle.encode(np.nextafter(mid, np.inf), fmt) == c + 1
        assert oracle.encode(-mid, fmt) == 0x80 | even
        tw = exact.encode(Fraction(mid), fmt)
        assert tw == even


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_random_fp32_vs_twin(oracle_lib, fmt):
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000))).astype(np.float32)
    for x in v:
        assert oracle.encode(float(x), fmt) == exact.encode(Fraction(float(x)), fmt)


# ----------------------------------------------------------------- E8M0 and the scale rule

def test_e8m0_pins(oracle_lib):
    g = load_golden("e8m0.json")
    assert oracle.decode_e8m0(0x77) == 2.0 ** -8 == exact.decode_e8m0(0x77)
    assert oracle.decode_e8m0(0x80) == 2.0 == exact.decode_e8m0(0x80)
    assert oracle.decode_e8m0(0) > 0 and exact.decode_e8m0(0) > 0
    assert math.isnan(oracle.decode_e8m0(255)) and math.isnan(exact.decode_e8m0(255))
    for bad in (-1, 256, 1.0, "x", True, None):
        with pytest.raises(ValueError):
            exact.decode_e8m0(bad)
    assert [hex(c) for c in (-8 + 127, 1 + 127)] == g["printed_scale_bytes"]
    # packed payload of the two-row X: 2 rows x 32 one-byte codes plus the scales
    assert 64 + 4 == g["packed_x_payload_bytes"]["tensor"]   # one fp32 tensor scale
    assert 64 + 2 == g["packed_x_payload_bytes"]["mx"]       # two E8M0 bytes
    b = g["bits_per_element"]
    assert (b["block_elems"] * b["elem_bits"] + b["scale_bits"]) / b["block_elems"] == 8.25


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_rule_exhaustive_bf16(oracle_lib, fmt):
    """For every positive finite bf16 amax: the oracle's search == the exact twin ==
    the pages' formula max(-127, ceil(log2(amax/fmax))), and amax/S lands in
    (fmax/2, fmax] unless the -127 clamp is active."""
    f = all_bf16_as_f32()
    pos = f[(f > 0) & np.isfinite(f)]
    fmax = FMAX[fmt]
    for a in pos:
        a = float(a)
        sb = oracle.scale_byte(a, fmt)
        e = sb - 127
        assert e == exact.scale_exponent(Fraction(a), fmt)
        assert e == max(-127, math.ceil(math.log2(a / fmax)))
        r = a / 2.0 ** e
        assert r <= fmax
        if e > -127:
            assert r > fmax / 2
    assert oracle.scale_byte(0.0, fmt) == 127                      # zero block -> S = 1
    assert oracle.scale_byte(float("nan"), fmt) == 255
    assert oracle.scale_byte(float("inf"), fmt) == 255


def test_round_bf16_matches_torch(oracle_lib):
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-140, 120, 20000))).astype(np.float32)
    v = np.concatenate([v, np.array([0.0, -0.0, 3.4e38, -3.4e38, 1e-45, 2.0 ** -133 * 1.5], np.float32)])
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.round_bf16(float(x)) for x in v], dtype=np.uint16)
    assert np.array_equal(ours, ref)

"""Exact-rational twin of the MXFP8 oracle, for pinning it on small inputs.

TEST INFRASTRUCTURE ONLY (used by the test suite).  Pure Python with
``fractions.Fraction`` and integers: no floating point enters any decision here,
and the algorithms deliberately differ from ``mxo.c`` (nearest-value brute force
over every code instead of a neighbour search; exponent from integer bit lengths
instead of a search loop), so that a mistake in one is unlikely to be repeated in
the other.

Source: "Low-Precision GPU Programming" (leetllm.com):
  * "Format taxonomy: range, spacing, and bitfields" -- E4M3 (bias 7, 3 mantissa bits,
    max 448, NaN 0x7F/0xFF, no Inf) and E5M2 (bias 15, 2 mantissa bits, max 57,344,
    smallest subnormal 2^-16).
  * "Numerical hazards" -- round-to-nearest-even with ties to the even code; a
    saturating conversion clamps the rounded value to +-fmax.
  * "Microscaling: the two-row experiment" -- E8M0 byte c is 2^(c-127), 255 is NaN,
    anything that is not an unsigned byte is rejected with ValueError; the block
    scale is the power of two obtained by rounding amax/fmax upward (exponent
    clamped below at -127), and a zero block takes scale 1.
  * "Scale ownership and the GEMM dataflow" -- the block-K contraction keeps the
    product of the two block scales inside the sum over blocks.
"""
from __future__ import annotations

import math
from fractions import Fraction

FORMATS = {
    # name: (exponent bits, mantissa bits, bias, max finite magnitude)
    "e4m3": (4, 3, 7, Fraction(448)),
    "e5m2": (5, 2, 15, Fraction(57344)),
}


_E8M0_NAN = 0xFF          # the one non-numeric E8M0 byte


def decode_e8m0(byte):
    """Value of an E8M0 scale byte: an 8-bit biased exponent with no sign and no mantissa,
    bias 127, so byte c stands for 2^(c - 127) exactly (a Fraction); 0xFF is NaN.
    Arguments that are not a Python int in 0..255 are not scale bytes (ValueError)."""
    is_byte = isinstance(byte, int) and not isinstance(byte, bool) and (byte & ~0xFF) == 0
    if not is_byte:
        raise ValueError("E8M0 scale bytes are integers 0..255, got %r" % (byte,))
    return math.nan if byte == _E8M0_NAN else Fraction(1, 1 << 127) * (1 << byte)


def e8m0_exact(code: int) -> Fraction:
    if not 0 <= code <= 254:
        raise ValueError("finite E8M0 byte required")
    return Fraction(2) ** (code - 127)


def decode(code: int, fmt: str):
    """Exact value of an FP8 code: a Fraction, or the strings 'nan' / '+inf' / '-inf'."""
    eb, mb, bias, _ = FORMATS[fmt]
    sign = -1 if code & 0x80 else 1
    E = (code >> mb) & ((1 << eb) - 1)
    m = code & ((1 << mb) - 1)
    if fmt == "e4m3" and E == 15 and m == 7:
        return "nan"
    if fmt == "e5m2" and E == 31:
        if m != 0:
            return "nan"
        return "+inf" if sign > 0 else "-inf"
    if E == 0:
        mag = Fraction(m, 1 << mb) * Fraction(2) ** (1 - bias)
    else:
        mag = (1 + Fraction(m, 1 << mb)) * Fraction(2) ** (E - bias)
    return sign * mag


def finite_magnitudes(fmt: str):
    """[(code, value)] for every finite non-negative code, in code order."""
    out = []
    for c in range(128):
        v = decode(c, fmt)
        if isinstance(v, str):
            continue
        out.append((c, v))
    return out


_MAGS = {f: finite_magnitudes(f) for f in FORMATS}


def encode(x: Fraction, fmt: str, negative_zero: bool = False) -> int:
    """RNE + satfinite encoding of an exact rational x by brute force over all codes.

    ``negative_zero`` marks x == 0 as -0 (Fractions carry no signed zero).
    """
    fmax = FORMATS[fmt][3]
    neg = x < 0 or (x == 0 and negative_zero)
    a = abs(x)
    sign = 0x80 if neg else 0x00
    if a >= fmax:
        best = max(_MAGS[fmt], key=lambda cv: cv[1])[0]
        return sign | best
    best_c, best_d = None, None
    for c, v in _MAGS[fmt]:
        d = abs(a - v)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best_c, best_d = c, d
    return sign | best_c


def encode_int(num: int, den_log2: int, fmt: str, negative: bool) -> int:
    """Same as :func:`encode` for x = num / 2^den_log2 (num >= 0), in integer arithmetic.

    All finite E4M3 values are multiples of 2^-9 and all E5M2 values multiples of 2^-16,
    so both sides are put over 2^max(den_log2, 16) and compared as integers.
    """
    D = max(den_log2, 16)
    a = num << (D - den_log2)
    sign = 0x80 if negative else 0x00
    cands = _INT_MAGS.get((fmt, D))
    if cands is None:
        cands = [(c, (v.numerator << D) // v.denominator) for c, v in _MAGS[fmt]]
        _INT_MAGS[(fmt, D)] = cands
    if a >= cands[-1][1]:
        return sign | cands[-1][0]
    best_c, best_d = None, None
    for c, v in cands:
        d = abs(a - v)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best_c, best_d = c, d
    return sign | best_c


_INT_MAGS: dict = {}


def ceil_log2(q: Fraction) -> int:
    """Exact ceil(log2(q)) for a positive rational q, from integer bit lengths."""
    n, d = q.numerator, q.denominator
    # floor(log2(n/d)) is bitlen(n) - bitlen(d) or one less
    f = n.bit_length() - d.bit_length()
    if Fraction(2) ** f > q:
        f -= 1
    return f if Fraction(2) ** f == q else f + 1


def scale_exponent(amax: Fraction, fmt: str) -> int:
    """Block scale exponent e with S = 2^e: max(-127, ceil(log2(amax/fmax))), 0 if amax == 0."""
    if amax == 0:
        return 0
    return max(-127, ceil_log2(amax / FORMATS[fmt][3]))


def largest_normal_exponent(fmt: str) -> int:
    """Exponent E of the format's largest finite value written 1.f * 2^E, from its code."""
    top = max(v for _, v in _MAGS[fmt])
    E = 0
    while Fraction(2) ** (E + 1) <= top:
        E += 1
    return E


def scale_exponent_ocp(amax: Fraction, fmt: str) -> int:
    """The OCP MX rule: floor(log2(amax)) - (exponent of the largest normal), at least -127;
    0 for a zero block.  floor(log2) by comparing powers of two, exactly."""
    if amax == 0:
        return 0
    E = 0
    while Fraction(2) ** E > amax:
        E -= 1
    while Fraction(2) ** (E + 1) <= amax:
        E += 1
    return max(-127, E - largest_normal_exponent(fmt))


def quantize_block(values, fmt: str, negzero=None, rule: str = "ceil"):
    """Quantize a list of <= 32 exact rationals (one MX block, zero-padded to 32).

    ``negzero[i]`` marks value i as -0.  ``rule`` picks the scale exponent ("ceil": the
    pages', "ocp": the OCP MX specification's).  Returns (codes[32], scale_byte).
    """
    assert len(values) <= 32
    amax = max((abs(v) for v in values), default=Fraction(0))
    e = scale_exponent(amax, fmt) if rule == "ceil" else scale_exponent_ocp(amax, fmt)
    S = Fraction(2) ** e
    codes = []
    for i in range(32):
        if i < len(values):
            nz = bool(negzero[i]) if negzero is not None else False
            codes.append(encode(values[i] / S, fmt, negative_zero=nz))
        else:
            codes.append(0x00)
    return codes, e + 127


def block_gemm(xc, xs, xfmt, wc, ws, wfmt, K, alpha=Fraction(1), bias=None):
    """Exact Y[i][j] = alpha * sum_b S_X[i][b] S_W[j][b] sum_{k in b} x~[i][k] w~[j][k] + bias[j].

    xc[i][k], wc[j][k] are codes (W as rows, i.e. column-major W), xs/ws E8M0 bytes.
    """
    M, N = len(xc), len(wc)
    nb = (K + 31) // 32
    Y = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for b in range(nb):
                inner = Fraction(0)
                for k in range(32 * b, min(32 * b + 32, K)):
                    inner += decode(xc[i][k], xfmt) * decode(wc[j][k], wfmt)
                acc += e8m0_exact(xs[i][b]) * e8m0_exact(ws[j][b]) * inner
            Y[i][j] = alpha * acc + (bias[j] if bias is not None else 0)
    return Y


def dequant_then_matmul(xc, xs, xfmt, wc, ws, wfmt, K):
    """Exact (dequantize X) @ (dequantize W)^T: the reconstructed-operand product."""
    M, N = len(xc), len(wc)
    Xh = [[decode(xc[i][k], xfmt) * e8m0_exact(xs[i][k // 32]) for k in range(K)] for i in range(M)]
    Wh = [[decode(wc[j][k], wfmt) * e8m0_exact(ws[j][k // 32]) for k in range(K)] for j in range(N)]
    return [[sum((Xh[i][k] * Wh[j][k] for k in range(K)), Fraction(0)) for j in range(N)]
            for i in range(M)]

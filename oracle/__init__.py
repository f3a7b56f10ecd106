"""CPU oracle for MXFP8 (OCP-MX block-scaled FP8) quantize, dequantize and GEMM.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.  The
arithmetic lives in ``mxo.c`` (plain C, built with gcc, FP64, table search for the
FP8 encoding, literal search for the scale exponent); this module only marshals
numpy arrays through ctypes.  ``oracle.exact`` is an independent exact-rational
twin used to pin the C code on small inputs.

Source: "Low-Precision GPU Programming" (leetllm.com) -- sections "Format taxonomy",
"Numerical hazards", "Scale ownership and the GEMM dataflow", "Scaling architectures",
"Microscaling: the two-row experiment".  See ``mxo.c`` for the per-function citations.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxo.c")
# MXO_SANITIZE=1 selects a build of mxo.c instrumented with AddressSanitizer and
# UndefinedBehaviorSanitizer (libmxo_san.so; the interpreter must then run with libasan
# preloaded, e.g. LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0).
_SANITIZE = os.environ.get("MXO_SANITIZE", "") == "1"
_LIB_PATH = os.path.join(_HERE, "libmxo_san.so" if _SANITIZE else "libmxo.so")

FMT = {"e4m3": 0, "e5m2": 1}
SRC = {"f32": 0, "bf16": 1}


def build(force: bool = True) -> str:
    """Compile mxo.c into libmxo.so with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        san = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined"] if _SANITIZE else []
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off"] + san + [_SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        # (re)build when the library is missing or older than its source
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        i64 = ctypes.c_int64
        vp = ctypes.c_void_p
        L.mxo_encode_sr.restype = ctypes.c_uint8
        L.mxo_encode_sr.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_uint32]
        L.mxo_philox4x32_10.restype = None
        L.mxo_philox4x32_10.argtypes = [vp, vp, vp]
        L.mxo_quantize_sr.restype = None
        L.mxo_quantize_sr.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                      vp, i64, vp, i64]
        L.mxo_quantize_scaled.restype = None
        L.mxo_quantize_scaled.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp, i64,
                                          vp, i64, vp, i64, vp, vp, i64]
        L.mxo_silu.restype = ctypes.c_double
        L.mxo_silu.argtypes = [ctypes.c_double]
        L.mxo_silu_array.restype = None
        L.mxo_silu_array.argtypes = [vp, vp, i64]
        L.mxo_decode.restype = ctypes.c_double
        L.mxo_decode.argtypes = [ctypes.c_uint8, ctypes.c_int]
        L.mxo_decode_e8m0.restype = ctypes.c_double
        L.mxo_decode_e8m0.argtypes = [ctypes.c_uint8]
        L.mxo_fmax.restype = ctypes.c_double
        L.mxo_fmax.argtypes = [ctypes.c_int]
        L.mxo_encode.restype = ctypes.c_uint8
        L.mxo_encode.argtypes = [ctypes.c_double, ctypes.c_int]
        L.mxo_scale_byte.restype = ctypes.c_int
        L.mxo_scale_byte.argtypes = [ctypes.c_double, ctypes.c_int]
        L.mxo_scale_byte_ocp.restype = ctypes.c_int
        L.mxo_scale_byte_ocp.argtypes = [ctypes.c_double, ctypes.c_int]
        L.mxo_quantize_rule.restype = None
        L.mxo_quantize_rule.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        vp, i64, vp, i64]
        L.mxo_num_finite_codes.restype = ctypes.c_int
        L.mxo_num_finite_codes.argtypes = [ctypes.c_int]
        L.mxo_num_threads.restype = ctypes.c_int
        L.mxo_num_threads.argtypes = []
        L.mxo_round_bf16.restype = ctypes.c_uint16
        L.mxo_round_bf16.argtypes = [ctypes.c_double]
        L.mxo_quantize.restype = None
        L.mxo_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                   vp, i64, vp, i64]
        L.mxo_dequantize.restype = None
        L.mxo_dequantize.argtypes = [vp, i64, vp, i64, ctypes.c_int, i64, i64, vp, ctypes.c_int, i64]
        L.mxo_gemm.restype = None
        L.mxo_gemm.argtypes = [i64, i64, i64, vp, i64, vp, i64, ctypes.c_int,
                               vp, i64, vp, i64, ctypes.c_int, ctypes.c_double, vp, vp, vp]
        L.mxo_gemm_sampled.restype = None
        L.mxo_gemm_sampled.argtypes = [i64, vp, i64, vp, i64, ctypes.c_int,
                                       vp, i64, vp, i64, ctypes.c_int, ctypes.c_double, vp,
                                       i64, vp, vp, vp, vp]
        _ = u8p
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------- scalar codec

def decode(code: int, fmt: str) -> float:
    return lib().mxo_decode(code, FMT[fmt])


def decode_e8m0(c: int) -> float:
    return lib().mxo_decode_e8m0(c)


def fmax(fmt: str) -> float:
    return lib().mxo_fmax(FMT[fmt])


def encode(a: float, fmt: str) -> int:
    return int(lib().mxo_encode(float(a), FMT[fmt]))


def scale_byte(amax: float, fmt: str) -> int:
    return int(lib().mxo_scale_byte(float(amax), FMT[fmt]))


def num_finite_codes(fmt: str) -> int:
    return int(lib().mxo_num_finite_codes(FMT[fmt]))


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().mxo_num_threads())


def round_bf16(v: float) -> int:
    return int(lib().mxo_round_bf16(float(v)))


# ----------------------------------------------------------------- array ops

def _src_type(src: np.ndarray) -> int:
    if src.dtype == np.float32:
        return SRC["f32"]
    if src.dtype == np.uint16:   # bf16 bit patterns
        return SRC["bf16"]
    raise TypeError("src must be float32 or uint16 (bf16 bits), got %s" % src.dtype)


RULE = {"ceil": 0, "ocp": 1}


def scale_byte_ocp(amax: float, fmt: str) -> int:
    """E8M0 byte of the OCP MX scale rule: floor(log2(amax)) - emax_elem, clamped at -127."""
    return lib().mxo_scale_byte_ocp(float(amax), FMT[fmt])


def quantize(src: np.ndarray, fmt: str, axis: int = 0, rule: str = "ceil"):
    """Quantize a 2-D array (float32, or uint16 holding bf16 bits).

    axis=0: 1x32 groups along each row; returns codes [rows][Kp], scales [rows][Kp/32].
    axis=1: 32x1 groups down each column, stored transposed: codes [cols][Kp], scales
            [cols][Kp/32] with K = rows.
    rule="ceil": the pages' scale rule (amax/fmax rounded up to a power of two);
    rule="ocp": the OCP MX specification's rule (floor(log2(amax)) - emax_elem, satfinite).
    """
    src = np.ascontiguousarray(src)
    rows, cols = src.shape
    L, K = (rows, cols) if axis == 0 else (cols, rows)
    Kp = 32 * ((K + 31) // 32)
    codes = np.zeros((L, max(Kp, 1)), dtype=np.uint8)
    scales = np.zeros((L, max(Kp // 32, 1)), dtype=np.uint8)
    if L > 0 and K > 0:
        lib().mxo_quantize_rule(_ptr(src), _src_type(src), rows, cols, cols, axis, FMT[fmt], RULE[rule],
                                _ptr(codes), codes.shape[1], _ptr(scales), scales.shape[1])
    return codes[:, :Kp], scales[:, :Kp // 32]


def encode_sr(a: float, fmt: str, r24: int) -> int:
    """Stochastically rounded code of the exact value a under the 24-bit random integer r24."""
    return int(lib().mxo_encode_sr(float(a), FMT[fmt], int(r24)))


def philox4x32_10(counter, key):
    """Philox4x32-10 block: four 32-bit counter words, two key words -> four output words."""
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().mxo_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return [int(v) for v in out]


def quantize_sr(src: np.ndarray, fmt: str, seed: int, axis: int = 0):
    """quantize() with stochastically rounded codes; element n = line * Kp + k draws word
    n % 4 of Philox4x32-10(counter (n // 4), key = seed) and keeps its top 24 bits."""
    src = np.ascontiguousarray(src)
    rows, cols = src.shape
    L, K = (rows, cols) if axis == 0 else (cols, rows)
    Kp = 32 * ((K + 31) // 32)
    codes = np.zeros((L, max(Kp, 1)), dtype=np.uint8)
    scales = np.zeros((L, max(Kp // 32, 1)), dtype=np.uint8)
    if L > 0 and K > 0:
        lib().mxo_quantize_sr(_ptr(src), _src_type(src), rows, cols, cols, axis, FMT[fmt], int(seed) & (2 ** 64 - 1),
                              _ptr(codes), codes.shape[1], _ptr(scales), scales.shape[1])
    return codes[:, :Kp], scales[:, :Kp // 32]


def quantize_scaled(src: np.ndarray, fmt: str, given_scales: np.ndarray, axis: int = 0):
    """Quantize with caller-owned E8M0 scale bytes given_scales [L][nb] (RNE-satfinite codes).

    Returns (codes [L][Kp], amax [L][nb] float32, clipped [L][nb] uint8, flushed [L][nb] uint8).
    """
    src = np.ascontiguousarray(src)
    rows, cols = src.shape
    L, K = (rows, cols) if axis == 0 else (cols, rows)
    Kp = 32 * ((K + 31) // 32)
    nb = Kp // 32
    gs = np.ascontiguousarray(given_scales, dtype=np.uint8)
    if gs.shape != (L, nb):
        raise ValueError("given_scales must be [L][nb] = %r" % ((L, nb),))
    codes = np.zeros((L, max(Kp, 1)), dtype=np.uint8)
    amax = np.zeros((L, max(nb, 1)), dtype=np.float32)
    clipped = np.zeros((L, max(nb, 1)), dtype=np.uint8)
    flushed = np.zeros((L, max(nb, 1)), dtype=np.uint8)
    if L > 0 and K > 0:
        lib().mxo_quantize_scaled(_ptr(src), _src_type(src), rows, cols, cols, axis, FMT[fmt], _ptr(gs), nb,
                                  _ptr(codes), codes.shape[1], _ptr(amax), amax.shape[1], _ptr(clipped),
                                  _ptr(flushed), clipped.shape[1])
    return codes[:, :Kp], amax[:, :nb], clipped[:, :nb], flushed[:, :nb]


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str, K: int, out: str = "f32"):
    """Reconstruct x_hat = dec(code) * 2^(s-127); returns float32 or uint16 (bf16 bits)."""
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    L = codes.shape[0]
    dst = np.zeros((L, K), dtype=np.float32 if out == "f32" else np.uint16)
    if L > 0 and K > 0:
        lib().mxo_dequantize(_ptr(codes), codes.shape[1], _ptr(scales), scales.shape[1], FMT[fmt],
                             L, K, _ptr(dst), SRC[out], K)
    return dst


def silu(v):
    """SiLU in FP64 of a scalar or an array (values converted to FP64 first)."""
    if np.isscalar(v):
        return lib().mxo_silu(float(v))
    a = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(a)
    if a.size:
        lib().mxo_silu_array(_ptr(a), _ptr(out), a.size)
    return out


def gemm(x_codes, x_scales, x_fmt, w_codes, w_scales, w_fmt, K, alpha=1.0, bias=None):
    """FP64 reference Y[M][N] and bound T[M][N]; W is given as rows w_codes[N][Kp]."""
    xc = np.ascontiguousarray(x_codes)
    xs = np.ascontiguousarray(x_scales)
    wc = np.ascontiguousarray(w_codes)
    ws = np.ascontiguousarray(w_scales)
    M, N = xc.shape[0], wc.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    t = np.zeros((M, N), dtype=np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    if M > 0 and N > 0:
        lib().mxo_gemm(M, N, K, _ptr(xc), xc.shape[1], _ptr(xs), xs.shape[1], FMT[x_fmt],
                       _ptr(wc), wc.shape[1], _ptr(ws), ws.shape[1], FMT[w_fmt], float(alpha),
                       _ptr(b), _ptr(y), _ptr(t))
    return y, t


def gemm_sampled(x_codes, x_scales, x_fmt, w_codes, w_scales, w_fmt, K, ii, jj, alpha=1.0,
                 bias=None):
    """Reference for the output elements (ii[s], jj[s]) only; returns (y[n], t[n])."""
    xc = np.ascontiguousarray(x_codes)
    xs = np.ascontiguousarray(x_scales)
    wc = np.ascontiguousarray(w_codes)
    ws = np.ascontiguousarray(w_scales)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    n = ii.shape[0]
    y = np.zeros(n, dtype=np.float64)
    t = np.zeros(n, dtype=np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    if n > 0:
        lib().mxo_gemm_sampled(K, _ptr(xc), xc.shape[1], _ptr(xs), xs.shape[1], FMT[x_fmt],
                               _ptr(wc), wc.shape[1], _ptr(ws), ws.shape[1], FMT[w_fmt],
                               float(alpha), _ptr(b), n, _ptr(ii), _ptr(jj), _ptr(y), _ptr(t))
    return y, t

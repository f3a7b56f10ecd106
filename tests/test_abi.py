"""CPU tests of the C ABI boundary: the library loads, exports every declared entry point,
and rejects invalid arguments on the host (before any HIP call, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import mxfp8_block_scaled_03_amd as mxq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    txt = open(os.path.join(ROOT, "include", "mxq.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mxq_[a-z_0-9]+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    assert {"mxq_quantize", "mxq_quantize_rule", "mxq_quantize_dual", "mxq_quantize_sr", "mxq_quantize_scaled", "mxq_dequantize", "mxq_gemm", "mxq_gemm_ex", "mxq_gemm_ex_noalloc", "mxq_gemm_exact_plan",
            "mxq_status_string", "mxq_version"} <= set(declared_symbols())


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mxq.library_path())
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    assert mxq.mxq_version() >= 100
    for st in range(-8, 1):
        s = mxq.mxq_status_string(st)
        assert s.startswith("MXQ_")
    assert "unknown" in mxq.mxq_status_string(-99)


# A 64 KiB-aligned non-null address.  Every call below must fail validation (or be an
# empty problem), so nothing is ever enqueued with it -- never add a case that passes.
FAKE = 0x10000


def q(**kw):
    a = dict(src=FAKE, src_type=mxq.MXQ_BF16, rows=4, cols=64, ld_src=64, axis=mxq.MXQ_ROWWISE,
             elem=mxq.MXQ_E4M3, codes=FAKE, ld_codes=64, scales=FAKE, ld_scales=2)
    a.update(kw)
    return mxq.mxq_quantize(a["src"], a["src_type"], a["rows"], a["cols"], a["ld_src"], a["axis"], a["elem"],
                            a["codes"], a["ld_codes"], a["scales"], a["ld_scales"], None)


def test_quantize_validation():
    assert q(src_type=mxq.MXQ_E4M3) == -5
    assert q(elem=mxq.MXQ_F32) == -5
    assert q(axis=7) == -6
    assert q(rows=-1) == -2
    assert q(src=None) == -1
    assert q(codes=None) == -1
    assert q(scales=None) == -1
    assert q(ld_src=63) == -3
    assert q(ld_codes=48) == -3              # < Kp = 64
    assert q(ld_scales=1) == -3
    assert q(ld_codes=80 + 1) == -4          # not a multiple of 16
    assert q(codes=FAKE + 8) == -4
    assert q(src=FAKE + 1) == -4             # bf16 needs 2-byte alignment
    # colwise: K = rows -> Kp = 32, lines = cols
    assert q(axis=mxq.MXQ_COLWISE, ld_codes=16) == -3
    # empty problems succeed without touching pointers
    assert q(rows=0, src=None, codes=None, scales=None) == 0
    assert q(cols=0, src=None, codes=None, scales=None) == 0


def test_quantize_rule_validation():
    def qr(rule, **kw):
        a = dict(src=FAKE, src_type=mxq.MXQ_BF16, rows=4, cols=64, ld_src=64, axis=mxq.MXQ_ROWWISE,
                 elem=mxq.MXQ_E4M3, codes=FAKE, ld_codes=64, scales=FAKE, ld_scales=2)
        a.update(kw)
        return mxq.mxq_quantize_rule(a["src"], a["src_type"], a["rows"], a["cols"], a["ld_src"], a["axis"],
                                     a["elem"], rule, a["codes"], a["ld_codes"], a["scales"], a["ld_scales"], None)
    assert qr(2) == -6
    assert qr(-1) == -6
    for rule in (mxq.MXQ_SCALE_CEIL, mxq.MXQ_SCALE_OCP):
        assert qr(rule, src_type=mxq.MXQ_E4M3) == -5
        assert qr(rule, axis=7) == -6
        assert qr(rule, rows=-1) == -2
        assert qr(rule, codes=None) == -1
        assert qr(rule, ld_codes=48) == -3
        assert qr(rule, codes=FAKE + 8) == -4
        assert qr(rule, rows=0, src=None, codes=None, scales=None) == 0


def test_quantize_sr_validation():
    def qs(**kw):
        a = dict(src=FAKE, src_type=mxq.MXQ_BF16, rows=4, cols=64, ld_src=64, axis=mxq.MXQ_ROWWISE,
                 elem=mxq.MXQ_E5M2, seed=2 ** 64 - 1, codes=FAKE, ld_codes=64, scales=FAKE, ld_scales=2)
        a.update(kw)
        return mxq.mxq_quantize_sr(a["src"], a["src_type"], a["rows"], a["cols"], a["ld_src"], a["axis"], a["elem"],
                                   a["seed"], a["codes"], a["ld_codes"], a["scales"], a["ld_scales"], None)
    assert qs(src_type=mxq.MXQ_E4M3) == -5
    assert qs(elem=mxq.MXQ_F32) == -5
    assert qs(axis=3) == -6
    assert qs(rows=-1) == -2
    assert qs(codes=None) == -1
    assert qs(ld_codes=48) == -3
    assert qs(ld_scales=1) == -3
    assert qs(ld_codes=80 + 1) == -4
    assert qs(src=FAKE + 1) == -4
    assert qs(axis=mxq.MXQ_COLWISE, ld_codes=16) == -3
    assert qs(rows=0, src=None, codes=None, scales=None) == 0


def test_quantize_scaled_validation():
    def qc(**kw):
        a = dict(src=FAKE, src_type=mxq.MXQ_F32, rows=4, cols=64, ld_src=64, axis=mxq.MXQ_ROWWISE,
                 elem=mxq.MXQ_E4M3, scales=FAKE, ld_scales=2, codes=FAKE, ld_codes=64, amax=None, ld_amax=0,
                 clipped=None, flushed=None, ld_diag=0)
        a.update(kw)
        return mxq.mxq_quantize_scaled(a["src"], a["src_type"], a["rows"], a["cols"], a["ld_src"], a["axis"],
                                       a["elem"], a["scales"], a["ld_scales"], a["codes"], a["ld_codes"], a["amax"],
                                       a["ld_amax"], a["clipped"], a["flushed"], a["ld_diag"], None)
    assert qc(elem=mxq.MXQ_BF16) == -5
    assert qc(axis=2) == -6
    assert qc(scales=None) == -1
    assert qc(ld_scales=1) == -3
    assert qc(amax=FAKE, ld_amax=1) == -3
    assert qc(clipped=FAKE, ld_diag=1) == -3
    assert qc(flushed=FAKE, ld_diag=1) == -3
    assert qc(amax=FAKE + 2, ld_amax=2) == -4
    assert qc(codes=FAKE + 4) == -4
    assert qc(src=FAKE + 2) == -4
    assert qc(cols=0, src=None, scales=None, codes=None) == 0


def qd(**kw):
    # rows = 40 -> column blocks Kp_c = 64; cols = 64 -> row blocks Kp_r = 64
    a = dict(src=FAKE, src_type=mxq.MXQ_F32, rows=40, cols=64, ld_src=64, elem=mxq.MXQ_E5M2, rc=FAKE, ld_rc=64,
             rs=FAKE, ld_rs=2, cc=FAKE, ld_cc=64, cs=FAKE, ld_cs=2)
    a.update(kw)
    return mxq.mxq_quantize_dual(a["src"], a["src_type"], a["rows"], a["cols"], a["ld_src"], a["elem"], a["rc"],
                                 a["ld_rc"], a["rs"], a["ld_rs"], a["cc"], a["ld_cc"], a["cs"], a["ld_cs"], None)


def test_quantize_dual_validation():
    assert qd(src_type=mxq.MXQ_E4M3) == -5
    assert qd(elem=mxq.MXQ_BF16) == -5
    assert qd(rows=-1) == -2
    assert qd(cols=1 << 40) == -2
    for k in ("src", "rc", "rs", "cc", "cs"):
        assert qd(**{k: None}) == -1
    assert qd(ld_src=63) == -3
    assert qd(ld_rc=48) == -3                # < Kp_r = 64
    assert qd(ld_rs=1) == -3
    assert qd(ld_cc=48) == -3                # < Kp_c = 64
    assert qd(ld_cs=1) == -3
    assert qd(ld_rc=72) == -4                # not a multiple of 16
    assert qd(ld_cc=72) == -4
    assert qd(rc=FAKE + 8) == -4
    assert qd(cc=FAKE + 4) == -4
    assert qd(src=FAKE + 2) == -4            # fp32 needs 4-byte alignment
    assert qd(rows=0, src=None, rc=None, rs=None, cc=None, cs=None) == 0
    assert qd(cols=0, src=None, rc=None, rs=None, cc=None, cs=None) == 0


def g(**kw):
    a = dict(M=8, N=8, K=64, xc=FAKE, ld_x=64, xs=FAKE, ld_xs=2, xe=mxq.MXQ_E4M3, wc=FAKE, ld_w=64, ws=FAKE,
             ld_ws=2, we=mxq.MXQ_E4M3, alpha=1.0, bias=None, y=FAKE, yt=mxq.MXQ_F32, ld_y=8, acc=0)
    a.update(kw)
    return mxq.mxq_gemm(a["M"], a["N"], a["K"], a["xc"], a["ld_x"], a["xs"], a["ld_xs"], a["xe"], a["wc"],
                        a["ld_w"], a["ws"], a["ld_ws"], a["we"], a["alpha"], a["bias"], a["y"], a["yt"], a["ld_y"],
                        a["acc"], None)


def test_gemm_validation():
    assert g(xe=mxq.MXQ_BF16) == -5
    assert g(yt=mxq.MXQ_E4M3) == -5
    assert g(M=-1) == -2
    assert g(K=1 << 24) == -2
    assert g(alpha=float("nan")) == -6
    assert g(alpha=float("inf")) == -6
    assert g(acc=2) == -6
    assert g(acc=-1) == -6
    assert g(y=None) == -1
    assert g(xc=None) == -1
    assert g(ws=None) == -1
    assert g(ld_x=32) == -3
    assert g(ld_ws=1) == -3
    assert g(ld_xs=1 << 23) == -3
    assert g(ld_y=7) == -3
    assert g(ld_x=72) == -4
    assert g(wc=FAKE + 4) == -4
    assert g(y=FAKE + 2) == -4
    assert g(bias=FAKE + 2) == -4
    assert g(M=0, xc=None, y=None) == 0
    assert g(N=0, wc=None, y=None) == 0


def gx(**kw):
    a = dict(M=8, N=40, K=64, xc=FAKE, ld_x=64, xs=FAKE, ld_xs=2, xe=mxq.MXQ_E4M3, wc=FAKE, ld_w=64, ws=FAKE,
             ld_ws=2, we=mxq.MXQ_E4M3, alpha=1.0, bias=None, act=mxq.MXQ_ACT_SILU, y=None, yt=mxq.MXQ_BF16, ld_y=0,
             qe=mxq.MXQ_E4M3, qc=FAKE, ld_qc=64, qs=FAKE, ld_qs=2, acc=0)     # N = 40 -> Np = 64
    a.update(kw)
    fn = a.pop("fn", mxq.mxq_gemm_ex)
    return fn(a["M"], a["N"], a["K"], a["xc"], a["ld_x"], a["xs"], a["ld_xs"], a["xe"], a["wc"],
              a["ld_w"], a["ws"], a["ld_ws"], a["we"], a["alpha"], a["bias"], a["act"], a["y"],
              a["yt"], a["ld_y"], a["qe"], a["qc"], a["ld_qc"], a["qs"], a["ld_qs"], a["acc"], None)


def test_gemm_ex_noalloc_validates_like_gemm_ex():
    """The allocation-free variant rejects exactly what mxq_gemm_ex rejects, on the host."""
    cases = [dict(act=2), dict(qe=mxq.MXQ_BF16), dict(qc=None), dict(ld_qc=48), dict(ld_qc=72), dict(y=FAKE, ld_y=39),
             dict(alpha=float("inf")), dict(acc=3), dict(K=-1), dict(M=0, xc=None, qc=None, qs=None)]
    for c in cases:
        assert gx(fn=mxq.mxq_gemm_ex_noalloc, **c) == gx(**c), c


def test_gemm_ex_validation():
    assert gx(act=2) == -6
    assert gx(act=-1) == -6
    assert gx(qe=mxq.MXQ_BF16) == -5
    assert gx(y=FAKE, yt=mxq.MXQ_E4M3, ld_y=40) == -5
    assert gx(qc=None) == -1                  # neither output
    assert gx(qs=None) == -1
    assert gx(ld_qc=48) == -3                 # < Np = 64
    assert gx(ld_qs=1) == -3
    assert gx(ld_qc=72) == -4                 # not a multiple of 16
    assert gx(qc=FAKE + 8) == -4
    assert gx(y=FAKE, ld_y=39) == -3
    assert gx(y=FAKE + 1, ld_y=40) == -4
    assert gx(alpha=float("nan")) == -6
    assert gx(M=0, xc=None, qc=None, qs=None) == 0
    # mxq_gemm keeps requiring y
    assert g(y=None) == -1


def test_dequantize_validation():
    def d(**kw):
        a = dict(c=FAKE, ldc=64, s=FAKE, lds=2, e=mxq.MXQ_E4M3, L=4, K=64, dst=FAKE, dt=mxq.MXQ_F32, ldd=64)
        a.update(kw)
        return mxq.mxq_dequantize(a["c"], a["ldc"], a["s"], a["lds"], a["e"], a["L"], a["K"], a["dst"], a["dt"],
                                  a["ldd"], None)
    assert d(e=mxq.MXQ_F32) == -5
    assert d(dt=mxq.MXQ_E5M2) == -5
    assert d(L=-2) == -2
    assert d(c=None) == -1
    assert d(ldc=63) == -3
    assert d(lds=1) == -3
    assert d(ldd=10) == -3
    assert d(dst=FAKE + 2) == -4
    assert d(L=0, c=None, s=None, dst=None) == 0


def test_python_wrapper_raises_value_error():
    with pytest.raises(ValueError):
        mxq._binding._check(-3, "x")

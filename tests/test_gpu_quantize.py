"""GPU parity of mxq_quantize / mxq_dequantize against the CPU oracle: bit-exact codes,
scales and reconstructions, on ragged, padded, unaligned and special-value inputs and on
the full-size workloads."""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_block_scaled_03_amd as mxq
from mxfp8_block_scaled_03_amd import workloads as wl
from gpu_helpers import host_src, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gpu_quantize(x_cpu: torch.Tensor, fmt: str, axis: str, pad_codes=16, pad_scales=3):
    """Quantize on the GPU into canary-filled, over-wide outputs; check the canaries."""
    rows, cols = x_cpu.shape
    L, K = (rows, cols) if axis == "row" else (cols, rows)
    Kp = 32 * ((K + 31) // 32)
    nb = Kp // 32
    codes = torch.full((L, Kp + pad_codes), 0xCD, dtype=torch.uint8, device=DEV)
    scales = torch.full((L, nb + pad_scales), 0xCD, dtype=torch.uint8, device=DEV)
    x = x_cpu.to(DEV)
    mxq.quantize(x, fmt, axis, codes=codes, scales=scales)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.all(c[:, Kp:] == 0xCD), "write past Kp"
    assert np.all(s[:, nb:] == 0xCD), "write past nb"
    return c[:, :Kp], s[:, :nb]


def oracle_quantize(x_cpu, fmt, axis):
    return oracle.quantize(host_src(x_cpu), fmt, axis=0 if axis == "row" else 1)


def assert_same(gc, gs, oc, os_, what):
    if not np.array_equal(gs, os_):
        i = np.argwhere(gs != os_)[0]
        raise AssertionError("%s: scale mismatch at %s gpu=%d oracle=%d" % (what, i.tolist(), gs[tuple(i)], os_[tuple(i)]))
    if not np.array_equal(gc, oc):
        i = np.argwhere(gc != oc)[0]
        raise AssertionError("%s: code mismatch at %s gpu=0x%02x oracle=0x%02x"
                             % (what, i.tolist(), gc[tuple(i)], oc[tuple(i)]))


SHAPES = [(1, 1), (3, 5), (7, 31), (5, 32), (4, 33), (16, 64), (9, 100), (130, 72), (64, 4096), (33, 4001), (200, 40)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("axis", ["row", "col"])
def test_quantize_shapes(dtype, fmt, axis):
    rng = np.random.default_rng(10)
    for rows, cols in SHAPES:
        say("quantize %s %s %s %dx%d" % (dtype, fmt, axis, rows, cols))
        scale = np.exp2(rng.integers(-20, 20, (rows, 1))).astype(np.float32)
        x = torch.from_numpy(rng.standard_normal((rows, cols)).astype(np.float32) * scale).to(dtype)
        gc, gs = gpu_quantize(x, fmt, axis)
        oc, os_ = oracle_quantize(x, fmt, axis)
        assert_same(gc, gs, oc, os_, "%dx%d" % (rows, cols))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_dense_outputs(dtype, fmt):
    """Outputs exactly Kp wide (no padding) with K a multiple of 32: the whole problem is
    one dense run of blocks (the fast path used by the benchmark)."""
    rng = np.random.default_rng(13)
    for rows, cols in [(1, 32), (2, 32), (3, 64), (7, 96), (130, 4096), (33, 2048)]:
        say("dense quantize %s %s %dx%d" % (dtype, fmt, rows, cols))
        x = torch.from_numpy(rng.standard_normal((rows, cols)).astype(np.float32)).to(dtype)
        c, s = mxq.quantize(x.to(DEV), fmt, "row")
        oc, os_ = oracle_quantize(x, fmt, "row")
        assert_same(c.cpu().numpy(), s.cpu().numpy(), oc, os_, "dense %dx%d" % (rows, cols))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("axis", ["row", "col"])
def test_quantize_strided_and_unaligned(dtype, axis):
    """A view with a leading dimension that is not the row length, starting one element
    into the allocation (so 16-byte loads are impossible): the generic path."""
    rng = np.random.default_rng(11)
    base = torch.from_numpy(rng.standard_normal((70, 101)).astype(np.float32)).to(dtype)
    for view in (base[:, 1:97], base[3:, :64], base[:, 5:38]):
        gpu_base = base.to(DEV)
        sl = view
        # rebuild the same view on the device
        r0 = (sl.data_ptr() - base.data_ptr()) // base.element_size() // base.shape[1]
        c0 = (sl.data_ptr() - base.data_ptr()) // base.element_size() % base.shape[1]
        xg = gpu_base[r0:r0 + sl.shape[0], c0:c0 + sl.shape[1]]
        rows, cols = sl.shape
        L, K = (rows, cols) if axis == "row" else (cols, rows)
        Kp = 32 * ((K + 31) // 32)
        codes = torch.full((L, Kp + 32), 0xCD, dtype=torch.uint8, device=DEV)
        scales = torch.full((L, Kp // 32 + 1), 0xCD, dtype=torch.uint8, device=DEV)
        mxq.quantize(xg, "e4m3", axis, codes=codes, scales=scales)
        c = codes.cpu().numpy()
        s = scales.cpu().numpy()
        oc, os_ = oracle_quantize(sl.contiguous(), "e4m3", axis)
        assert np.all(c[:, Kp:] == 0xCD) and np.all(s[:, Kp // 32:] == 0xCD)
        assert_same(c[:, :Kp], s[:, :Kp // 32], oc, os_, "view %s" % (tuple(sl.shape),))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("axis", ["row", "col"])
def test_quantize_special_values(dtype, fmt, axis):
    """Zero blocks, signed zeros, NaN/Inf blocks, tiny blocks whose scale byte is 0 (the
    software-encoder branch), bf16/fp32 subnormals, exact rounding ties, spikes."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2, :32] = np.nan
    x[2, 40] = np.inf
    x[3, 70] = -np.inf
    x[4] = rng.standard_normal(256).astype(np.float32) * 1e-38          # scale byte 0
    x[5] = rng.standard_normal(256).astype(np.float32) * 1e-40          # subnormal inputs
    x[6, :] = 2.0 ** -133                                                # bf16 min subnormal
    x[7] = rng.standard_normal(256).astype(np.float32) * 3e38            # near FLT_MAX
    x[8, ::7] = 500.0                                                    # spikes
    d = 2.0 ** -9
    x[9, :32] = [448.0] + [0.5 * d * 448 / 448, 0.75 * d, -0.5 * d, 1.0625, 1.1875] * 6 + [0.0]
    x[10] = (rng.integers(-16, 16, 256) * 2.0 ** -4).astype(np.float32)  # many exact ties
    x[11, 1::2] = -x[11, 0::2]
    x[12, :] = -1e-30
    x[12, 0] = 1.0
    xt = torch.from_numpy(x).to(dtype)
    if axis == "col":
        xt = xt.t().contiguous()
    gc, gs = gpu_quantize(xt, fmt, axis)
    oc, os_ = oracle_quantize(xt, fmt, axis)
    assert_same(gc, gs, oc, os_, "special")


def test_quantize_empty_is_a_no_op():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    c, s = mxq.quantize(x, "e4m3", "row")
    assert c.shape == (0, 64) and s.shape == (0, 2)


def test_two_row_fixture_bytes():
    """The pages' two-row X and weight column: codes and scales on the GPU equal the oracle's
    (which are pinned to the printed reconstructions)."""
    from conftest import load_golden
    g = load_golden("two_row_projection.json")
    x = torch.tensor([g["pattern_small"] * 4, g["pattern_large"] * 4], dtype=torch.float32)
    w_kn = torch.tensor(g["weight_pattern"] * 4, dtype=torch.float32).reshape(32, 1)
    gc, gs = gpu_quantize(x, "e4m3", "row")
    assert [hex(v) for v in gs[:, 0]] == ["0x77", "0x80"]
    oc, os_ = oracle_quantize(x, "e4m3", "row")
    assert_same(gc, gs, oc, os_, "two-row X")
    wc, ws = gpu_quantize(w_kn, "e4m3", "col")
    oc, os_ = oracle_quantize(w_kn, "e4m3", "col")
    assert_same(wc, ws, oc, os_, "two-row W")


# ----------------------------------------------------------------- full-size workloads

def test_workload1_quantize():
    d = wl.workload1()
    for name, t, axis in (("X", d["x"], "row"), ("W colwise", d["w_kn"], "col"),
                          ("W^T rowwise", d["w_kn"].t().contiguous(), "row")):
        say("workload1 %s" % name)
        gc, gs = gpu_quantize(t, "e4m3", axis)
        oc, os_ = oracle_quantize(t, "e4m3", axis)
        assert_same(gc, gs, oc, os_, name)


def test_workload2_quantize():
    d = wl.workload2()
    for name in ("x", "w"):
        say("workload2 %s" % name)
        gc, gs = gpu_quantize(d[name], "e4m3", "row", pad_codes=0, pad_scales=0)
        oc, os_ = oracle_quantize(d[name], "e4m3", "row")
        assert_same(gc, gs, oc, os_, name)


def test_workload4_quantize_both_orientations():
    d = wl.workload4()
    jobs = (("dY row e5m2", d["dy"], "e5m2", "row"), ("dY col e5m2", d["dy"], "e5m2", "col"),
            ("X col e4m3", d["x"], "e4m3", "col"), ("W col e4m3", d["w"], "e4m3", "col"))
    for name, t, fmt, axis in jobs:
        say("workload4 %s" % name)
        gc, gs = gpu_quantize(t, fmt, axis, pad_codes=0, pad_scales=0)
        oc, os_ = oracle_quantize(t, fmt, axis)
        assert_same(gc, gs, oc, os_, name)


@pytest.mark.parametrize("K", [4000, 4001, 4031])
def test_workload5_quantize(K):
    d = wl.workload5(K=K, M=1024, N=64)
    say("workload5 K=%d" % K)
    gc, gs = gpu_quantize(d["x"], "e4m3", "row")
    oc, os_ = oracle_quantize(d["x"], "e4m3", "row")
    assert_same(gc, gs, oc, os_, "X K=%d" % K)
    # the 448 ceiling is reached: every block's largest element maps to the top codes
    assert np.mean((gc & 0x7F) == 0x7E) > 0.001


def test_standalone_quantize_2p28():
    d = wl.workload_q()
    for fmt, axis in (("e4m3", "row"), ("e5m2", "row"), ("e4m3", "col")):
        say("2^28 %s %s" % (fmt, axis))
        gc, gs = gpu_quantize(d["x"], fmt, axis, pad_codes=0, pad_scales=0)
        oc, os_ = oracle_quantize(d["x"], fmt, axis)
        assert_same(gc, gs, oc, os_, "2^28 %s %s" % (fmt, axis))
        del gc, gs, oc, os_


# ----------------------------------------------------------------- both orientations at once

def gpu_quantize_dual(x_cpu: torch.Tensor, fmt: str, pad=16, x_dev=None):
    """mxq_quantize_dual into canary-filled, over-wide outputs; checks the canaries and
    returns (row codes, row scales, col codes, col scales) trimmed to Kp and nb."""
    rows, cols = x_cpu.shape
    kr, kc = 32 * ((cols + 31) // 32), 32 * ((rows + 31) // 32)
    bufs = [torch.full(shape, 0xCD, dtype=torch.uint8, device=DEV)
            for shape in ((rows, kr + pad), (rows, kr // 32 + 3), (cols, kc + pad), (cols, kc // 32 + 3))]
    x = x_cpu.to(DEV) if x_dev is None else x_dev
    st = mxq.mxq_quantize_dual(x.data_ptr(), mxq._binding._wide_type(x), rows, cols, x.stride(0), mxq._binding._ELEM[fmt],
                               *[v for b in bufs for v in (b.data_ptr(), b.stride(0))],
                               mxq._binding._stream_handle())
    assert st == 0, mxq.mxq_status_string(st)
    torch.cuda.synchronize()
    rc, rs, cc, cs = (b.cpu().numpy() for b in bufs)
    assert np.all(rc[:, kr:] == 0xCD) and np.all(rs[:, kr // 32:] == 0xCD), "rowwise write past the end"
    assert np.all(cc[:, kc:] == 0xCD) and np.all(cs[:, kc // 32:] == 0xCD), "columnwise write past the end"
    return rc[:, :kr], rs[:, :kr // 32], cc[:, :kc], cs[:, :kc // 32]


def check_dual(x_cpu, fmt, what, **kw):
    rc, rs, cc, cs = gpu_quantize_dual(x_cpu, fmt, **kw)
    oc, os_ = oracle_quantize(x_cpu, fmt, "row")
    assert_same(rc, rs, oc, os_, what + " rowwise")
    oc, os_ = oracle_quantize(x_cpu, fmt, "col")
    assert_same(cc, cs, oc, os_, what + " columnwise")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_dual_shapes(dtype, fmt):
    """Ragged in both directions (partial 32-blocks, partial 128x64 tiles), tiny and
    several-tile shapes, column counts that do and do not allow 16-byte loads."""
    rng = np.random.default_rng(20)
    for rows, cols in SHAPES + [(128, 64), (129, 65), (300, 136), (257, 1000), (1000, 48)]:
        say("dual %s %s %dx%d" % (dtype, fmt, rows, cols))
        scale = np.exp2(rng.integers(-20, 20, (rows, 1))).astype(np.float32)
        x = torch.from_numpy(rng.standard_normal((rows, cols)).astype(np.float32) * scale).to(dtype)
        check_dual(x, fmt, "%dx%d" % (rows, cols))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_dual_special_values(dtype, fmt):
    """The special-value rows of test_quantize_special_values, which also put NaN, Inf,
    zero and tiny columns into the columnwise blocks."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((96, 256)).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2, :32] = np.nan
    x[2, 40] = np.inf
    x[3, 70] = -np.inf
    x[4] = rng.standard_normal(256).astype(np.float32) * 1e-38
    x[5] = rng.standard_normal(256).astype(np.float32) * 1e-40
    x[6, :] = 2.0 ** -133
    x[7] = rng.standard_normal(256).astype(np.float32) * 3e38
    x[8, ::7] = 500.0
    x[10] = (rng.integers(-16, 16, 256) * 2.0 ** -4).astype(np.float32)
    x[32:64, 100:132] = 1e-39                                            # a tiny columnwise block
    x[64:96, 200] = np.nan
    check_dual(torch.from_numpy(x).to(dtype), fmt, "special")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_dual_strided_and_unaligned(dtype):
    """Views whose leading dimension is not the row length, starting one element into the
    allocation (the path with element loads)."""
    rng = np.random.default_rng(22)
    base = torch.from_numpy(rng.standard_normal((170, 101)).astype(np.float32)).to(dtype)
    gpu_base = base.to(DEV)
    for r0, c0, rows, cols in ((0, 1, 170, 96), (3, 0, 140, 64), (1, 5, 130, 33)):
        say("dual view %d,%d %dx%d" % (r0, c0, rows, cols))
        view = base[r0:r0 + rows, c0:c0 + cols]
        check_dual(view.contiguous(), "e4m3", "view", x_dev=gpu_base[r0:r0 + rows, c0:c0 + cols])


def test_quantize_dual_matches_separate_calls_2p28():
    """The 2^28-element bf16 tensor: the fused call gives the same bytes as the rowwise and
    columnwise calls (which are checked against the oracle in test_standalone_quantize_2p28),
    so the fused kernel is pinned to the oracle at full size too."""
    d = wl.workload_q()
    x = d["x"].to(DEV)
    for fmt in ("e4m3", "e5m2"):
        say("dual 2^28 %s" % fmt)
        rc, rs, cc, cs = mxq.quantize_dual(x, fmt)
        c, s = mxq.quantize(x, fmt, "row")
        assert torch.equal(rc, c) and torch.equal(rs, s)
        c, s = mxq.quantize(x, fmt, "col")
        assert torch.equal(cc, c) and torch.equal(cs, s)
        del rc, rs, cc, cs, c, s


def test_workload4_quantize_dual():
    """The backward gradient dY in e5m2, both orientations, against the oracle."""
    d = wl.workload4()
    say("workload4 dual dY")
    check_dual(d["dy"], "e5m2", "dY", pad=0)


def test_quantize_dual_empty_is_a_no_op():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    rc, rs, cc, cs = mxq.quantize_dual(x)
    assert rc.shape == (0, 64) and cc.shape == (64, 0)


# ----------------------------------------------------------------- dequantize

@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K", [1, 29, 64, 200])
def test_dequantize_exact(fmt, out, K):
    rng = np.random.default_rng(K)
    L = 37
    Kp = 32 * ((K + 31) // 32)
    codes = rng.integers(0, 256, (L, Kp)).astype(np.uint8)
    scales = rng.integers(0, 256, (L, Kp // 32)).astype(np.uint8)
    scales[0, 0] = 255
    scales[1, 0] = 0
    scales[2, 0] = 254
    gc = torch.from_numpy(codes).to(DEV)
    gs = torch.from_numpy(scales).to(DEV)
    y = mxq.dequantize(gc, gs, K, fmt, out).cpu()
    ref = oracle.dequantize(codes, scales, fmt, K, "f32" if out == torch.float32 else "bf16")
    if out == torch.float32:
        a = y.numpy()
        assert np.array_equal(np.isnan(a), np.isnan(ref))
        m = ~np.isnan(ref)
        assert np.array_equal(a[m].view(np.uint32), ref[m].view(np.uint32))
    else:
        a = y.view(torch.int16).numpy().view(np.uint16)
        nan_a = (a & 0x7FFF) > 0x7F80
        nan_r = (ref & 0x7FFF) > 0x7F80
        assert np.array_equal(nan_a, nan_r)
        assert np.array_equal(a[~nan_r], ref[~nan_r])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_dequantize_layouts(fmt, out):
    """Leading dimensions through the C ABI: code rows holding only K bytes (the
    element-wise path), padded code rows with an output row wider than K (the block path
    with a partial last block: nothing is written past K), and a dense array of 2^20
    elements (the flat block path); every element bitwise against the oracle."""
    import ctypes
    rng = np.random.default_rng(90)
    es = 4 if out == torch.float32 else 2
    wide = mxq.MXQ_F32 if out == torch.float32 else mxq.MXQ_BF16
    for L, K, ld_c, ld_d in ((33, 40, 40, 40), (33, 40, 48, 48), (33, 40, 64, 48), (21, 100, 128, 104),
                             (1024, 1024, 1024, 1024)):
        say("dequantize layout %s %s L=%d K=%d ld_codes=%d ld_dst=%d" % (fmt, out, L, K, ld_c, ld_d))
        nb = (K + 31) // 32
        codes = rng.integers(0, 256, (L, ld_c)).astype(np.uint8)
        scales = rng.integers(100, 160, (L, nb)).astype(np.uint8)
        scales[0, 0], scales[-1, -1] = 255, 0
        gc, gs = torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV)
        canary = -7.0 if out == torch.float32 else -7.0
        dst = torch.full((L, ld_d), canary, dtype=out, device=DEV)
        st = mxq.mxq_dequantize(gc.data_ptr(), ld_c, gs.data_ptr(), nb, mxq.MXQ_E4M3 if fmt == "e4m3" else mxq.MXQ_E5M2,
                                L, K, dst.data_ptr(), wide, ld_d, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0
        torch.cuda.synchronize()
        y = dst.cpu()
        assert torch.all(y[:, K:] == canary), "write past K"
        ref = oracle.dequantize(np.ascontiguousarray(codes[:, :K]), scales, fmt, K, "f32" if es == 4 else "bf16")
        a = y[:, :K].contiguous()
        if es == 4:
            a = a.numpy()
            assert np.array_equal(np.isnan(a), np.isnan(ref))
            m = ~np.isnan(ref)
            assert np.array_equal(a[m].view(np.uint32), ref[m].view(np.uint32))
        else:
            a = a.view(torch.int16).numpy().view(np.uint16)
            nan_r = (ref & 0x7FFF) > 0x7F80
            assert np.array_equal((a & 0x7FFF) > 0x7F80, nan_r)
            assert np.array_equal(a[~nan_r], ref[~nan_r])


def test_quantize_dequantize_roundtrip_two_row():
    from conftest import load_golden
    g = load_golden("two_row_projection.json")
    x = torch.tensor([g["pattern_small"] * 4, g["pattern_large"] * 4], dtype=torch.float32, device=DEV)
    c, s = mxq.quantize(x, "e4m3", "row")
    xh = mxq.dequantize(c, s, 32, "e4m3").cpu().numpy()
    assert "%.8f" % xh[0, 0] == "%.8f" % g["printed"]["x00"]["mxfp8"]
    assert xh[1, 3] == g["printed"]["x13"]["mxfp8"]

"""Seeded random sweep of the quantize kernels against the CPU oracle, byte for byte: random
shapes (ragged in both dimensions, up to a few thousand), bf16 or fp32 sources with padded
row pitches (aligned pitches take the LDS-staged columnwise kernels, others the direct
ones), E4M3 / E5M2, rowwise and columnwise, the pages' scale rule and the OCP rule, values
spread over many binades with zeros, signed zeros, outliers and a few all-zero blocks;
then, on the same inputs, the dual-orientation quantize, the stochastically rounded codes
(E5M2) and the dequantized reconstruction of the GPU's own codes."""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_block_scaled_03_amd as mxq
from gpu_helpers import host_src, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CASES = 30


def source(rng, rows, cols, dtype, pad):
    """Values of mixed magnitudes in a [rows][cols + pad] buffer; returns the [rows][cols]
    view on the GPU and its CPU copy."""
    mag = 10.0 ** rng.uniform(-8, 8, size=(rows, 1)) * 10.0 ** rng.uniform(-2, 2, size=(rows, cols))
    v = (rng.standard_normal((rows, cols)) * mag).astype(np.float32)
    v[rng.random((rows, cols)) < 0.03] = 0.0
    v[rng.random((rows, cols)) < 0.01] = -0.0
    v[rng.random((rows, cols)) < 0.002] *= 1e4                       # outliers
    if rows >= 32 and cols >= 32 and rng.random() < 0.5:
        r0, c0 = int(rng.integers(0, rows - 31)), int(rng.integers(0, cols - 31))
        v[r0:r0 + 32, c0:c0 + 32] = 0.0                               # all-zero blocks
    t = torch.from_numpy(v).to(dtype)
    buf = torch.zeros((rows, cols + pad), dtype=dtype, device=DEV)
    buf[:, :cols].copy_(t.to(DEV))
    return buf[:, :cols], t


def same(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    if not np.array_equal(a, b):
        i = np.argwhere(a != b)[0]
        raise AssertionError("%s: mismatch at %s gpu=%d oracle=%d" % (what, i.tolist(), a[tuple(i)], b[tuple(i)]))


@pytest.mark.parametrize("case", range(CASES))
def test_quantize_random_sweep(case):
    rng = np.random.default_rng(9000 + case)
    big = case % 5 == 0
    rows = int(rng.integers(1, 3000 if big else 400))
    cols = int(rng.integers(1, 3000 if big else 400))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    fmt = str(rng.choice(["e4m3", "e5m2"]))
    rule = "ocp" if rng.random() < 0.25 else "ceil"
    step = 8 if dtype == torch.bfloat16 else 4                      # 16-byte row pieces
    pad = int(rng.integers(0, 3)) * step if rng.random() < 0.6 else int(rng.integers(1, 9))
    if rng.random() < 0.5:                                          # whole 16-byte rows
        cols = max(step, cols - cols % step)
    say("quantize sweep %d: %dx%d %s %s rule=%s pad=%d" % (case, rows, cols, dtype, fmt, rule, pad))
    x, x_cpu = source(rng, rows, cols, dtype, pad)
    src = host_src(x_cpu)
    for axis in ("row", "col"):
        c, s = mxq.quantize(x, fmt, axis, rule=rule)
        oc, os_ = oracle.quantize(src, fmt, axis=0 if axis == "row" else 1, rule=rule)
        torch.cuda.synchronize()
        same(s.cpu().numpy(), os_, "case %d %s scales" % (case, axis))
        same(c.cpu().numpy(), oc, "case %d %s codes" % (case, axis))
        # the reconstruction of the GPU's own codes
        K = cols if axis == "row" else rows
        for out in ("f32", "bf16"):
            d = mxq.dequantize(c, s, K, fmt, out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
            od = oracle.dequantize(c.cpu().numpy(), s.cpu().numpy(), fmt, K, out=out)
            dg = d.cpu().contiguous()
            dg = dg.numpy() if out == "f32" else dg.view(torch.int16).numpy().view(np.uint16)
            same(dg.view(np.uint32) if out == "f32" else dg, od.view(np.uint32) if out == "f32" else od,
                 "case %d %s dequantize %s" % (case, axis, out))
    if rule == "ceil":
        rc, rs, cc, cs = mxq.quantize_dual(x, fmt)
        orc, ors = oracle.quantize(src, fmt, axis=0)
        occ, ocs = oracle.quantize(src, fmt, axis=1)
        torch.cuda.synchronize()
        same(rs.cpu().numpy(), ors, "case %d dual row scales" % case)
        same(rc.cpu().numpy(), orc, "case %d dual row codes" % case)
        same(cs.cpu().numpy(), ocs, "case %d dual col scales" % case)
        same(cc.cpu().numpy(), occ, "case %d dual col codes" % case)
        seed = int(rng.integers(0, 2 ** 63))
        axis = str(rng.choice(["row", "col"]))
        c, s = mxq.quantize_sr(x, seed, "e5m2", axis)
        oc, os_ = oracle.quantize_sr(src, "e5m2", seed, axis=0 if axis == "row" else 1)
        torch.cuda.synchronize()
        same(s.cpu().numpy(), os_, "case %d sr %s scales" % (case, axis))
        same(c.cpu().numpy(), oc, "case %d sr %s codes" % (case, axis))

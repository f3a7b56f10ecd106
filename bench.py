"""Benchmark of the MXFP8 hot path on one MI355X.

One step = the whole path over one batch of the projection workload (M=8192, K=4096,
N=4096, bf16 activations ~N(0,1) with 0.1% outliers x100, bf16 weights ~N(0,0.02)):
    mxq_quantize(X) rowwise E4M3 -> mxq_quantize(W) rowwise E4M3 -> mxq_gemm (bf16 out)
with the GEMM in its exact-product accumulation mode (MXQ_ACC_FP32), the mode that meets
the per-element bound |Y - Y_ref| <= 1e-5 * sum_k |s x w|.  Inputs are resident in HBM
before timing starts.  `value` is the whole step's throughput, 2*M*N*K / step time, in
TFLOP/s.  The dominant kernel (the GEMM) is also timed on its own with HIP events around
each of its launches inside the timed region (the events sit on the stream the kernels
are launched on) and reported against the dense MXFP8 matrix-core peak, with its fraction
of the dense bf16 peak (the matrix cores it runs on) beside it.  The FP8 matrix-core mode
(MXQ_ACC_FP8_MFMA), whose 8-product groups are truncated and which does not meet that
bound, is timed only as a labelled component.  The standalone quantize of 2^28 bf16
elements is reported against the HBM peak.  The CPU oracle is timed on a bounded sample
of the same step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms T] [--no-cpu]
                       [--copy-calibration] [--headline-only] [--only KERNEL]

Before the W warmup steps the step runs untimed, in blocks of 20, for at least T ms of
wall time (default 150; 0 skips it): the clock of a GPU that was idle rises over the first
~40 ms of sustained load, and the timed steps should see the sustained rate.  The JSON
line reports these steps under "settle".

--headline-only times the step alone (no components, no CPU leg): the short run that
counter passes profile.

--only quantize_2p28 | quantize_2p28_colwise | quantize_2p28_dual runs that one quantize
launch on the [16384][16384] bf16 input, W untimed then K timed, and prints its time and
GB/s; --only gemm_exact | gemm_fp8 runs that GEMM mode alone on the projection workload
(the short runs that the kernels' counter passes profile).

--copy-calibration adds a plain elementwise copy of a known size (256 MiB read, 256 MiB
written) after the measurement, so that one hardware-counter run sees both the GEMM and a
kernel whose HBM traffic is known; the ratio calibrates FETCH_SIZE / WRITE_SIZE.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MXFP8_TFLOPS = 5000.0      # MI355X dense FP8 / MXFP8 matrix-core peak
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 matrix-core peak (the exact-product mode's MFMAs)
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle-ms", type=float, default=150.0,
                   help="untimed steps before the warmup, for at least this much wall time (0: none)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-oracle sample time")
    p.add_argument("--copy-calibration", action="store_true", help="also run a copy of known size (counter runs)")
    p.add_argument("--headline-only", action="store_true", help="time the step only (counter runs)")
    p.add_argument("--only", choices=sorted(ONLY_KERNELS), default=None,
                   help="time one kernel alone: a quantize entry point on the 2^28 input, a GEMM mode on the "
                        "projection, or a torch reference kernel (counter runs, ceilings)")
    return p.parse_args()


# --only: one quantize entry point on the [16384][16384] bf16 input, E4M3, or one GEMM
# mode on the projection workload
ONLY_KERNELS = {"quantize_2p28": "rowwise", "quantize_2p28_colwise": "colwise", "quantize_2p28_dual": "dual",
                "gemm_exact": "exact", "gemm_fp8": "fp8",
                # practical ceilings on the same machine, from torch's own kernels (context only):
                # an elementwise bf16 -> int8 cast and a bf16 copy of the 2^28 input (the byte mixes
                # of one and two quantize orientations), and torch.mm on bf16 operands of the
                # projection shape (the library GEMM on the matrix cores the exact mode uses)
                "ref_cast_2p28": "ref_cast", "ref_copy_2p28": "ref_copy", "ref_mm_bf16": "ref_mm"}


_CSRC = os.path.join(ROOT, "mxfp8_block_scaled_03_amd", "csrc")
# the sources a recorded HBM-traffic measurement was taken on, per kernel
KERNEL_SOURCES = {
    "gemm_exact": [os.path.join(_CSRC, "gemm_exact.hip"), os.path.join(_CSRC, "gemm_common.hpp")],
    "gemm_fp8": [os.path.join(_CSRC, "gemm_fp8.hip"), os.path.join(_CSRC, "gemm_common.hpp")],
}
GEMM_KERNEL_NAME = "mxq gemm, exact-product mode (ex::k_gemm_ex<0,0,256>: codes decoded to bf16 in registers, bf16 matrix cores)"
FP8_LABEL = "FP8 matrix cores, 8-product groups truncated ~13 bits below their largest (outside 1e-5*T)"


def settle(torch, fn, ms: float, block: int = 10) -> int:
    """Runs fn untimed, in blocks of `block` calls, until `ms` of wall time have passed (the
    clock of a GPU that was idle rises over the first tens of ms of sustained load); returns
    the number of calls (0 when ms <= 0)."""
    n, t = 0, time.perf_counter()
    while (time.perf_counter() - t) * 1e3 < ms:
        for _ in range(block):
            fn()
        torch.cuda.synchronize()
        n += block
    return n


def source_digest(paths) -> str:
    """sha256 over the bytes of the given source files, in order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(kernel: str):
    """HBM bytes per launch of `kernel` measured with rocprofv3 counters (profiles/), or
    None when there is no measurement or the kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[kernel]
        if t.get("source_sha256") != source_digest(KERNEL_SOURCES[kernel]):
            return None
        return int(t["bytes_per_launch"])
    except (OSError, ValueError, KeyError, TypeError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp8_block_scaled_03_amd as mxq
    from mxfp8_block_scaled_03_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mxq.lib()
    if args.only:
        if args.only.startswith("ref_"):
            only_reference(args, torch, wl, dev)
        elif args.only.startswith("gemm"):
            only_gemm(args, torch, mxq, wl, dev)
        else:
            only_quantize(args, torch, mxq, wl, dev)
        return

    d = wl.workload2()
    M, K, N = d["M"], d["K"], d["N"]
    x = d["x"].to(dev)
    w = d["w"].to(dev)
    Kp = 32 * ((K + 31) // 32)
    xc = torch.empty((M, Kp), dtype=torch.uint8, device=dev)
    xs = torch.empty((M, Kp // 32), dtype=torch.uint8, device=dev)
    wc = torch.empty((N, Kp), dtype=torch.uint8, device=dev)
    ws = torch.empty((N, Kp // 32), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    # The step calls the C entry points directly with arguments prepared once, so the host
    # enqueues far faster than the GPU runs and no host gap lands between the events.
    import ctypes
    L = mxq.lib()
    sh = ctypes.c_void_p(stream.cuda_stream)
    q_x = (x.data_ptr(), mxq.MXQ_BF16, M, K, x.stride(0), mxq.MXQ_ROWWISE, mxq.MXQ_E4M3, xc.data_ptr(), xc.stride(0),
           xs.data_ptr(), xs.stride(0), sh)
    q_w = (w.data_ptr(), mxq.MXQ_BF16, N, K, w.stride(0), mxq.MXQ_ROWWISE, mxq.MXQ_E4M3, wc.data_ptr(), wc.stride(0),
           ws.data_ptr(), ws.stride(0), sh)
    g_args = (M, N, K, xc.data_ptr(), xc.stride(0), xs.data_ptr(), xs.stride(0), mxq.MXQ_E4M3, wc.data_ptr(),
              wc.stride(0), ws.data_ptr(), ws.stride(0), mxq.MXQ_E4M3, ctypes.c_float(1.0), None, y.data_ptr(),
              mxq.MXQ_BF16, y.stride(0), mxq.MXQ_ACC_FP32, sh)
    for a in (L.mxq_quantize(*q_x), L.mxq_quantize(*q_w), L.mxq_gemm(*g_args)):
        if a != 0:
            raise RuntimeError("mxq call failed: %s" % mxq.mxq_status_string(a))

    def step(ev=None):
        L.mxq_quantize(*q_x)
        L.mxq_quantize(*q_w)
        if ev is not None:
            ev[0].record(stream)
        L.mxq_gemm(*g_args)
        if ev is not None:
            ev[1].record(stream)

    # an idle GPU's clock rises over the first ~40 ms of sustained load (the GEMM from a
    # cold start: 242, 228, 223, ... 211 us per call in blocks of 20 calls), so the step
    # runs untimed for --settle-ms of wall time before the warmup steps
    t_settle = time.perf_counter()
    settle_steps = settle(torch, step, args.settle_ms, 20)
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    gemm_events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(gemm_events[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    gemm_ms = [a.elapsed_time(b) for a, b in gemm_events]
    gemm_ms_avg = sum(gemm_ms) / len(gemm_ms)
    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms_avg * 1e-3) / 1e12
    gemm_bytes = (M + N) * Kp * (1 + 1 / 32) + M * N * 2

    out = {
        "metric": "MXFP8 GEMM TFLOP/s (% dense MFMA peak); mx_quantize GB/s (% HBM peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"steps": settle_steps, "ms": round(settle_ms, 1),
                   "why": "untimed steps before the warmup until the clock of an idle GPU has risen"},
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 codes (MXFP8, E8M0 block scales); exact products, fp32 accumulate "
                 "(codes decoded with their scale to bf16, bf16 matrix cores)",
        "data": "synthetic",
        "config": {"workload": "projection GEMM M=8192 K=4096 N=4096: bf16 X ~N(0,1) with 0.1% x100, "
                               "bf16 W ~N(0,0.02); quantize X and W rowwise to MXFP8 E4M3, GEMM with bf16 output",
                   "M": M, "K": K, "N": N, "step": "quantize(X) + quantize(W) + gemm (exact-product accumulation)"},
        "roofline": {"bound": "mfma", "kernel": GEMM_KERNEL_NAME,
                     "achieved": round(gemm_tflops, 2), "peak": PEAK_MXFP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_MXFP8_TFLOPS, 4),
                     "frac_of_bf16_peak": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic("gemm_exact"), "algorithmic_bytes": int(gemm_bytes),
                     "ms_avg": round(gemm_ms_avg, 5)},
    }
    if args.headline_only:
        if args.copy_calibration:
            copy_calibration(torch, dev)
        print(json.dumps(out))
        return

    # ---- the same GEMM on the FP8 matrix cores (outside the 1e-5*T bound: each group of 8
    #      products is aligned to its largest and truncated ~13 bits below it)
    yf = torch.empty_like(y)
    gf_args = list(g_args)
    gf_args[15] = yf.data_ptr()
    gf_args[18] = mxq.MXQ_ACC_FP8_MFMA
    comp_settle_ms = args.settle_ms / 2          # each component runs untimed this long first
    settle(torch, lambda: L.mxq_gemm(*gf_args), comp_settle_ms)
    ee = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a, b in ee:
        a.record(stream)
        L.mxq_gemm(*gf_args)
        b.record(stream)
    torch.cuda.synchronize()
    fp8_ms = sum(a.elapsed_time(b) for a, b in ee) / len(ee)
    fp8_tflops = flops / (fp8_ms * 1e-3) / 1e12
    del yf

    # ---- standalone quantize: 2^28 bf16 elements, rowwise E4M3 (HBM-bound)
    q = wl.workload_q()
    qx = q["x"].to(dev)
    del q
    qc = torch.empty((qx.shape[0], qx.shape[1]), dtype=torch.uint8, device=dev)
    qs = torch.empty((qx.shape[0], qx.shape[1] // 32), dtype=torch.uint8, device=dev)
    q_q = (qx.data_ptr(), mxq.MXQ_BF16, qx.shape[0], qx.shape[1], qx.stride(0), mxq.MXQ_ROWWISE, mxq.MXQ_E4M3,
           qc.data_ptr(), qc.stride(0), qs.data_ptr(), qs.stride(0), sh)
    L.mxq_quantize(*q_q)
    settle(torch, lambda: L.mxq_quantize(*q_q), comp_settle_ms)
    nq = 20
    qe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nq)]
    for a, b in qe:
        a.record(stream)
        L.mxq_quantize(*q_q)
        b.record(stream)
    torch.cuda.synchronize()
    q_ms = sum(a.elapsed_time(b) for a, b in qe) / nq
    q_bytes = qx.numel() * (2 + 1 + 1 / 32)
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9

    # secondary quantize rows on the same 2^28 input: rowwise E5M2, columnwise E4M3
    # (codes [cols][rows]), and dequantize of the rowwise codes back to bf16
    def time_calls(fn, n=10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        settle(torch, fn, comp_settle_ms)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    q_e5 = list(q_q)
    q_e5[6] = mxq.MXQ_E5M2
    e5_ms = time_calls(lambda: L.mxq_quantize(*q_e5))
    q_col = list(q_q)
    q_col[5] = mxq.MXQ_COLWISE
    col_ms = time_calls(lambda: L.mxq_quantize(*q_col))
    # stochastically rounded E5M2 (gradients): same bytes, Philox random numbers per element
    q_sr = (qx.data_ptr(), mxq.MXQ_BF16, qx.shape[0], qx.shape[1], qx.stride(0), mxq.MXQ_ROWWISE, mxq.MXQ_E5M2,
            ctypes.c_uint64(20261202), qc.data_ptr(), qc.stride(0), qs.data_ptr(), qs.stride(0), sh)
    if L.mxq_quantize_sr(*q_sr) != 0:
        raise RuntimeError("mxq_quantize_sr failed")
    sr_ms = time_calls(lambda: L.mxq_quantize_sr(*q_sr))
    # both orientations from one read of the tensor (rowwise into qc/qs, columnwise into
    # separate [cols][rows] outputs): 2 B read + 2 x (1 + 1/32) B written per element
    dc = torch.empty((qx.shape[1], qx.shape[0]), dtype=torch.uint8, device=dev)
    ds = torch.empty((qx.shape[1], qx.shape[0] // 32), dtype=torch.uint8, device=dev)
    q_dual = (qx.data_ptr(), mxq.MXQ_BF16, qx.shape[0], qx.shape[1], qx.stride(0), mxq.MXQ_E4M3, qc.data_ptr(),
              qc.stride(0), qs.data_ptr(), qs.stride(0), dc.data_ptr(), dc.stride(0), ds.data_ptr(), ds.stride(0), sh)
    dual_ms = time_calls(lambda: L.mxq_quantize_dual(*q_dual))
    dual_bytes = qx.numel() * (2 + 2 * (1 + 1 / 32))
    del dc, ds
    dq = torch.empty_like(qx)
    dq_args = (qc.data_ptr(), qc.stride(0), qs.data_ptr(), qs.stride(0), mxq.MXQ_E4M3, qx.shape[0], qx.shape[1],
               dq.data_ptr(), mxq.MXQ_BF16, dq.stride(0), sh)
    L.mxq_quantize(*q_q)
    dq_ms = time_calls(lambda: L.mxq_dequantize(*dq_args))
    dq_bytes = qx.numel() * (1 + 1 / 32 + 2)
    del qx, qc, qs, dq

    # quantize of the step's X alone (8192 x 4096 bf16)
    # X alone: 20 launches between two events (a single launch is short enough that the
    # host could fall behind the GPU)
    xa, xb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settle(torch, lambda: L.mxq_quantize(*q_x), comp_settle_ms)
    xa.record(stream)
    for _ in range(20):
        L.mxq_quantize(*q_x)
    xb.record(stream)
    torch.cuda.synchronize()
    xq_ms = xa.elapsed_time(xb) / 20
    xq_gbs = M * K * (2 + 1 + 1 / 32) / (xq_ms * 1e-3) / 1e9

    # ---- FFN up projection with bias and SiLU (T=16384, H=5120, I=8192).  Unfused: the GEMM
    #      writes bf16 Y1, then the rowwise quantize of Y1 that the down projection consumes.
    #      Fused: the GEMM epilogue writes Y1's MX codes and scales directly (same bytes).
    d3 = wl.workload3()
    T3, H3, I3 = d3["T"], d3["H"], d3["I"]
    f_xc, f_xs = mxq.quantize(d3["x"].to(dev), "e4m3", "row")
    f_wc, f_ws = mxq.quantize(d3["w1"].to(dev), "e4m3", "row")
    f_b = d3["b1"].to(dev)
    del d3
    y1 = torch.empty((T3, I3), dtype=torch.bfloat16, device=dev)
    y1c = torch.empty((T3, I3), dtype=torch.uint8, device=dev)
    y1s = torch.empty((T3, I3 // 32), dtype=torch.uint8, device=dev)

    def up_args(yp, yld, qc, qld, qs, qsld, acc=mxq.MXQ_ACC_FP32):
        return (T3, I3, H3, f_xc.data_ptr(), f_xc.stride(0), f_xs.data_ptr(), f_xs.stride(0), mxq.MXQ_E4M3,
                f_wc.data_ptr(), f_wc.stride(0), f_ws.data_ptr(), f_ws.stride(0), mxq.MXQ_E4M3, ctypes.c_float(1.0),
                f_b.data_ptr(), mxq.MXQ_ACT_SILU, yp, mxq.MXQ_BF16, yld, mxq.MXQ_E4M3, qc, qld, qs, qsld, acc, sh)
    up_unfused = up_args(y1.data_ptr(), y1.stride(0), None, 0, None, 0)
    q_y1 = (y1.data_ptr(), mxq.MXQ_BF16, T3, I3, y1.stride(0), mxq.MXQ_ROWWISE, mxq.MXQ_E4M3, y1c.data_ptr(),
            y1c.stride(0), y1s.data_ptr(), y1s.stride(0), sh)
    up_fused = up_args(None, 0, y1c.data_ptr(), y1c.stride(0), y1s.data_ptr(), y1s.stride(0))
    up_fused_fp8 = up_args(None, 0, y1c.data_ptr(), y1c.stride(0), y1s.data_ptr(), y1s.stride(0),
                           mxq.MXQ_ACC_FP8_MFMA)
    for a in (L.mxq_gemm_ex(*up_unfused), L.mxq_quantize(*q_y1), L.mxq_gemm_ex(*up_fused_fp8),
              L.mxq_gemm_ex(*up_fused)):
        if a != 0:
            raise RuntimeError("mxq call failed: %s" % mxq.mxq_status_string(a))

    def unfused_pair():
        L.mxq_gemm_ex(*up_unfused)
        L.mxq_quantize(*q_y1)
    up_gemm_ms = time_calls(lambda: L.mxq_gemm_ex(*up_unfused))
    up_unfused_ms = time_calls(unfused_pair)
    up_fused_fp8_ms = time_calls(lambda: L.mxq_gemm_ex(*up_fused_fp8))
    up_fused_ms = time_calls(lambda: L.mxq_gemm_ex(*up_fused))
    up_flops = 2.0 * T3 * I3 * H3

    # ---- the other configurations' GEMMs, each timed in both accumulation modes (raw C
    #      calls, 10 launches between two events).  FFN down consumes the fused up
    #      projection's Y1 codes; backward dgrad/wgrad use E5M2 gradient codes; K=4000 runs
    #      the kernel with a masked last K step; the 256x256x512 case is launch-bound.
    def gemm_args(Mg, Ng, Kg, a, b, fa, fb, yt, ydt, bias=None):
        (ac, as_), (bc, bs) = a, b
        return [Mg, Ng, Kg, ac.data_ptr(), ac.stride(0), as_.data_ptr(), as_.stride(0), fa, bc.data_ptr(), bc.stride(0),
                bs.data_ptr(), bs.stride(0), fb, ctypes.c_float(1.0), None if bias is None else bias.data_ptr(),
                yt.data_ptr(), ydt, yt.stride(0), mxq.MXQ_ACC_FP32, sh]

    def time_gemm(name, ga, flops_g):
        res = {"M": ga[0], "N": ga[1], "K": ga[2]}
        for acc, key in ((mxq.MXQ_ACC_FP32, ""), (mxq.MXQ_ACC_FP8_MFMA, "fp8_truncated_")):
            ga[18] = acc
            st = L.mxq_gemm(*ga)
            if st != 0:
                raise RuntimeError("%s gemm failed: %s" % (name, mxq.mxq_status_string(st)))
            ms_g = time_calls(lambda: L.mxq_gemm(*ga))
            res[key + "ms"] = round(ms_g, 5)
            res[key + "tflops"] = round(flops_g / (ms_g * 1e-3) / 1e12, 2)
        res["frac_of_mxfp8_peak"] = round(res["tflops"] / PEAK_MXFP8_TFLOPS, 4)
        res["frac_of_bf16_peak"] = round(res["tflops"] / PEAK_BF16_TFLOPS, 4)
        res["fp8_truncated_frac_of_mxfp8_peak"] = round(res["fp8_truncated_tflops"] / PEAK_MXFP8_TFLOPS, 4)
        return res

    configs = {}
    d3 = wl.workload3()
    w2q = mxq.quantize(d3["w2"].to(dev), "e4m3", "row")
    b2 = d3["b2"].to(dev)
    del d3
    y2 = torch.empty((T3, H3), dtype=torch.bfloat16, device=dev)
    configs["ffn_down_16384x5120x8192_bias_bf16"] = time_gemm(
        "ffn down", gemm_args(T3, H3, I3, (y1c, y1s), w2q, mxq.MXQ_E4M3, mxq.MXQ_E4M3, y2, mxq.MXQ_BF16, b2),
        2.0 * T3 * H3 * I3)
    del f_xc, f_xs, f_wc, f_ws, f_b, y1, y1c, y1s, w2q, b2, y2

    d4 = wl.workload4()
    M4, K4, N4 = d4["M"], d4["K"], d4["N"]
    dy_row = mxq.quantize(d4["dy"].to(dev), "e5m2", "row")       # [M][N] along N
    w_col = mxq.quantize(d4["w"].to(dev), "e4m3", "col")         # W [N][K] -> [K][N] along N
    dx = torch.empty((M4, K4), dtype=torch.float32, device=dev)
    configs["dgrad_8192x4096x4096_e5m2xe4m3_fp32"] = time_gemm(
        "dgrad", gemm_args(M4, K4, N4, dy_row, w_col, mxq.MXQ_E5M2, mxq.MXQ_E4M3, dx, mxq.MXQ_F32),
        2.0 * M4 * K4 * N4)
    del dy_row, w_col, dx
    dy_col = mxq.quantize(d4["dy"].to(dev), "e5m2", "col")       # [N][M] along M
    x_col = mxq.quantize(d4["x"].to(dev), "e4m3", "col")         # [K][M] along M
    dw = torch.empty((N4, K4), dtype=torch.float32, device=dev)
    configs["wgrad_4096x4096x8192_e5m2xe4m3_fp32"] = time_gemm(
        "wgrad", gemm_args(N4, K4, M4, dy_col, x_col, mxq.MXQ_E5M2, mxq.MXQ_E4M3, dw, mxq.MXQ_F32),
        2.0 * N4 * K4 * M4)
    del d4, dy_col, x_col, dw

    d5 = wl.workload5()
    M5, K5, N5 = d5["M"], d5["K"], d5["N"]
    x5 = mxq.quantize(d5["x"].to(dev), "e4m3", "row")
    w5 = mxq.quantize(d5["w"].to(dev), "e4m3", "row")
    del d5
    y5 = torch.empty((M5, N5), dtype=torch.float32, device=dev)
    configs["ragged_4096x6144x4000_fp32"] = time_gemm(
        "ragged", gemm_args(M5, N5, K5, x5, w5, mxq.MXQ_E4M3, mxq.MXQ_E4M3, y5, mxq.MXQ_F32), 2.0 * M5 * N5 * K5)
    del x5, w5, y5

    d1 = wl.workload1()
    M1, K1, N1 = d1["M"], d1["K"], d1["N"]
    x1 = mxq.quantize(d1["x"].to(dev), "e4m3", "row")
    w1 = mxq.quantize(d1["w_kn"].to(dev), "e4m3", "col")
    del d1
    y1f = torch.empty((M1, N1), dtype=torch.float32, device=dev)
    configs["small_256x256x512_fp32_launch_bound"] = time_gemm(
        "small", gemm_args(M1, N1, K1, x1, w1, mxq.MXQ_E4M3, mxq.MXQ_E4M3, y1f, mxq.MXQ_F32), 2.0 * M1 * N1 * K1)
    del x1, w1, y1f

    out["components"] = {
        "gemm_fp8_truncated": {"ms": round(fp8_ms, 5), "tflops": round(fp8_tflops, 2),
                               "frac_of_mxfp8_peak": round(fp8_tflops / PEAK_MXFP8_TFLOPS, 4),
                               "accum": FP8_LABEL, "traffic": load_traffic("gemm_fp8")},
        "quantize_x": {"ms": round(xq_ms, 5), "gbs": round(xq_gbs, 1), "bytes": int(M * K * 3.03125)},
        "quantize_2p28_e5m2": {"ms": round(e5_ms, 5), "gbs": round(q_bytes / (e5_ms * 1e-3) / 1e9, 1)},
        "quantize_2p28_colwise": {"ms": round(col_ms, 5), "gbs": round(q_bytes / (col_ms * 1e-3) / 1e9, 1)},
        "quantize_2p28_sr_e5m2": {"ms": round(sr_ms, 5), "gbs": round(q_bytes / (sr_ms * 1e-3) / 1e9, 1),
                                  "rounding": "stochastic (Philox4x32-10)"},
        "quantize_2p28_dual": {"ms": round(dual_ms, 5), "gbs": round(dual_bytes / (dual_ms * 1e-3) / 1e9, 1),
                               "vs_two_calls_ms": round(q_ms + col_ms, 5)},
        "dequantize_2p28_bf16": {"ms": round(dq_ms, 5), "gbs": round(dq_bytes / (dq_ms * 1e-3) / 1e9, 1)},
        "ffn_up_silu_unfused": {"ms": round(up_unfused_ms, 5), "gemm_ms": round(up_gemm_ms, 5),
                                "gemm_tflops": round(up_flops / (up_gemm_ms * 1e-3) / 1e12, 2),
                                "what": "T=16384 H=5120 I=8192 exact-product GEMM (bias, SiLU, bf16 Y1) "
                                        "+ quantize(Y1)"},
        "ffn_up_silu_fused": {"ms": round(up_fused_ms, 5),
                              "tflops": round(up_flops / (up_fused_ms * 1e-3) / 1e12, 2),
                              "speedup_vs_unfused": round(up_unfused_ms / up_fused_ms, 3),
                              "fp8_truncated_ms": round(up_fused_fp8_ms, 5),
                              "what": "same exact-product GEMM writing Y1's MX codes and scales from its epilogue"},
        "configs": configs,
        "quantize_2p28": {"ms": round(q_ms, 5), "gbs": round(q_gbs, 1), "frac_hbm": round(q_gbs / PEAK_HBM_GBS, 4),
                          "bytes": int(q_bytes), "workload": "[16384][16384] bf16 Laplace(0,1) 1% x1e4, rowwise E4M3"},
    }

    if args.copy_calibration:
        copy_calibration(torch, dev)

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(d, xc, xs, wc, ws, M, N, K, args.cpu_seconds)
    print(json.dumps(out))


def only_quantize(args, torch, mxq, wl, dev):
    """One quantize entry point alone on the 2^28-element input: bytes moved per launch are
    2 B read + (1 + 1/32) B written per element and orientation."""
    import ctypes
    L = mxq.lib()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    qx = wl.workload_q()["x"].to(dev)
    R, C = qx.shape
    kind = ONLY_KERNELS[args.only]
    rc = torch.empty((R, C), dtype=torch.uint8, device=dev)
    rs = torch.empty((R, C // 32), dtype=torch.uint8, device=dev)
    if kind == "dual":
        cc = torch.empty((C, R), dtype=torch.uint8, device=dev)
        cs = torch.empty((C, R // 32), dtype=torch.uint8, device=dev)
        a = (qx.data_ptr(), mxq.MXQ_BF16, R, C, qx.stride(0), mxq.MXQ_E4M3, rc.data_ptr(), rc.stride(0),
             rs.data_ptr(), rs.stride(0), cc.data_ptr(), cc.stride(0), cs.data_ptr(), cs.stride(0), sh)
        call = lambda: L.mxq_quantize_dual(*a)  # noqa: E731
        nbytes = R * C * (2 + 2 * (1 + 1 / 32))
    else:
        axis = mxq.MXQ_ROWWISE if kind == "rowwise" else mxq.MXQ_COLWISE
        if kind == "colwise":
            rc = rc.view(C, R)
            rs = torch.empty((C, R // 32), dtype=torch.uint8, device=dev)
        a = (qx.data_ptr(), mxq.MXQ_BF16, R, C, qx.stride(0), axis, mxq.MXQ_E4M3, rc.data_ptr(), rc.stride(0),
             rs.data_ptr(), rs.stride(0), sh)
        call = lambda: L.mxq_quantize(*a)  # noqa: E731
        nbytes = R * C * (2 + 1 + 1 / 32)
    st = call()
    if st != 0:
        raise RuntimeError("%s failed: %s" % (args.only, mxq.mxq_status_string(st)))
    settle(torch, call, args.settle_ms)
    for _ in range(args.warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)
    print(json.dumps({"kernel": args.only, "workload": "[16384][16384] bf16, E4M3", "steps": args.steps,
                      "ms": round(ms, 5), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                      "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}))
    if args.copy_calibration:
        copy_calibration(torch, dev)


def only_gemm(args, torch, mxq, wl, dev):
    """One GEMM mode alone on the projection workload (codes quantized once, untimed):
    bf16 output, W untimed launches then K timed ones."""
    import ctypes
    L = mxq.lib()
    stream = torch.cuda.current_stream()
    d = wl.workload2()
    M, K, N = d["M"], d["K"], d["N"]
    xc, xs = mxq.quantize(d["x"].to(dev), "e4m3", "row")
    wc, ws = mxq.quantize(d["w"].to(dev), "e4m3", "row")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    acc = mxq.MXQ_ACC_FP32 if ONLY_KERNELS[args.only] == "exact" else mxq.MXQ_ACC_FP8_MFMA
    a = (M, N, K, xc.data_ptr(), xc.stride(0), xs.data_ptr(), xs.stride(0), mxq.MXQ_E4M3, wc.data_ptr(), wc.stride(0),
         ws.data_ptr(), ws.stride(0), mxq.MXQ_E4M3, ctypes.c_float(1.0), None, y.data_ptr(), mxq.MXQ_BF16, y.stride(0),
         acc, ctypes.c_void_p(stream.cuda_stream))
    st = L.mxq_gemm(*a)
    if st != 0:
        raise RuntimeError("%s failed: %s" % (args.only, mxq.mxq_status_string(st)))
    settle(torch, lambda: L.mxq_gemm(*a), args.settle_ms)
    for _ in range(args.warmup):
        L.mxq_gemm(*a)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        L.mxq_gemm(*a)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    print(json.dumps({"kernel": args.only, "workload": "projection M=%d K=%d N=%d, E4M3, bf16 out" % (M, K, N),
                      "steps": args.steps, "ms": round(ms, 5), "tflops": round(tflops, 2),
                      "frac_of_mxfp8_peak": round(tflops / PEAK_MXFP8_TFLOPS, 4),
                      "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}))
    if args.copy_calibration:
        copy_calibration(torch, dev)


def only_reference(args, torch, wl, dev):
    """torch's own kernels on the same shapes, timed like the --only legs: what a plain
    streaming kernel (cast, copy) and the library bf16 GEMM reach on this machine."""
    kind = ONLY_KERNELS[args.only]
    if kind == "ref_mm":
        d = wl.workload2()
        M, K, N = d["M"], d["K"], d["N"]
        xb = d["x"].to(dev)
        wt = d["w"].to(dev).t().contiguous()          # [K][N]: a plain NN product
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        call = lambda: torch.mm(xb, wt, out=y)  # noqa: E731
        work = 2.0 * M * N * K
        what = "torch.mm bf16 [%d][%d] x [%d][%d], bf16 out" % (M, K, K, N)
    else:
        x = wl.workload_q()["x"].to(dev)
        y = torch.empty(x.shape, dtype=torch.int8 if kind == "ref_cast" else torch.bfloat16, device=dev)
        call = lambda: y.copy_(x)  # noqa: E731
        work = x.numel() * (2 + y.element_size())
        what = "[16384][16384] bf16 -> %s elementwise copy" % ("int8" if kind == "ref_cast" else "bf16")
    stream = torch.cuda.current_stream()
    settle(torch, call, args.settle_ms)
    for _ in range(args.warmup + 1):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)
    res = {"kernel": args.only, "workload": what, "steps": args.steps, "ms": round(ms, 5)}
    if kind == "ref_mm":
        tflops = work / (ms * 1e-3) / 1e12
        res.update({"tflops": round(tflops, 2), "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4)})
    else:
        gbs = work / (ms * 1e-3) / 1e9
        res.update({"gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
    print(json.dumps(res))


def copy_calibration(torch, dev):
    """A plain copy of known size for the FETCH_SIZE / WRITE_SIZE calibration."""
    a = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(2):
        torch.mul(a, 1.0, out=b)      # reads 256 MiB, writes 256 MiB
    torch.cuda.synchronize()
    del a, b


def cpu_baseline(d, xc, xs, wc, ws, M, N, K, target_s):
    """Time the oracle on a bounded sample of the same step and scale to TFLOP/s:
    quantize of a row slice of X and W, and the FP64 reference of a sample of outputs."""
    import numpy as np

    import oracle
    from mxfp8_block_scaled_03_amd.workloads import bf16_bits

    x_bits = bf16_bits(d["x"])
    w_bits = bf16_bits(d["w"])
    rows = 512
    t = time.perf_counter()
    oracle.quantize(x_bits[:rows], "e4m3")
    tq = time.perf_counter() - t
    quant_per_elem = tq / (rows * K)
    xc_h, xs_h, wc_h, ws_h = xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy()
    rng = np.random.default_rng(0)
    n = 2048
    ii, jj = rng.integers(0, M, n), rng.integers(0, N, n)
    t = time.perf_counter()
    oracle.gemm_sampled(xc_h, xs_h, "e4m3", wc_h, ws_h, "e4m3", K, ii, jj)
    tg = time.perf_counter() - t
    per_out = tg / n
    # grow the GEMM sample to roughly the target time
    n2 = int(min(max(target_s / max(per_out, 1e-9) * 0.8, n), 1 << 22))
    ii, jj = rng.integers(0, M, n2), rng.integers(0, N, n2)
    t = time.perf_counter()
    oracle.gemm_sampled(xc_h, xs_h, "e4m3", wc_h, ws_h, "e4m3", K, ii, jj)
    tg2 = time.perf_counter() - t
    per_out = tg2 / n2
    step_s = quant_per_elem * (M * K + N * K) + per_out * M * N
    del w_bits
    return {"value": round(2.0 * M * N * K / step_s / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "oracle quantize of %d of the %d X rows and FP64 reference of %d of the %d outputs "
                      "(%.1f s CPU); step time extrapolated per element" % (rows, M, n2, M * N, tq + tg2),
            "step_seconds_extrapolated": round(step_s, 2)}


if __name__ == "__main__":
    main()

"""Build libmxq.so (the HIP kernels + the C ABI of include/mxq.h) for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmxq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU ops (v_pk_{add,mul,fma}_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-inline-asm", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _compile(src: str, obj: str, verbose: bool):
    cmd = [HIPCC] + FLAGS + ["-c", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), src, "-o", obj]
    if verbose:
        print(" ".join(cmd))
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every csrc/*.hip to an object in parallel (one hipcc per source), then link."""
    from concurrent.futures import ThreadPoolExecutor
    srcs = sources()
    tag = "%d" % os.getpid()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + "." + tag + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 1)))
    try:
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            results = list(pool.map(lambda so: _compile(so[0], so[1], verbose), zip(srcs, objs)))
        for src, r in zip(srcs, results):
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError("hipcc failed compiling %s" % os.path.basename(src))
        tmp = LIB + ".tmp" + tag
        cmd = [HIPCC] + FLAGS + objs + ["-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking libmxq.so")
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

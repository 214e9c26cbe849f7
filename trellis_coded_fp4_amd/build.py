"""Build libtrellis.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

Also builds libtq_bitcheck.so, a host-only build of the decoder's integer
arithmetic that the CPU tests use. Run: python -m trellis_coded_fp4_amd.build
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtrellis.so")
BITCHECK = os.path.join(HERE, "libtq_bitcheck.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep fp32 arithmetic out of the packed-FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build failed: {' '.join(cmd[:3])} ...")
    return r


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 (one translation unit per process,
    in parallel), link libtrellis.so, and build the host check library."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with tempfile.TemporaryDirectory(prefix="tq_build_") as obj_dir:
        objs = [os.path.join(obj_dir, os.path.basename(s) + ".o") for s in srcs]
        jobs = max(1, min(len(srcs), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda so: _run(["hipcc", *HIPCC_FLAGS, "-c", "-o", so[1], so[0]]), zip(srcs, objs)))
        tmp = LIB + f".tmp{os.getpid()}"
        _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    tmp = BITCHECK + f".tmp{os.getpid()}"
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-o", tmp,
          os.path.join(CSRC, "tq_bitcheck.cpp")])
    os.replace(tmp, BITCHECK)
    if verbose:
        print("built", LIB, BITCHECK)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

"""Build libw4a16.so in-tree with hipcc for gfx950.

Every HIP source is compiled on its own (in parallel), then linked into one
shared library next to this file.  Packed fp32 instructions are disabled for
the device code (the kernels are written in scalar fp32).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libw4a16.so")

HIP_SOURCES = ["prepack.hip", "gemm_small.hip", "gemm_tile.hip", "msd.hip", "moe.hip", "mxfp4.hip", "w8.hip", "fzero.hip"]
CPP_SOURCES = ["api.cpp"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if p and os.path.exists(p):
            return p
    raise RuntimeError("hipcc not found")


# hipcc passes the target feature to the host (x86) compile too, which
# rejects it with exactly this message; the device compile must accept it
# (checked by _check_device_feature before every build).
_HOST_FEATURE_MSG = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if l.strip() != _HOST_FEATURE_MSG and l.strip() and "warning generated" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def _check_device_feature(cc):
    """The device compile alone must accept '-packed-fp32-ops' without any
    message, so that the only rejection the full build can print (and
    _run drops) is the host compile's."""
    os.makedirs(BUILD, exist_ok=True)
    src = os.path.join(BUILD, "feature_probe.hip")
    with open(src, "w") as f:
        f.write("#include <hip/hip_runtime.h>\n__global__ void k(float *p) { p[threadIdx.x] *= 2.f; }\n")
    r = subprocess.run([cc, *COMMON, *DEVICE, "--offload-device-only", "-c", src, "-o", src + ".o"],
                       capture_output=True, text=True)
    msg = (r.stdout + r.stderr).strip()
    if r.returncode != 0 or "packed-fp32-ops" in msg:
        raise RuntimeError(f"device compile does not accept -packed-fp32-ops:\n{msg}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    _check_device_feature(cc)
    jobs = []
    for s in HIP_SOURCES:
        jobs.append([cc, *COMMON, *DEVICE, "-c", os.path.join(CSRC, s), "-o", os.path.join(BUILD, s + ".o")])
    for s in CPP_SOURCES:
        jobs.append([cc, *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, s),
                     "-o", os.path.join(BUILD, s + ".o")])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(lambda c: _run(c, verbose), jobs):
            if out and verbose:
                print(out)
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + CPP_SOURCES]
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

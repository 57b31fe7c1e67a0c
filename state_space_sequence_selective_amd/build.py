"""Build the HIP library libmamba_scan.so for gfx950 (in-tree).

Every .hip file under csrc/ is compiled to an object with hipcc (in
parallel), then linked into state_space_sequence_selective_amd/libmamba_scan.so
(with rocBLAS, which the layer entry points use for their projections).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmamba_scan.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# no packed-FP32 instructions: the compiler emits plain v_fma/v_mul/v_add only
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# the layer entry points hand their dense projections to rocBLAS
LINK = ["-L/opt/rocm/lib", "-lrocblas", "-Wl,-rpath,/opt/rocm/lib"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + DEVICE_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    return obj, msg


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    for obj, msg in results:
        if verbose and msg.strip():
            print(msg)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + [o for o, _ in results] + LINK
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

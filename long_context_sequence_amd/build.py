"""Build the HIP library ``libvla.so`` in-tree for gfx950.

Each ``csrc/*.hip`` is compiled to an object in parallel, then linked with
``hipcc -shared``.  Packed FP32 instructions are disabled for the device code
(``-packed-fp32-ops``); the host pass prints a harmless warning about that
target feature.  Matrix-core instructions keep their accumulators in VGPRs
(``-amdgpu-mfma-vgpr-form``).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvla.so")
# the benchmark's attainable-throughput probe, a library of its own
PEAK_SRC = os.path.join(PKG, "peak", "vla_peak.hip")
PEAK_LIB = os.path.join(PKG, "libvla_peak.so")
ARCH = os.environ.get("VLA_OFFLOAD_ARCH", "gfx950")

# MFMA accumulators in VGPRs: the matrix-core results feed vector code (scales,
# negations, LDS stores), and with accumulators in AGPRs every such use costs a
# copy instruction; the penalty pass measured 330 -> 314 us with this form
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-Wall", "-Wno-unused-result"]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed for {src}")
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if err:
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None) -> str:
    """Compile every csrc/*.hip and link libvla.so, and build the probe library
    libvla_peak.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [PEAK_SRC]
    n = jobs or min(16, max(1, os.cpu_count() or 1), len(srcs))
    with ThreadPoolExecutor(max_workers=n) as ex:
        objs = list(ex.map(_compile, srcs))
    peak_obj = objs.pop()
    for lib, parts in ((LIB, objs), (PEAK_LIB, [peak_obj])):
        tmp = lib + ".tmp"
        subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *parts, "-o", tmp],
                       check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build())

"""Build libmoe.so (HIP, gfx950 only) in-tree with hipcc.

    python -m top_routing_expert_gemm_amd.build
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe.so")

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def flags():
    """Flags common to the device and the host compilation of a source."""
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-I", INCLUDE, "-I", CSRC,
        "-Wno-unused-command-line-argument",
    ]


# Packed fp32 arithmetic is kept off in the device code (plain scalar fp32
# only).  The switch is a target feature of the device compiler alone, so each
# source is compiled in two passes: the device pass with the feature turned off
# (its output is the offload bundle of the gfx950 code object), then the host
# pass, which embeds that bundle.  The host compiler never sees the feature.
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def _compile(cc, src, tmpd, verbose):
    base = os.path.join(tmpd, os.path.basename(src)[:-4])
    dev = [cc, *flags(), "--offload-device-only", *DEVICE_ONLY, "-c", src, "-o", base + ".dev"]
    host = [cc, *flags(), "--offload-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", base + ".dev",
            "-c", src, "-o", base + ".o"]
    for c in (dev, host):
        if verbose:
            print(" ".join(c), flush=True)
        _run(c)
    return base + ".o"


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every .hip source (in parallel), link the objects into one shared
    library, and return its path.  Intermediate files go to a temporary folder."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    cc = hipcc()
    srcs = sources()
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmpd:
        with ThreadPoolExecutor(jobs) as ex:
            objs = list(ex.map(lambda src: _compile(cc, src, tmpd, verbose), srcs))
        tmp = LIB + ".tmp"
        link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        _run(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

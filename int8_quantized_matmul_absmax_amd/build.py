"""Build libi8mm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m int8_quantized_matmul_absmax_amd.build

Compiles every csrc/*.hip to an object under _build/ (in parallel) and links
the shared library next to this file, where the binding loads it from.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libi8mm.so")

ARCH = "gfx950"

COMMON_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-fvisibility=hidden",
    # Scale arithmetic of the quantizers must be one IEEE fp32 operation at a
    # time with a correctly rounded divide.
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # No packed fp32 instructions in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + COMMON_FLAGS + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the device feature flag; that warning
    # is expected and dropped from the log.
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (src, "\n".join(lines)))
    if verbose and lines:
        print("\n".join(lines), flush=True)
    return obj


def build_library(verbose=False):
    """Compile and link libi8mm.so; returns its path. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build_library(verbose="-v" in sys.argv)
    print(path)

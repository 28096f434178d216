"""The C ABI's argument validation under the host address and
undefined-behaviour sanitizers (no GPU needed).

Every csrc/*.hip file is compiled with the sanitizers on its host pass only
(device code is built as usual), linked with tests/abi_sanitizer_driver.cpp,
and run: each entry point is called with null, negative, misaligned,
overflowing and NaN arguments and undersized workspaces, and must return the
documented status with no sanitizer report. Only where the host has no GPU
driver does the driver also make one fully valid call (it must report
I8MM_ENODEVICE), since the addresses it passes are fake.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess

import pytest

from int8_quantized_matmul_absmax_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "abi_sanitizer_driver.cpp")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")

# Sanitizers for the host pass of hipcc only, each behind -Xarch_host.
HOST_SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]


def _hipcc_flags():
    flags = [f for f in B.COMMON_FLAGS if f != "-O3"] + ["-O1", "-g"]
    for f in HOST_SAN:
        flags += ["-Xarch_host", f]
    return flags


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    return r.returncode, out


def test_abi_validation_under_host_sanitizers(tmp_path):
    if not (shutil.which("hipcc") or os.path.exists(os.path.join(ROCM, "bin", "hipcc"))):
        pytest.skip("hipcc not available")
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not available")
    hipcc = B._hipcc()
    srcs = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        rc, out = _run([hipcc] + _hipcc_flags() + ["-c", src, "-o", obj])
        assert rc == 0, "compile %s:\n%s" % (src, out)
        return obj

    with concurrent.futures.ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv_obj = str(tmp_path / "driver.o")
    rc, out = _run([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(B.ROOT, "include"),
                    "-c", DRIVER, "-o", drv_obj])
    assert rc == 0, out
    exe = str(tmp_path / "driver")
    rc, out = _run([CLANG, "-fsanitize=address,undefined", drv_obj] + objs
                   + ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                      "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    assert rc == 0, out
    args = [exe] + ([] if os.path.exists("/dev/kfd") else ["--no-device"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    rc, out = _run(args, env=env, timeout=300)
    assert rc == 0 and "ALL OK" in out, out

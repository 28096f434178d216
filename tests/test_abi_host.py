"""Host-side checks of the C ABI (no GPU needed, no compute calls).

The library must load, export every symbol include/i8mm.h declares, and reject
invalid arguments on the host with the documented status before touching a
device. Fake device addresses are used only where validation fails first.
"""

import ctypes
import math
import os
import re

import pytest

import int8_quantized_matmul_absmax_amd as i8
from int8_quantized_matmul_absmax_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "i8mm.h")

A = ctypes.c_void_p(0x10000)      # aligned, never dereferenced
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)    # not 16-byte aligned
NUL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return i8.ensure_built()


def _declared_names():
    src = open(HEADER).read()
    return set(re.findall(r"I8MM_API\s+[\w\s\*]+?\b(\w+)\s*\(", src))


def test_header_and_exports_agree(lib):
    names = _declared_names()
    assert names == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_only_the_abi_is_exported(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(_lib.EXPORTS) <= syms
    assert not [s for s in syms if "i8mm" in s and s not in _lib.EXPORTS and s.startswith("_Z")]


def test_status_strings(lib):
    assert lib.i8mm_status_string(0) == b"I8MM_OK"
    assert lib.i8mm_status_string(-3) == b"I8MM_EWORKSPACE"
    assert lib.i8mm_status_string(99) == b"I8MM_UNKNOWN"


def test_workspace_layout_is_pure_and_consistent(lib):
    for M, K in [(1, 16), (16, 256), (2048, 4096), (4096, 12288), (0, 64)]:
        off = (ctypes.c_int64 * 7)()
        assert lib.i8mm_workspace_layout(M, K, off) == 0
        off = list(off)
        assert off[0] == 0 and all(b >= a for a, b in zip(off, off[1:]))
        assert all(o % 256 == 0 for o in off)
        assert off[1] - off[0] >= (K + 31) // 32 * 4
        assert off[2] - off[1] >= 4 * K
        assert off[4] - off[3] >= 4 * M
        assert off[5] - off[4] >= M * K
        assert off[6] - off[5] >= M * ((K + 31) // 32 * 32) * 2
        assert lib.linear_int8_mixed_workspace_bytes(M, K) == off[6]
    assert lib.linear_int8_mixed_workspace_bytes(4, 20) == 0
    assert lib.linear_int8_mixed_workspace_bytes(-1, 16) == 0
    assert lib.i8mm_workspace_layout(4, 16, None) == _lib.I8MM_EINVAL


def test_many_outlier_region_is_capped(lib):
    """The optional region of recovered outlier weights holds at most
    I8MM_OUTLIER_REGION_COLS (512) columns per output row, whatever K: its
    memory is bounded by N x 1 KiB, not N x K halfs."""
    assert i8.ops.OUTLIER_REGION_COLS == 512
    for M, K, N in [(16, 256, 100), (2048, 4096, 16384), (4096, 12288, 49152), (1024, 16384, 4096)]:
        base = lib.linear_int8_mixed_workspace_bytes(M, K)
        big = lib.linear_int8_mixed_workspace_bytes_many_outliers(M, K, N)
        cols = min(K, 512)
        region = N * ((cols + 31) // 32 * 32) * 2
        assert big - base == (region + 255) // 256 * 256
    assert lib.linear_int8_mixed_workspace_bytes_many_outliers(16, 4096, -1) == 0


def test_outlier_region_room():
    """The room of the recovered-weight region is what the extra bytes hold,
    in whole 32-column groups, at most LD(K): the default region has room for
    512 columns (K >= 512), the all-outliers size for every count, and a
    region one byte short of a group loses that group."""
    ops = i8.ops
    for M, K, N in [(16, 256, 100), (2048, 4096, 16384), (300, 2064, 4100), (1, 16, 1)]:
        base = ops.workspace_bytes(M, K)
        assert ops.outlier_region_cols(base, M, K, N) == 0
        assert ops.outlier_region_cols(ops.workspace_bytes(M, K, N), M, K, N) == \
            min(512, ops.outlier_ld(K))
        assert ops.outlier_region_cols(ops.workspace_bytes_all_outliers(M, K, N), M, K, N) == \
            ops.outlier_ld(K)
        assert ops.outlier_region_cols(base + 64 * N - 1, M, K, N) == 0
        assert ops.outlier_region_cols(base + 64 * N, M, K, N) == min(32, ops.outlier_ld(K))


def test_validation_quantize_weight(lib):
    f = lib.int8_quantize_colwise_weight
    assert f(NUL, 4, 16, A, A2, NUL) == _lib.I8MM_EINVAL
    assert f(A, 4, 16, NUL, A2, NUL) == _lib.I8MM_EINVAL
    assert f(A, -1, 16, A, A2, NUL) == _lib.I8MM_EINVAL
    assert f(A, 4, 24, A, A2, NUL) == _lib.I8MM_EALIGN
    assert f(MIS, 4, 16, A, A2, NUL) == _lib.I8MM_EALIGN
    kmax16 = _lib.I8MM_MAX_K // 16 * 16          # largest valid K (multiple of 16)
    assert f(A, 4, kmax16 + 16, A, A2, NUL) == _lib.I8MM_ERANGE
    assert f(A, 4, kmax16, NUL, A2, NUL) == _lib.I8MM_EINVAL    # K itself accepted
    assert f(A, 0, 16, A, A2, NUL) == _lib.I8MM_OK              # empty: no-op


def test_validation_last_error_text(lib):
    assert lib.int8_quantize_colwise_weight(A, 4, 24, A, A2, NUL) == _lib.I8MM_EALIGN
    assert b"multiple of 16" in lib.i8mm_last_error()


def test_validation_rowwise(lib):
    f = lib.int8_quantize_rowwise
    assert f(NUL, 4, 16, NUL, A, A2, NUL) == _lib.I8MM_EINVAL
    assert f(A, 4, 16, MIS, A, A2, NUL) == _lib.I8MM_EALIGN
    assert f(A, 4, 8, NUL, A, A2, NUL) == _lib.I8MM_EALIGN
    assert f(A, 0, 16, NUL, A, A2, NUL) == _lib.I8MM_OK


def test_validation_outlier_detect(lib):
    f = lib.outlier_detect_gather
    assert f(A, 4, 16, math.nan, A, A, A, NUL, NUL) == _lib.I8MM_EINVAL
    assert f(A, 4, 16, 6.0, NUL, A, A, NUL, NUL) == _lib.I8MM_EINVAL
    assert f(A, 4, 16, 6.0, A, NUL, A, NUL, NUL) == _lib.I8MM_EINVAL
    assert f(A, 4, 16, 6.0, A, A, NUL, NUL, NUL) == _lib.I8MM_EINVAL
    assert f(A, 4, 16, 6.0, A, A, A, MIS, NUL) == _lib.I8MM_EALIGN
    assert f(A, 4, 40, 6.0, A, A, A, NUL, NUL) == _lib.I8MM_EALIGN


def test_validation_mm_dequant(lib):
    f = lib.int8_mm_dequant
    ok = [A, A, A, A, 4, 4, 16, NUL, NUL, NUL, NUL, A, NUL, NUL]
    bad = list(ok); bad[0] = NUL
    assert f(*bad) == _lib.I8MM_EINVAL
    bad = list(ok); bad[7] = A           # Xo without cols / n
    assert f(*bad) == _lib.I8MM_EINVAL
    bad = list(ok); bad[11] = NUL        # neither Y nor C
    assert f(*bad) == _lib.I8MM_EINVAL
    bad = list(ok); bad[10] = MIS        # misaligned bias
    assert f(*bad) == _lib.I8MM_EALIGN
    bad = list(ok); bad[6] = 17
    assert f(*bad) == _lib.I8MM_EALIGN
    bad = list(ok); bad[5] = -2
    assert f(*bad) == _lib.I8MM_EINVAL
    bad = list(ok); bad[4] = 0           # M == 0: no-op
    assert f(*bad) == _lib.I8MM_OK


def test_validation_linear(lib):
    f = lib.linear_int8_mixed
    M, K, N = 8, 64, 32
    need = lib.linear_int8_mixed_workspace_bytes(M, K)
    ws = ctypes.c_void_p(0x100000)
    args = [A, M, K, A, A, N, NUL, 6.0, A2, ws, need, NUL]
    bad = list(args); bad[10] = need - 1
    assert f(*bad) == _lib.I8MM_EWORKSPACE
    bad = list(args); bad[9] = NUL
    assert f(*bad) == _lib.I8MM_EWORKSPACE
    bad = list(args); bad[9] = ctypes.c_void_p(0x100010)     # 16- but not 256-aligned
    assert f(*bad) == _lib.I8MM_EALIGN
    bad = list(args); bad[7] = math.nan
    assert f(*bad) == _lib.I8MM_EINVAL
    bad = list(args); bad[8] = NUL
    assert f(*bad) == _lib.I8MM_EINVAL
    bad = list(args); bad[2] = 72
    assert f(*bad) == _lib.I8MM_EALIGN
    bad = list(args); bad[1] = 0; bad[10] = lib.linear_int8_mixed_workspace_bytes(0, K)
    assert f(*bad) == _lib.I8MM_OK


def test_validation_linear_fp16_weights(lib):
    """The fp16-weight layer call: the weight W is required and aligned, the
    rest is validated as in linear_int8_mixed, all before any launch."""
    f = lib.linear_int8_mixed_fp16_weights
    M, K, N = 8, 64, 32
    need = lib.linear_int8_mixed_workspace_bytes(M, K)
    ws = ctypes.c_void_p(0x100000)
    args = [A, M, K, A2, N, A, A2, 1, NUL, 6.0, A2, ws, need, NUL]
    bad = list(args); bad[3] = NUL
    assert f(*bad) == _lib.I8MM_EINVAL
    bad = list(args); bad[3] = MIS
    assert f(*bad) == _lib.I8MM_EALIGN
    bad = list(args); bad[5] = NUL
    assert f(*bad) == _lib.I8MM_EINVAL
    bad = list(args); bad[6] = NUL
    assert f(*bad) == _lib.I8MM_EINVAL
    bad = list(args); bad[12] = need - 1
    assert f(*bad) == _lib.I8MM_EWORKSPACE
    bad = list(args); bad[9] = math.nan
    assert f(*bad) == _lib.I8MM_EINVAL
    bad = list(args); bad[10] = NUL
    assert f(*bad) == _lib.I8MM_EINVAL
    bad = list(args); bad[2] = K + 8
    assert f(*bad) == _lib.I8MM_EALIGN
    bad = list(args); bad[2] = (_lib.I8MM_MAX_K // 16 + 1) * 16
    assert f(*bad) == _lib.I8MM_ERANGE
    bad = list(args); bad[1] = 0; bad[12] = lib.linear_int8_mixed_workspace_bytes(0, K)
    assert f(*bad) == _lib.I8MM_OK


def test_validation_gelu(lib):
    assert lib.i8mm_gelu_f16(A, -1, A, NUL) == _lib.I8MM_EINVAL
    assert lib.i8mm_gelu_f16(MIS, 4, A, NUL) == _lib.I8MM_EALIGN
    assert lib.i8mm_gelu_f16(A, 0, A, NUL) == _lib.I8MM_OK


def test_no_gfx950_device_is_reported(lib):
    """Without a gfx950 GPU, a valid call fails loudly with ENODEVICE and
    launches nothing (the product path has no CPU fallback)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; the no-device path is not reachable")
    st = lib.int8_quantize_colwise_weight(A, 4, 16, A, A2, NUL)
    assert st == _lib.I8MM_ENODEVICE


def test_python_ops_refuse_cpu_tensors():
    import torch
    W = torch.zeros((4, 16), dtype=torch.float16)
    with pytest.raises(ValueError):
        i8.ops.int8_quantize_colwise_weight(W)
    with pytest.raises(TypeError):
        i8.ops.int8_quantize_colwise_weight(W.float())


def test_python_ops_check_every_size_before_launch():
    """Every tensor a caller hands to the binding is checked for dtype and size
    on the host, before anything reaches the library: a too-small output,
    bias, scale vector, outlier buffer or count would otherwise become device
    writes or reads out of bounds. Host tensors of the right sizes reach the
    device check and stop there (the path runs on the GPU only)."""
    import torch
    ops = i8.ops
    M, K, N = 8, 64, 32
    f16, i8t, f32, i32 = torch.float16, torch.int8, torch.float32, torch.int32
    X = torch.zeros((M, K), dtype=f16)
    Wq = torch.zeros((N, K), dtype=i8t)
    sw = torch.zeros((N,), dtype=f32)
    Xq = torch.zeros((M, K), dtype=i8t)
    sx = torch.zeros((M,), dtype=f32)
    Xo = torch.zeros((M * ops.outlier_ld(K),), dtype=f16)
    cols = torch.zeros((K,), dtype=i32)
    n = torch.zeros((1,), dtype=i32)
    ws = torch.zeros((ops.workspace_bytes(M, K),), dtype=torch.uint8)

    def bad(fn, *a, **kw):
        with pytest.raises(ValueError) as e:
            fn(*a, **kw)
        assert "GPU" not in str(e.value), e.value   # refused for its size, not its device

    # layer call: out, bias, sw, Wq width, workspace
    bad(ops.linear_int8_mixed, X, Wq, sw, out=torch.zeros((M * N - 1,), dtype=f16))
    bad(ops.linear_int8_mixed, X, Wq, sw, bias=torch.zeros((N - 1,), dtype=f16))
    bad(ops.linear_int8_mixed, X, Wq, torch.zeros((N + 1,), dtype=f32))
    bad(ops.linear_int8_mixed, X, torch.zeros((N, K + 16), dtype=i8t), sw)
    bad(ops.linear_int8_mixed, X, Wq, sw, workspace=ws[:-1])
    bad(ops.linear_int8_mixed_fp16_weights, X, torch.zeros((N, K), dtype=f16),
        torch.zeros((N, K - 16), dtype=i8t), sw)
    bad(ops.linear_int8_mixed_fp16_weights, X, torch.zeros((N, K), dtype=f16), Wq,
        torch.zeros((N - 1,), dtype=f32))
    # step calls
    bad(ops.int8_quantize_colwise_weight, torch.zeros((N, K), dtype=f16), Wq[:-1])
    bad(ops.int8_quantize_colwise_weight, torch.zeros((N, K), dtype=f16), Wq, sw[:-1])
    bad(ops.int8_quantize_rowwise, X, torch.zeros((K // 32 - 1,), dtype=i32))
    bad(ops.int8_quantize_rowwise, X, None, Xq[:-1])
    bad(ops.int8_quantize_rowwise, X, None, Xq, sx[:-1])
    bad(ops.int8_mm_dequant, Xq, Wq, sx[:-1], sw)
    bad(ops.int8_mm_dequant, Xq, Wq, sx, sw[:-1])
    bad(ops.int8_mm_dequant, Xq, torch.zeros((N, K + 16), dtype=i8t), sx, sw)
    bad(ops.int8_mm_dequant, Xq, Wq, sx, sw, Xo[:-1], cols, n)
    bad(ops.int8_mm_dequant, Xq, Wq, sx, sw, Xo, cols[:-1], n)
    bad(ops.int8_mm_dequant, Xq, Wq, sx, sw, Xo, cols, torch.zeros((2,), dtype=i32))
    bad(ops.int8_mm_dequant, Xq, Wq, sx, sw, Xo, cols, None)
    bad(ops.int8_mm_dequant, Xq, Wq, sx, sw, bias=torch.zeros((N + 1,), dtype=f16))
    bad(ops.int8_mm_dequant, Xq, Wq, sx, sw, out=torch.zeros((M, N - 1), dtype=f16))
    bad(ops.gelu_f16, X, torch.zeros((M * K - 1,), dtype=f16))
    with pytest.raises(TypeError):
        ops.int8_mm_dequant(Xq, Wq, sx, sw, Xo, cols, n.to(torch.int64))
    # the right sizes on the host: refused by the device check
    for fn, a in [(ops.linear_int8_mixed, (X, Wq, sw)),
                  (ops.int8_mm_dequant, (Xq, Wq, sx, sw, Xo, cols, n)),
                  (ops.int8_quantize_rowwise, (X,))]:
        with pytest.raises(ValueError, match="GPU"):
            fn(*a)


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_present(), reason="the calls would launch on placeholder pointers")
def test_empty_arrays_may_be_null(lib):
    """With K == 0, X, Wq (and W, Xq, bitmap, cols) hold no elements and may be
    NULL: validation passes and the call only stops at the device check here.
    With K > 0 the same NULLs are rejected."""
    M, K, N = 8, 0, 32
    need = lib.linear_int8_mixed_workspace_bytes(M, K)
    ws = ctypes.c_void_p(0x100000)
    nodev = _lib.I8MM_ENODEVICE
    assert lib.linear_int8_mixed(NUL, M, K, NUL, A, N, NUL, 6.0, A2, ws, need, NUL) == nodev
    assert lib.linear_int8_mixed(NUL, M, 64, NUL, A, N, NUL, 6.0, A2, ws,
                                 lib.linear_int8_mixed_workspace_bytes(M, 64), NUL) == _lib.I8MM_EINVAL
    assert lib.linear_int8_mixed_fp16_weights(NUL, M, K, NUL, N, NUL, A, 1, NUL, 6.0, A2, ws, need,
                                              NUL) == nodev
    assert lib.int8_quantize_colwise_weight(NUL, N, K, NUL, A, NUL) == nodev
    assert lib.int8_quantize_rowwise(NUL, M, K, NUL, NUL, A, NUL) == nodev
    assert lib.outlier_detect_gather(NUL, M, K, 6.0, NUL, NUL, A, NUL, NUL) == nodev
    assert lib.int8_mm_dequant(NUL, NUL, A, A2, M, N, K, NUL, NUL, NUL, NUL, A, NUL, NUL) == nodev
    assert lib.int8_mm_dequant(NUL, NUL, A, A2, M, N, 16, NUL, NUL, NUL, NUL, A, NUL,
                               NUL) == _lib.I8MM_EINVAL

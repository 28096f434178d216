"""The single-launch few-token layer: the layer calls take it for M <= 16
tokens with K <= 16384 (M <= 4), 8192 (M <= 8) or 4096 (M <= 16), the
columns of X an X-side thread holds in registers; other few-token shapes (up
to 64 tokens) take the separate kernels (also here).

Against the oracle: every intermediate it writes to the workspace bit for
bit (bitmap, cols, n, codes, scales, gathered outlier columns and their zero
pads) and Y within the tolerance. Against the composed step calls (detection,
row quantization and the few-token GEMV as separate kernels): Y bit for bit,
since both form the same fp32 sums in the same order. Shapes reach each
register layout at its largest K, K = 16, ragged N, more tiles than
blocks (the persistent loop), more than 32 outlier columns (the epilogue's
bitmap walk) and the fp16-weight source.
"""

import numpy as np
import pytest
import torch

from int8_quantized_matmul_absmax_amd import synth
from oracle import llm_int8 as O
from tests.gpu_helpers import Y_TOL, dev, host, note, y_err
from tests.test_gpu_parity import _check_intermediates

pytestmark = pytest.mark.gpu

# (M, K, N, planted outlier columns, bias, weight kept in fp16)
CASES = {
    "m1_k4096_n4096": (1, 4096, 4096, 6, False, False),
    "m4_k4096_n4096": (4, 4096, 4096, 6, False, False),
    "m16_k4096_n4096": (16, 4096, 4096, 6, False, False),
    "m4_k16384": (4, 16384, 520, 10, True, False),
    "m5_k2064": (5, 2064, 300, 3, False, False),
    "m8_k8192_n40": (8, 8192, 257, 40, True, False),
    "m9_k1040": (9, 1040, 100, 20, False, False),
    "m12_k2048_n40": (12, 2048, 130, 40, True, False),
    "m16_k4112_separate": (16, 4112, 200, 7, False, False),
    "m8_k4096_many_tiles": (8, 4096, 16400, 6, True, False),
    "m16_k4096_many_tiles": (16, 4096, 16400, 6, True, False),
    "m3_k16": (3, 16, 64, 0, False, False),
    "m7_fp16w": (7, 4096, 300, 8, True, True),
    "m16_fp16w": (16, 4096, 300, 8, True, True),
    "m2_fp16w_n33": (2, 4112, 333, 33, False, True),
    "m20_fp16w_separate": (20, 4096, 300, 8, True, True),
    "m24_k4096_separate": (24, 4096, 520, 6, True, False),
    "m10_k8192_separate": (10, 8192, 300, 12, False, False),
    "m13_k4096_n40": (13, 4096, 1000, 40, False, False),
    "m1_k16384": (1, 16384, 700, 9, True, False),
    "m2_k8192_n7": (2, 8192, 300, 7, True, False),
    "m10_k4096_n6": (10, 4096, 400, 6, False, False),
    "m11_k4096_n6": (11, 4096, 400, 6, False, False),
    "m1_k4096_n15_many_tiles": (1, 4096, 16400, 15, True, False),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_decode_layer(gpu, case):
    M, K, N, n_plant, bias, f16w = CASES[case]
    note("decode %s" % case)
    ops = gpu.ops
    rng = np.random.default_rng(1200 + sum(map(ord, case)))
    X = synth.normal_f16(rng, (M, K), 1.0)
    W = synth.normal_f16(rng, (N, K), 0.02)
    if n_plant:
        synth.plant_outlier_columns(rng, X, n_plant, 7.0, 30.0, 1.0)
    b = synth.normal_f16(rng, (N,), 0.5) if bias else None
    Wq, sw = O.quantize_weight_rows(W)
    if f16w:
        ref = O.linear_int8_mixed_fp16_weights(X, W, 6.0, b)
    else:
        ref = O.linear_int8_mixed(X, Wq, sw, 6.0, b)
    assert ref["n"] >= n_plant
    ws = torch.empty((ops.workspace_bytes(M, K, N),), dtype=torch.uint8, device="cuda")
    Xd, bd = dev(X), (None if b is None else dev(b))
    Wqd, swd = dev(Wq), dev(sw)
    if f16w:
        Y = ops.linear_int8_mixed_fp16_weights(Xd, dev(W), Wqd, swd, False, bd, 6.0, ws)
    else:
        Y = ops.linear_int8_mixed(Xd, Wqd, swd, bd, 6.0, ws)
    torch.cuda.synchronize()
    views = ops.workspace_views(ws, M, K)
    _check_intermediates(gpu, views, X, ref)
    assert np.array_equal(host(views["bitmap"]).view(np.uint32), O.outlier_bitmap(ref["cols"], K))
    err = y_err(host(Y), ref["Y"])
    assert err <= Y_TOL, err
    if not f16w:
        # the composed step calls: separate detection, quantization and GEMV
        note("decode %s composed" % case)
        bm, cols, n, Xo = ops.outlier_detect_gather(Xd, 6.0)
        Xq, sx = ops.int8_quantize_rowwise(Xd, bm)
        Y2 = ops.int8_mm_dequant(Xq, Wqd, sx, swd, Xo, cols, n, bd)
        torch.cuda.synchronize()
        assert np.array_equal(host(Y).view(np.uint16), host(Y2).view(np.uint16))


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_subnormal_rows(gpu, M):
    """Token rows of fp16 subnormals: the row scale is 127 / a for a
    subnormal a, and every code comes from a subnormal times that scale."""
    note("decode subnormal M=%d" % M)
    ops = gpu.ops
    K, N = 4096, 256
    rng = np.random.default_rng(900 + M)
    X = synth.normal_f16(rng, (M, K), 1.0)
    synth.plant_outlier_columns(rng, X, 5, 7.0, 20.0, 1.0)
    bits = rng.integers(1, 0x400, size=(K,), dtype=np.uint16)
    bits |= rng.integers(0, 2, size=(K,), dtype=np.uint16) << 15
    X[0] = bits.view(np.float16)      # row 0: subnormals only (no outliers in it)
    if M > 2:
        X[2, ::5] = np.float16(6e-8)
    W = synth.normal_f16(rng, (N, K), 0.02)
    Wq, sw = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq, sw, 6.0, None)
    ws = torch.empty((ops.workspace_bytes(M, K),), dtype=torch.uint8, device="cuda")
    Y = ops.linear_int8_mixed(dev(X), dev(Wq), dev(sw), None, 6.0, ws)
    torch.cuda.synchronize()
    views = ops.workspace_views(ws, M, K)
    _check_intermediates(gpu, views, X, ref)
    assert np.count_nonzero(ref["Xq"][0]) > K // 2   # the subnormal row has real codes
    err = y_err(host(Y), ref["Y"])
    assert err <= Y_TOL, err


"""linear_int8_mixed_noalloc, the layer call whose workspace is the library's
own static scratch (for callers that cannot allocate), through the C ABI:
on two calls in a row, the second with a smaller input, its output equals
that of linear_int8_mixed with a caller-allocated workspace bit for bit (the
same kernels on the same intermediates) and is within the tolerance of the
oracle; sizes beyond the scratch are refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

from int8_quantized_matmul_absmax_amd import synth
from oracle import llm_int8 as O
from tests.gpu_helpers import Y_TOL, dev, host, note, y_err

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def test_noalloc_matches_layer_call(gpu):
    lib = gpu.load_library()
    ops = gpu.ops
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # (M, K, N, planted outlier columns, bias): the first call takes the tiled
    # GEMM with more than 16 outlier columns, the second (smaller) the
    # single-launch few-token path
    cases = [(700, 4096, 1000, 20, True), (5, 1040, 300, 3, False)]
    for M, K, N, n_plant, with_bias in cases:
        note("noalloc M=%d K=%d N=%d" % (M, K, N))
        rng = np.random.default_rng(7000 + M)
        X = synth.normal_f16(rng, (M, K), 1.0)
        synth.plant_outlier_columns(rng, X, n_plant, 7.0, 30.0, 0.5)
        W = synth.normal_f16(rng, (N, K), 0.03)
        b = synth.normal_f16(rng, (N,), 0.5) if with_bias else None
        Wq_ref, sw_ref = O.quantize_weight_rows(W)
        ref = O.linear_int8_mixed(X, Wq_ref, sw_ref, 6.0, b)
        assert ref["n"] >= n_plant
        Xd, Wqd, swd = dev(X), dev(Wq_ref), dev(sw_ref)
        bd = dev(b) if b is not None else None
        Y_layer = ops.linear_int8_mixed(Xd, Wqd, swd, bd, 6.0)
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        torch.cuda.synchronize()
        st = lib.linear_int8_mixed_noalloc(_p(Xd), M, K, _p(Wqd), _p(swd), N, _p(bd), 6.0, _p(Y),
                                           stream)
        assert st == 0, lib.i8mm_last_error()
        torch.cuda.synchronize()
        assert np.array_equal(host(Y).view(np.uint16), host(Y_layer).view(np.uint16))
        assert y_err(host(Y), ref["Y"]) <= Y_TOL

    # beyond the scratch: refused with EWORKSPACE, nothing launched
    M, K = 8192, 8192
    assert lib.linear_int8_mixed_workspace_bytes(M, K) > gpu._lib.I8MM_NOALLOC_SCRATCH_BYTES
    st = lib.linear_int8_mixed_noalloc(_p(Xd), M, K, _p(Wqd), _p(swd), 16, None, 6.0, _p(Y),
                                       stream)
    assert st == gpu._lib.I8MM_EWORKSPACE
    assert b"scratch" in lib.i8mm_last_error()

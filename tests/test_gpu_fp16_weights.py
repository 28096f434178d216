"""Parity of the layer with the weight kept in fp16 (has_fp16_weights=True)
against the oracle, through the C ABI.

Bit-exact: the weight codes and absmaxes the call writes, and the layer's
intermediates (outlier set, activation codes and scales, gathered columns).
Tolerance: Y within max |dY| / max |Y_ref| <= 1e-3 of the oracle's fp64
value. Cases cover the few-token and tiled GEMM paths (small and large
tiles), few and many outlier columns, both workspace sizes, codes given
instead of quantized at the call, and the module. Each case plants weight
columns too small for a nonzero int8 code under large outlier activations,
so that using the recovered weights instead of W's own columns would miss the
tolerance (checked on the oracle side).
"""

import numpy as np
import pytest
import torch

from int8_quantized_matmul_absmax_amd import synth
from oracle import llm_int8 as O
from tests.gpu_helpers import Y_TOL, dev, host, note, sample_rows, y_err

pytestmark = pytest.mark.gpu


def _inputs(seed, M, K, N, n_plant, bias=False):
    rng = np.random.default_rng(seed)
    X = synth.normal_f16(rng, (M, K), 1.0)
    W = synth.normal_f16(rng, (N, K), 0.02)
    if n_plant:
        cols, _ = synth.plant_outlier_columns(rng, X, n_plant, 7.0, 30.0, 0.5)
        # weak weight columns under strong outlier activations: their int8
        # codes (and so the recovered weights) are 0, W's own values are not
        for c in cols[:4]:
            X[:, c] = np.float16(40.0)
            W[:, c] = np.float16(2e-4)
    b = synth.normal_f16(rng, (N,), 0.5) if bias else None
    return X, W, b


def _discriminates(X, W, tau, b, ref):
    """The case tells the two weight sources apart (on the oracle side)."""
    Wq, sw = O.quantize_weight_rows(W)
    rec = O.linear_int8_mixed(X, Wq, sw, tau, b)
    return y_err(rec["Y"].astype(np.float16), ref["Y"]) > 2 * Y_TOL


def _run(gpu, X, W, tau, b, big_ws, quantize=True, Wq0=None, sw0=None):
    ops = gpu.ops
    M, K = X.shape
    N = W.shape[0]
    ws = torch.empty((ops.workspace_bytes(M, K, N if big_ws else None),), dtype=torch.uint8,
                     device="cuda")
    Wq = dev(Wq0) if Wq0 is not None else torch.full((N, K), 99, dtype=torch.int8, device="cuda")
    sw = dev(sw0) if sw0 is not None else torch.full((N,), -1.0, dtype=torch.float32, device="cuda")
    Y = ops.linear_int8_mixed_fp16_weights(dev(X), dev(W), Wq, sw, quantize,
                                           None if b is None else dev(b), tau, ws)
    torch.cuda.synchronize()
    return host(Y), host(Wq), host(sw), ops.workspace_views(ws, M, K, N if big_ws else None)


def _check(gpu, X, W, ref, Y, Wq, sw, views):
    M, K = X.shape
    n = ref["n"]
    assert np.array_equal(Wq, ref["Wq"])
    assert np.array_equal(sw.view(np.uint32), ref["sw"].view(np.uint32))
    assert int(host(views["n"])[0]) == n
    assert np.array_equal(host(views["cols"])[:n], ref["cols"])
    assert np.array_equal(host(views["Xq"]), ref["Xq"])
    assert np.array_equal(host(views["sx"]).view(np.uint32), ref["sx"].view(np.uint32))
    ld = gpu.ops.outlier_ld(n)
    Xo = host(views["Xo"])[: M * ld].reshape(M, ld)
    assert np.array_equal(Xo[:, :n].view(np.uint16), X[:, ref["cols"]].view(np.uint16))
    err = y_err(Y, ref["Y"])
    assert err <= Y_TOL, err


# (M, K, N, planted outlier columns, bias, larger workspace)
CASES = {
    "gemv_m1": (1, 1040, 300, 6, False, False),
    "gemv_m16_n40": (16, 1040, 300, 40, True, False),
    "gemv_m64_n20": (64, 528, 200, 20, False, True),
    "gemm_small_n6": (200, 1040, 300, 6, True, False),
    "gemm_small_n17": (200, 1040, 300, 17, False, False),
    "gemm_small_n17_big_ws": (200, 1040, 300, 17, False, True),
    "gemm_small_n50_big_ws": (97, 2064, 520, 50, True, True),
    "gemm_large_n9": (4100, 528, 4100, 9, True, False),
    "gemm_large_n40_big_ws": (4100, 528, 4100, 40, False, True),
    "gemm_large_n40": (4100, 528, 4100, 40, True, False),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_fp16_weights_layer(gpu, case):
    M, K, N, n_plant, bias, big = CASES[case]
    note("fp16 weights %s" % case)
    X, W, b = _inputs(500 + sum(map(ord, case)), M, K, N, n_plant, bias)
    ref = O.linear_int8_mixed_fp16_weights(X, W, 6.0, b)
    assert ref["n"] >= min(n_plant, 4)
    assert _discriminates(X, W, 6.0, b, ref)
    Y, Wq, sw, views = _run(gpu, X, W, 6.0, b, big)
    _check(gpu, X, W, ref, Y, Wq, sw, views)
    if big and case.startswith("gemm") and ref["n"] > 16:
        # the tiled path's materialized fp16 weight columns, bit for bit,
        # and their zero pad
        n, ld = ref["n"], gpu.ops.outlier_ld(ref["n"])
        Wo = host(views["Wo"])[: N * ld].reshape(N, ld).view(np.uint16)
        assert np.array_equal(Wo[:, :n], W[:, ref["cols"]].view(np.uint16))
        assert not Wo[:, n:].any()


@pytest.mark.parametrize("M", [40, 300])
def test_fp16_weights_both_workspaces(gpu, M):
    """More than 16 outlier columns: with the region, the tiled path gathers
    W's columns and runs the outlier product as a second loop over them; the
    minimal workspace takes the dense loop over all K columns with W's own
    fp16 values (normal columns zeroed). The few-token path ignores the
    region (bit-identical either way). Both within the tolerance."""
    note("fp16 weights both workspaces M=%d" % M)
    X, W, b = _inputs(700 + M, M, 1040, 330, 33, True)
    ref = O.linear_int8_mixed_fp16_weights(X, W, 6.0, b)
    Y_big, _, _, _ = _run(gpu, X, W, 6.0, b, True)
    Y_small, _, _, _ = _run(gpu, X, W, 6.0, b, False)
    assert y_err(Y_big, ref["Y"]) <= Y_TOL
    assert y_err(Y_small, ref["Y"]) <= Y_TOL
    if M <= 64:
        assert np.array_equal(Y_big.view(np.uint16), Y_small.view(np.uint16))


@pytest.mark.parametrize("M", [8, 200])
def test_fp16_weights_threshold_zero(gpu, M):
    """tau = 0: every column is an outlier; Y is the fp16 matmul of X with W
    itself (the int8 part is all zero)."""
    note("fp16 weights tau=0 M=%d" % M)
    X, W, _ = _inputs(800 + M, M, 528, 260, 0)
    ref = O.linear_int8_mixed_fp16_weights(X, W, 0.0)
    assert ref["n"] == 528
    for big in (False, True):
        Y, Wq, sw, views = _run(gpu, X, W, 0.0, None, big)
        _check(gpu, X, W, ref, Y, Wq, sw, views)


@pytest.mark.parametrize("M", [4, 250])
def test_fp16_weights_codes_given(gpu, M):
    """quantize_weight = 0 with the codes of the same W already in Wq, sw:
    the call leaves them as they are and gives the same Y bit for bit."""
    note("fp16 weights codes given M=%d" % M)
    X, W, b = _inputs(900 + M, M, 1040, 300, 8, True)
    ref = O.linear_int8_mixed_fp16_weights(X, W, 6.0, b)
    Y1, Wq1, sw1, _ = _run(gpu, X, W, 6.0, b, False)
    Y2, Wq2, sw2, views = _run(gpu, X, W, 6.0, b, False, quantize=False,
                               Wq0=ref["Wq"], sw0=ref["sw"])
    _check(gpu, X, W, ref, Y2, Wq2, sw2, views)
    assert np.array_equal(Y1.view(np.uint16), Y2.view(np.uint16))


def test_fp16_weights_module(gpu):
    """Int8Linear(has_fp16_weights=True): the output follows the current fp16
    weight (re-quantized at every call by default, or after set_weight_ only)."""
    note("fp16 weights module")
    X, W1, b = _inputs(950, 33, 512, 96, 5, True)
    _, W2, _ = _inputs(951, 33, 512, 96, 5)
    lin = gpu.Int8Linear(512, 96, bias=True, has_fp16_weights=True)
    with pytest.raises(RuntimeError):
        lin.quantize_(dev(W1))
    lin.set_weight_(dev(W1), dev(b))
    Xd = dev(X)
    r1 = O.linear_int8_mixed_fp16_weights(X, W1, 6.0, b)
    assert y_err(host(lin(Xd)), r1["Y"]) <= Y_TOL
    lin.weight.copy_(dev(W2))           # changed in place, as an optimizer would
    r2 = O.linear_int8_mixed_fp16_weights(X, W2, 6.0, b)
    Y2 = host(lin(Xd))
    assert y_err(Y2, r2["Y"]) <= Y_TOL
    assert np.array_equal(host(lin.CB), r2["Wq"])
    lin.requantize_every_call = False
    assert np.array_equal(host(lin(Xd)).view(np.uint16), Y2.view(np.uint16))
    lin.set_weight_(dev(W1))
    assert y_err(host(lin(Xd)), r1["Y"]) <= Y_TOL


def test_fp16_weights_opt_ffn_up_full(gpu):
    """OPT-6.7B FFN up-projection (2048 x 4096 -> 16384, 6 outlier dims) with
    the weight kept in fp16 and quantized at the call: weight codes and every
    intermediate in full, Y on sampled rows."""
    d = synth.opt_ffn_up()
    X, W = d["X"], d["W"]
    M, K = X.shape
    N = W.shape[0]
    note("fp16 weights OPT FFN up")
    ops = gpu.ops
    ws = torch.empty((ops.workspace_bytes(M, K, N),), dtype=torch.uint8, device="cuda")
    Wq = torch.empty((N, K), dtype=torch.int8, device="cuda")
    sw = torch.empty((N,), dtype=torch.float32, device="cuda")
    Y = ops.linear_int8_mixed_fp16_weights(dev(X), dev(W), Wq, sw, True, None, 6.0, ws)
    torch.cuda.synchronize()
    Wq_ref, sw_ref = O.quantize_weight_rows(W)
    assert np.array_equal(host(Wq), Wq_ref)
    assert np.array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))
    rows = sample_rows(M, 64, 3)
    ref = O.linear_int8_mixed_fp16_weights(X, W, 6.0, rows=rows, Wq=Wq_ref, sw=sw_ref)
    v = ops.workspace_views(ws, M, K)
    assert int(host(v["n"])[0]) == ref["n"]
    assert np.array_equal(host(v["Xq"])[rows], ref["Xq"])
    err = y_err(host(Y[torch.from_numpy(rows).cuda()]), ref["Y"])
    assert err <= Y_TOL, err

"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: int8 codes, absmax scales, outlier bitmap / column list / count,
gathered outlier columns, int32 accumulators. Tolerance: fp16 outputs within
max |dY| / max |Y_ref| <= 1e-3 of the oracle's fp64 value.
"""

import numpy as np
import pytest
import torch

from int8_quantized_matmul_absmax_amd import synth
from oracle import llm_int8 as O
from tests.gpu_helpers import Y_TOL, bitmap_u32, dev, f16_ulp, host, note, sample_rows, y_err

pytestmark = pytest.mark.gpu


def _ops(gpu):
    return gpu.ops


# ------------------------------------------------------------------ a4: weight

@pytest.mark.parametrize("shape", [(256, 256), (1000, 4112), (64, 16), (33, 12288), (7, 32)])
def test_weight_quant_bitexact(gpu, shape):
    N, K = shape
    note("weight quant %s" % (shape,))
    rng = np.random.default_rng(N * 7 + K)
    W = synth.normal_f16(rng, (N, K), 0.02)
    W[min(3, N - 1), :] = 0                       # an all-zero row
    Wq_ref, sw_ref = O.quantize_weight_rows(W)
    Wq, sw = _ops(gpu).int8_quantize_colwise_weight(dev(W))
    torch.cuda.synchronize()
    assert np.array_equal(host(Wq), Wq_ref)
    assert np.array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))


def test_weight_quant_ties(gpu):
    note("weight quant ties")
    W = np.zeros((2, 16), np.float16)
    W[0, :4] = [127.0, 2.5, 0.5, -3.5]            # scale 1: 2.5 -> 2, -3.5 -> -4
    W[1, :3] = [np.float16(127 / 32), 0.078125, 0.109375]   # scale 32: 2.5 -> 2, 3.5 -> 4
    Wq, sw = _ops(gpu).int8_quantize_colwise_weight(dev(W))
    assert host(Wq)[0, :4].tolist() == [127, 2, 0, -4]
    assert host(Wq)[1, :3].tolist() == [127, 2, 4]
    Wq_ref, _ = O.quantize_weight_rows(W)
    assert np.array_equal(host(Wq), Wq_ref)


# ------------------------------------------------------------------ a1, a2: detection

def _check_detect(gpu, X, tau):
    M, K = X.shape
    cols_ref = O.detect_outlier_columns(X, tau)
    n_ref = cols_ref.size
    bitmap, cols, n, Xo = _ops(gpu).outlier_detect_gather(dev(X), tau)
    torch.cuda.synchronize()
    assert int(host(n)[0]) == n_ref
    assert np.array_equal(bitmap_u32(bitmap), O.outlier_bitmap(cols_ref, K))
    assert np.array_equal(host(cols)[:n_ref], cols_ref)
    ld = _ops(gpu).outlier_ld(n_ref)
    Xo_h = host(Xo)[: M * ld].reshape(M, ld) if M else np.zeros((0, ld), np.float16)
    assert np.array_equal(Xo_h[:, :n_ref].view(np.uint16), X[:, cols_ref].view(np.uint16))
    assert np.all(Xo_h[:, n_ref:].view(np.uint16) == 0)
    return cols_ref


@pytest.mark.parametrize("case", ["tiny", "planted_ragged", "single_row", "many_outliers"])
def test_outlier_detect_gather(gpu, case):
    note("detect %s" % case)
    if case == "tiny":
        X = synth.tiny()["X"]
    elif case == "planted_ragged":
        X = synth.opt_ffn_up(M=300, K=4112, N=16)["X"]
    elif case == "single_row":
        X = synth.decode(1)["X"]
    else:
        rng = np.random.default_rng(21)
        X = synth.normal_f16(rng, (37, 1040), 1.0)
        synth.plant_outlier_columns(rng, X, 100, 6.0, 9.0, 0.1)
    cols = _check_detect(gpu, X, 6.0)
    assert cols.size >= 1


def test_outlier_threshold_edges(gpu):
    note("detect edges")
    rng = np.random.default_rng(5)
    X = synth.normal_f16(rng, (9, 160), 1.0)
    X = np.clip(X.astype(np.float32), -5.5, 5.5).astype(np.float16)
    X[4, 13] = 6.0                     # exactly tau: outlier (>=)
    X[2, 140] = -6.0
    X[0, 15] = np.float16(5.99609375)  # just below: not an outlier
    cols = _check_detect(gpu, X, 6.0)
    assert cols.tolist() == [13, 140]
    assert _check_detect(gpu, X, float("inf")).size == 0
    assert _check_detect(gpu, X, 0.0).size == 160
    assert _check_detect(gpu, X, -1.0).size == 160


def test_outlier_nan_inf_columns(gpu):
    note("detect nan/inf")
    rng = np.random.default_rng(6)
    X = synth.normal_f16(rng, (33, 528), 1.0)
    X = np.clip(X.astype(np.float32), -5.0, 5.0).astype(np.float16)
    X[7, 70] = np.float16(np.nan)
    X[30, 300] = np.float16(np.inf)
    X[0, 500] = np.float16(-7.0)
    assert _check_detect(gpu, X, 6.0).tolist() == [70, 300, 500]
    assert _check_detect(gpu, X, float("inf")).tolist() == [70, 300]
    assert _check_detect(gpu, X, 1e9).tolist() == [70, 300]
    # the int8 path stays finite: codes and scales exclude those columns
    cols = O.detect_outlier_columns(X, 6.0)
    Xq_ref, sx_ref = O.quantize_activation_rows(X, cols)
    Xq, sx = _ops(gpu).int8_quantize_rowwise(dev(X), dev(O.outlier_bitmap(cols, 528).view(np.int32)))
    torch.cuda.synchronize()
    assert np.array_equal(host(Xq), Xq_ref)
    assert np.array_equal(host(sx).view(np.uint32), sx_ref.view(np.uint32))


def test_outlier_detect_empty_rows(gpu):
    note("detect M=0")
    X = torch.empty((0, 64), dtype=torch.float16, device="cuda")
    bitmap, cols, n, Xo = _ops(gpu).outlier_detect_gather(X, 6.0)
    torch.cuda.synchronize()
    assert int(host(n)[0]) == 0 and np.all(host(bitmap) == 0)


# ------------------------------------------------------------------ a3: rows of X

def _subnormal_rows(rng, X, rows):
    """Rows made of fp16 subnormals (exponent field 0, random sign), so that
    a row's absmax and every product x * s come from subnormal inputs."""
    bits = rng.integers(1, 0x400, size=(len(rows), X.shape[1]), dtype=np.uint16)
    bits |= (rng.integers(0, 2, size=bits.shape, dtype=np.uint16) << 15)
    X[rows] = bits.view(np.float16)


@pytest.mark.parametrize("case", ["tiny", "medium", "no_bitmap", "subnormal"])
def test_rowwise_quant_bitexact(gpu, case):
    note("rowwise %s" % case)
    if case == "tiny":
        X = synth.tiny()["X"]
    else:
        X = synth.opt_ffn_up(M=257, K=4096, N=16)["X"]
    X[1, :] = 0
    if case == "subnormal":
        rng = np.random.default_rng(77)
        _subnormal_rows(rng, X, [0, 2, 100, 256])
        X[3, ::7] = np.float16(6e-8)    # subnormal elements in a normal row
    if case == "no_bitmap":
        cols = np.zeros(0, np.int32)
        bm = None
    else:
        cols = O.detect_outlier_columns(X, 6.0)
        bm = dev(O.outlier_bitmap(cols, X.shape[1]).view(np.int32))
    Xq_ref, sx_ref = O.quantize_activation_rows(X, cols)
    Xq, sx = _ops(gpu).int8_quantize_rowwise(dev(X), bm)
    torch.cuda.synchronize()
    assert np.array_equal(host(Xq), Xq_ref)
    assert np.array_equal(host(sx).view(np.uint32), sx_ref.view(np.uint32))


# ------------------------------------------------------------------ a5: int32 GEMM

@pytest.mark.parametrize("mnk", [(1, 1, 16), (7, 50, 48), (130, 260, 272), (300, 1000, 4112),
                                 (16, 4096, 4096), (256, 384, 1024), (17, 33, 272),
                                 (33, 130, 1040), (64, 64, 4096), (65, 40, 528), (63, 17, 8208),
                                 (4100, 4100, 272)])
def test_int32_accumulators_bitexact(gpu, mnk):
    M, N, K = mnk
    note("int32 gemm %s" % (mnk,))
    Xq = synth.random_codes(M + 1, (M, K))
    Wq = synth.random_codes(N + 2, (N, K))
    C_ref = O.int32_accumulators(Xq, Wq)
    sx = np.ones(M, np.float32)
    sw = np.ones(N, np.float32)
    C = _ops(gpu).int8_mm_dequant(dev(Xq), dev(Wq), dev(sx), dev(sw), want_y=False,
                                  want_int32=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(C), C_ref)


def test_int32_accumulators_extremes(gpu):
    note("int32 gemm extremes")
    M, N, K = 64, 96, 8192
    Xq = np.full((M, K), 127, np.int8)
    Xq[1::2] = -127
    Wq = np.full((N, K), -127, np.int8)
    C = _ops(gpu).int8_mm_dequant(dev(Xq), dev(Wq), dev(np.ones(M, np.float32)),
                                  dev(np.ones(N, np.float32)), want_y=False, want_int32=True)
    C_ref = O.int32_accumulators(Xq, Wq)
    assert np.array_equal(host(C), C_ref)
    assert int(np.abs(C_ref).max()) == K * 127 * 127


# ------------------------------------------------------------------ a7: the fp32 dequantize order

def _dequant_fp32(C, sx, sw, bias):
    """fp16(fl32(fl32(fl32(C) * fl32(sx / 127)) * fl32(sw / 127)) + bias) in
    IEEE single precision (numpy's float32 operations round to nearest even,
    as does its float32 -> float16 conversion): the order in which every
    kernel forms an output with no outlier column. The oracle's fp64 value
    only bounds this within the 1e-3 bar; this pins the fp32 arithmetic and
    the final rounding bit for bit."""
    ax = sx.astype(np.float32) / np.float32(127.0)
    fw = sw.astype(np.float32) / np.float32(127.0)
    with np.errstate(over="ignore"):
        y = (C.astype(np.float32) * ax[:, None]) * fw[None, :]
        if bias is not None:
            y = y + bias.astype(np.float32)[None, :]
        return y.astype(np.float16)


# (M, N, K, bias): 256 x 256 tiles with ragged token and feature tiles, with
# N not a multiple of 8 (element stores), with whole ones only, 128 x 128
# tiles with N not a multiple of 8, few-token GEMV
DEQUANT_CASES = {
    "large_ragged": (1000, 16392, 128, False),
    "large_n_odd_bias": (1030, 16388, 64, True),
    "large_whole_bias": (1024, 16384, 192, True),
    "small_n_odd_bias": (300, 1003, 272, True),
    "gemv": (40, 520, 1040, False),
}


@pytest.mark.parametrize("case", sorted(DEQUANT_CASES))
def test_dequant_fp32_order(gpu, case):
    """int8_mm_dequant without outlier columns against the fp32 expression,
    with scales over six decades so that outputs reach the fp16 subnormals
    and overflow to infinity."""
    M, N, K, with_bias = DEQUANT_CASES[case]
    note("dequant fp32 order %s" % case)
    rng = np.random.default_rng(4400 + M + N)
    Xq = synth.random_codes(M + 11, (M, K))
    Wq = synth.random_codes(N + 13, (N, K))
    sx = np.exp(rng.uniform(np.log(1e-4), np.log(1e3), M)).astype(np.float32)
    sw = np.exp(rng.uniform(np.log(1e-3), np.log(1e2), N)).astype(np.float32)
    b = synth.normal_f16(rng, (N,), 0.5) if with_bias else None
    Y = _ops(gpu).int8_mm_dequant(dev(Xq), dev(Wq), dev(sx), dev(sw),
                                  bias=None if b is None else dev(b))
    torch.cuda.synchronize()
    Y_ref = _dequant_fp32(O.int32_accumulators(Xq, Wq), sx, sw, b)
    tiny = (Y_ref != 0) & (np.abs(Y_ref) < np.float16(6.1e-5))   # fp16 subnormals
    assert np.isinf(Y_ref).any() and tiny.any()
    assert np.array_equal(host(Y).view(np.uint16), Y_ref.view(np.uint16))


@pytest.mark.parametrize("M", [1, 8, 40, 520])
def test_layer_dequant_fp32_order(gpu, M):
    """The whole layer on X without outlier columns (the single-launch decode
    for 1 and 8 tokens, the GEMV for 40, the tiled GEMM for 520): Y equals
    the fp32 expression over the oracle's codes and scales bit for bit."""
    note("layer dequant fp32 order M=%d" % M)
    K, N = 4096, 1000
    rng = np.random.default_rng(4500 + M)
    X = np.clip(synth.normal_f16(rng, (M, K), 1.0).astype(np.float32), -5.0, 5.0).astype(np.float16)
    W = synth.normal_f16(rng, (N, K), 0.02)
    b = synth.normal_f16(rng, (N,), 0.5) if M % 2 == 0 else None
    Wq, sw = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq, sw, 6.0, b)
    assert ref["n"] == 0
    Y, _ = _run_linear(gpu, X, Wq, sw, bias=b)
    Y_ref = _dequant_fp32(ref["C"], ref["sx"], sw, b)
    assert np.array_equal(Y.view(np.uint16), Y_ref.view(np.uint16))


# ------------------------------------------------------------------ whole layer

def _run_linear(gpu, X, Wq_ref, sw_ref, tau=6.0, bias=None):
    """GPU layer from the oracle's own quantized weight (uploaded), returns
    (Y, workspace views)."""
    ops = _ops(gpu)
    M, K = X.shape
    ws = torch.empty((ops.workspace_bytes(M, K),), dtype=torch.uint8, device="cuda")
    Y = ops.linear_int8_mixed(dev(X), dev(Wq_ref), dev(sw_ref),
                              None if bias is None else dev(bias), tau, ws)
    torch.cuda.synchronize()
    return host(Y), ops.workspace_views(ws, M, K)


def _check_intermediates(gpu, views, X, ref):
    M, K = X.shape
    n = ref["n"]
    assert int(host(views["n"])[0]) == n
    assert np.array_equal(host(views["cols"])[:n], ref["cols"])
    assert np.array_equal(host(views["bitmap"]).view(np.uint32), O.outlier_bitmap(ref["cols"], K))
    assert np.array_equal(host(views["Xq"]), ref["Xq"])
    assert np.array_equal(host(views["sx"]).view(np.uint32), ref["sx"].view(np.uint32))
    ld = _ops(gpu).outlier_ld(n)
    Xo = host(views["Xo"])[: M * ld].reshape(M, ld)
    assert np.array_equal(Xo[:, :n].view(np.uint16), X[:, ref["cols"]].view(np.uint16))
    assert not np.any(Xo[:, n:ld].view(np.uint16))   # pad columns hold +0.0


@pytest.mark.parametrize("case", ["tiny", "decode1", "decode4", "decode16", "medium_ragged",
                                  "bias"])
def test_linear_full_oracle(gpu, case):
    note("linear %s" % case)
    if case == "tiny":
        d = synth.tiny()
    elif case.startswith("decode"):
        d = synth.decode(int(case[6:]))
    elif case == "medium_ragged":
        d = synth.opt_ffn_up(M=300, K=4112, N=1000)
    else:
        d = synth.opt_ffn_up(M=130, K=1024, N=520)
    X, W = d["X"], d["W"]
    Wq, sw = O.quantize_weight_rows(W)
    bias = None
    if case == "bias":
        bias = synth.normal_f16(np.random.default_rng(3), (W.shape[0],), 0.5)
    ref = O.linear_int8_mixed(X, Wq, sw, 6.0, bias)
    Y, views = _run_linear(gpu, X, Wq, sw, 6.0, bias)
    _check_intermediates(gpu, views, X, ref)
    assert set(d["planted"].tolist()) <= set(ref["cols"].tolist())
    err = y_err(Y, ref["Y"])
    assert err <= Y_TOL, err
    # the dequantized int8 part and the fp16 part both matter on these inputs
    assert np.abs(ref["Yo"]).max() > 0


@pytest.mark.parametrize("case", ["tau_zero_all_outliers", "tau_inf_none", "n17", "n33",
                                  "exact_threshold", "zero_rows", "k16", "three_d"])
def test_linear_edge_cases(gpu, case):
    note("linear edge %s" % case)
    rng = np.random.default_rng(17)
    tau = 6.0
    if case == "k16":
        X = synth.normal_f16(rng, (5, 16), 2.0)
        W = synth.normal_f16(rng, (70, 16), 0.1)
    else:
        X = synth.normal_f16(rng, (70, 512), 1.0)
        W = synth.normal_f16(rng, (150, 512), 0.05)
    if case == "tau_zero_all_outliers":
        tau = 0.0
    elif case == "tau_inf_none":
        tau = float("inf")
    elif case in ("n17", "n33"):
        synth.plant_outlier_columns(rng, X, int(case[1:]), 7.0, 30.0, 0.3)
    elif case == "exact_threshold":
        X = np.clip(X.astype(np.float32), -5.0, 5.0).astype(np.float16)
        X[3, 100] = 6.0
        X[10, 7] = -6.0
    elif case == "zero_rows":
        X[0, :] = 0
        X[5, :] = 0
        X[5, 9] = 20.0
    Wq, sw = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq, sw, tau)
    if case == "three_d":
        ops = _ops(gpu)
        Y3 = ops.linear_int8_mixed(dev(X).reshape(7, 10, 512), dev(Wq), dev(sw), None, tau)
        torch.cuda.synchronize()
        assert tuple(Y3.shape) == (7, 10, 150)
        assert y_err(host(Y3).reshape(70, 150), ref["Y"]) <= Y_TOL
        return
    Y, views = _run_linear(gpu, X, Wq, sw, tau)
    _check_intermediates(gpu, views, X, ref)
    assert y_err(Y, ref["Y"]) <= Y_TOL
    if case == "tau_zero_all_outliers":
        assert ref["n"] == X.shape[1]
    if case == "exact_threshold":
        assert ref["cols"].tolist() == [7, 100]
    if case in ("n17", "n33"):
        assert ref["n"] >= int(case[1:])


@pytest.mark.parametrize("case", ["n17", "n33", "n70", "n100", "all_columns", "large_tiles_n40",
                                  "large_tiles_all", "wide_all", "n600", "block_run",
                                  "tail_block", "chunks3_all"])
def test_linear_many_outliers(gpu, case):
    """More than 16 outlier columns, three workspaces: the minimal one, the
    default region of recovered weights (workspace_bytes(M, K, N), room for
    512 columns) and a region with room for every count
    (workspace_bytes_all_outliers). With room for the n columns the recovered
    weights are materialized, bit for bit against the oracle, and the outlier
    product runs as a second GEMM loop over them; its Y is bit-identical to
    the step call's, which adds the same fp16 MFMA products in the same order
    in the epilogue. Without room the GEMM's dense second loop runs over all
    K columns (all columns outliers: the int8 loop is skipped). Every Y within
    the tolerance of the oracle. wide_all: N * LD(K) / 8 = 1.07M 16-byte
    pieces, more than one pass of the recovery's grid. chunks3_all: rows of
    three 2048-column chunks on a grid of 2048 blocks, so a block's chunk
    changes from task to task (96 tokens: at most 64 the few-token kernel
    takes the layer and no weights are recovered). block_run and
    tail_block make whole 64-column k-blocks outlier columns (ten in a row;
    the partial last block), which the int8 loop of the segment modes skips:
    their codes are all zero, so the int32 sums, and Y against the step
    call, stay bit for bit."""
    note("linear many outliers %s" % case)
    rng = np.random.default_rng(300 + len(case))
    large = case.startswith("large_tiles")
    M, K, N = (4100, 528, 4100) if large else (300, 2064, 4100) if case in ("wide_all", "n600") \
        else (96, 4224, 2100) if case == "chunks3_all" else (200, 1040, 300)
    X = synth.normal_f16(rng, (M, K), 1.0)
    W = synth.normal_f16(rng, (N, K), 0.05)
    tau = 6.0
    if case.endswith("all") or case == "all_columns":
        tau = 0.0
    elif case in ("block_run", "tail_block"):
        run = list(range(64, 704)) if case == "block_run" else list(range(100, 140)) + \
            list(range(1024, 1040))
        rows = rng.integers(0, M, size=len(run))
        X[rows, run] = np.where(rng.random(len(run)) < 0.5, -7.5, 7.5).astype(np.float16)
    else:
        n_plant = int(case.split("n")[-1])
        synth.plant_outlier_columns(rng, X, n_plant, 7.0, 30.0, (0.05, 0.6))
    bias = synth.normal_f16(rng, (N,), 0.5)
    Wq, sw = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq, sw, tau, bias)
    assert ref["n"] > 16
    ops = _ops(gpu)
    ws_all = torch.empty((ops.workspace_bytes_all_outliers(M, K, N),), dtype=torch.uint8,
                         device="cuda")
    ws_big = torch.empty((ops.workspace_bytes(M, K, N),), dtype=torch.uint8, device="cuda")
    ws_small = torch.empty((ops.workspace_bytes(M, K),), dtype=torch.uint8, device="cuda")
    assert ops.outlier_region_cols(ws_all.numel(), M, K, N) == ops.outlier_ld(K)
    Xd, Wqd, swd, bd = dev(X), dev(Wq), dev(sw), dev(bias)
    Y_big = ops.linear_int8_mixed(Xd, Wqd, swd, bd, tau, ws_big)
    Y_small = ops.linear_int8_mixed(Xd, Wqd, swd, bd, tau, ws_small)
    Y_all = ops.linear_int8_mixed(Xd, Wqd, swd, bd, tau, ws_all)
    torch.cuda.synchronize()
    views = ops.workspace_views(ws_all, M, K, N)
    _check_intermediates(gpu, views, X, ref)
    for Y in (Y_big, Y_small, Y_all):
        assert y_err(host(Y), ref["Y"]) <= Y_TOL
    # the recovered weights, bit for bit, and their zero pad
    n, ld = ref["n"], ops.outlier_ld(ref["n"])
    Wo = host(views["Wo"])[: N * ld].reshape(N, ld).view(np.uint16)
    Wo_ref = O.recover_outlier_weights(Wq, sw, ref["cols"]).view(np.uint16)
    assert np.array_equal(Wo[:, :n], Wo_ref)
    assert not Wo[:, n:].any()
    Y_step = ops.int8_mm_dequant(views["Xq"], Wqd, views["sx"], swd, views["Xo"],
                                 views["cols"], views["n"], bd)
    torch.cuda.synchronize()
    assert np.array_equal(host(Y_all).view(np.uint16), host(Y_step).view(np.uint16))
    if n <= ops.OUTLIER_REGION_COLS:
        assert np.array_equal(host(Y_big).view(np.uint16), host(Y_step).view(np.uint16))
    else:
        # no room for that many in the default region: it takes the dense
        # loop, as the minimal workspace does
        assert np.array_equal(host(Y_big).view(np.uint16), host(Y_small).view(np.uint16))


@pytest.mark.parametrize("case", ["clustered", "ragged_k", "sparse_words", "small_tiles_all",
                                  "large_tiles_600", "wide_rows_many", "widest_rows_many"])
def test_linear_dense_outlier_loop(gpu, case):
    """The GEMM's dense second loop (the workspace without the region of
    recovered weights): outlier columns clustered in a few 32-column words
    (the other words' stages issue no MFMA), K with a half-empty last stage
    (K % 32 == 16), outlier columns spread one per word, every column an
    outlier on the 128 x 128 tiles, 600 columns on the 256 x 256 tiles
    with ragged M and N, and rows wider than 12288 with about 3000 outlier
    columns at unaligned positions over more token rows than row-pass
    blocks (the row pass then assembles Xo in LDS, two rows per block, with
    an odd number of bitmap words, and at K = 16384, where its two row
    buffers need more than 64 KB of LDS). Intermediates bit for bit, Y within the tolerance;
    with the int32 step call, the accumulators of the normal part bit for
    bit."""
    note("dense outlier loop %s" % case)
    rng = np.random.default_rng(640 + len(case))
    M, K, N = {"clustered": (300, 2048, 700), "ragged_k": (200, 1040, 330),
               "sparse_words": (130, 2048, 260), "small_tiles_all": (256, 1024, 384),
               "large_tiles_600": (4100, 2064, 4100), "wide_rows_many": (1100, 13008, 64),
               "widest_rows_many": (1100, 16384, 64)}[case]
    X = np.clip(synth.normal_f16(rng, (M, K), 1.0).astype(np.float32), -5.0, 5.0).astype(np.float16)
    tau = 6.0
    if case == "clustered":
        cols = np.concatenate([np.arange(64, 96), np.arange(1000, 1010), np.arange(2040, 2048)])
    elif case == "ragged_k":
        cols = np.concatenate([np.arange(0, 20), np.arange(1030, 1040)])
    elif case == "sparse_words":
        cols = np.arange(5, K, 32)
    elif case == "small_tiles_all":
        cols, tau = np.arange(K), 0.0
    elif case in ("wide_rows_many", "widest_rows_many"):
        cols = np.unique(np.concatenate([np.arange(96, 136), rng.choice(K, 3000, replace=False)]))
    else:
        cols = np.sort(rng.choice(K, 600, replace=False))
    for c in cols:
        rows = rng.choice(M, size=max(1, M // 4), replace=False)
        X[rows, c] = (rng.uniform(7.0, 40.0, rows.size) * rng.choice([-1.0, 1.0], rows.size)).astype(np.float16)
    W = synth.normal_f16(rng, (N, K), 0.05)
    bias = synth.normal_f16(rng, (N,), 0.5)
    Wq, sw = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq, sw, tau, bias)
    if tau > 0:
        assert ref["cols"].tolist() == sorted(cols.tolist())
    Y, views = _run_linear(gpu, X, Wq, sw, tau, bias)
    _check_intermediates(gpu, views, X, ref)
    err = y_err(Y, ref["Y"])
    assert err <= Y_TOL, err
    ops = _ops(gpu)
    C = ops.int8_mm_dequant(views["Xq"], dev(Wq), views["sx"], dev(sw), want_y=False,
                            want_int32=True)
    torch.cuda.synchronize()
    rows = sample_rows(M, 64, 7)
    assert np.array_equal(host(C)[rows], O.int32_accumulators(ref["Xq"][rows], Wq))


def test_linear_large_tiles_ragged(gpu):
    """A shape with enough 256 x 256 tiles for the large-tile GEMM, ragged in M
    and N, with outlier columns and a bias."""
    note("linear large tiles ragged")
    rng = np.random.default_rng(41)
    X = synth.normal_f16(rng, (4100, 528), 1.0)
    W = synth.normal_f16(rng, (4100, 528), 0.05)
    synth.plant_outlier_columns(rng, X, 9, 7.0, 30.0, 0.5)
    bias = synth.normal_f16(rng, (4100,), 0.5)
    Wq, sw = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq, sw, 6.0, bias)
    Y, views = _run_linear(gpu, X, Wq, sw, 6.0, bias)
    _check_intermediates(gpu, views, X, ref)
    assert y_err(Y, ref["Y"]) <= Y_TOL


@pytest.mark.parametrize("M", [1, 2, 15, 16, 17, 31, 33, 48, 63, 64, 65, 97])
def test_linear_token_counts(gpu, M):
    """Token counts around the 16-token groups of the few-token path and its
    hand-over to the tiled GEMM, with ragged N and K and 20 outlier columns."""
    note("linear M=%d" % M)
    rng = np.random.default_rng(100 + M)
    X = synth.normal_f16(rng, (M, 1040), 1.0)
    W = synth.normal_f16(rng, (300, 1040), 0.05)
    synth.plant_outlier_columns(rng, X, 20, 7.0, 30.0, (0.0, 1.0))
    Wq, sw = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq, sw, 6.0)
    Y, views = _run_linear(gpu, X, Wq, sw, 6.0)
    _check_intermediates(gpu, views, X, ref)
    assert y_err(Y, ref["Y"]) <= Y_TOL
    C = _ops(gpu).int8_mm_dequant(views["Xq"], dev(Wq), views["sx"], dev(sw), want_y=False,
                                  want_int32=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(C), O.int32_accumulators(ref["Xq"], Wq))


@pytest.mark.parametrize("M", [1, 3, 16])
@pytest.mark.parametrize("case", ["mixed", "tau_zero", "no_outliers"])
def test_linear_few_tokens_x_side(gpu, M, case):
    """Few tokens: bitmap, cols, n, codes, scales and gathered outliers against
    the oracle, with K not a multiple of 32, an exact +-6.0, a NaN column, an
    inf column, threshold 0 (every column) and a case with no outlier column."""
    note("few tokens x side M=%d %s" % (M, case))
    rng = np.random.default_rng(500 + M)
    K = 528
    X = synth.normal_f16(rng, (M, K), 1.0)
    W = synth.normal_f16(rng, (77, K), 0.05)
    tau = 6.0
    if case == "mixed":
        X[0, 3] = 6.0
        X[M - 1, 200] = -6.0
        X[0, 517] = np.float16(np.inf)
        X[M // 2, 40] = np.float16(np.nan)
        X[:, 301] = 9.5
    elif case == "tau_zero":
        tau = 0.0
    else:
        X = np.clip(X.astype(np.float32), -5.0, 5.0).astype(np.float16)
    Wq, sw = O.quantize_weight_rows(W)
    with np.errstate(invalid="ignore"):   # the planted NaN reaches the oracle's sums
        ref = O.linear_int8_mixed(X, Wq, sw, tau)
    Y, views = _run_linear(gpu, X, Wq, sw, tau)
    _check_intermediates(gpu, views, X, ref)
    if case == "mixed":
        assert {3, 40, 200, 301, 517} <= set(ref["cols"].tolist())
        # The NaN (row M//2) and the inf (row 0) reach Y only through the fp16
        # outlier product of their own rows: every other row is finite and
        # within the tolerance, and an output the oracle makes non-finite is
        # non-finite on the GPU too.
        bad = {0, M // 2}
        finite_rows = np.array([i for i in range(M) if i not in bad], dtype=np.int64)
        assert np.all(np.isfinite(ref["Y"][finite_rows]))
        if finite_rows.size:
            assert y_err(Y[finite_rows], ref["Y"][finite_rows]) <= Y_TOL
        nonfinite = ~np.isfinite(ref["Y"])
        assert nonfinite[M // 2].all()          # NaN times every weight
        assert not np.isfinite(Y.astype(np.float64)[nonfinite]).any()
        return
    assert y_err(Y, ref["Y"]) <= Y_TOL


def test_linear_is_deterministic(gpu):
    note("determinism")
    d = synth.opt_ffn_up(M=200, K=1024, N=700)
    Wq, sw = O.quantize_weight_rows(d["W"])
    Y1, _ = _run_linear(gpu, d["X"], Wq, sw)
    Y2, _ = _run_linear(gpu, d["X"], Wq, sw)
    assert np.array_equal(Y1.view(np.uint16), Y2.view(np.uint16))


def test_mm_dequant_matches_linear(gpu):
    """The step-level calls composed by hand give the same bits as the fused call."""
    note("composed steps")
    d = synth.opt_ffn_up(M=96, K=1024, N=384)
    ops = _ops(gpu)
    X = dev(d["X"])
    Wq, sw = ops.int8_quantize_colwise_weight(dev(d["W"]))
    bitmap, cols, n, Xo = ops.outlier_detect_gather(X, 6.0)
    Xq, sx = ops.int8_quantize_rowwise(X, bitmap)
    Y1 = ops.int8_mm_dequant(Xq, Wq, sx, sw, Xo, cols, n)
    Y2 = ops.linear_int8_mixed(X, Wq, sw)
    torch.cuda.synchronize()
    assert np.array_equal(host(Y1).view(np.uint16), host(Y2).view(np.uint16))


def test_int8_linear_module(gpu):
    note("Int8Linear")
    d = synth.tiny()
    lin = gpu.Int8Linear(256, 256)
    lin.quantize_(dev(d["W"]))
    with pytest.raises(RuntimeError):
        lin.quantize_(dev(d["W"]))
    Wq_ref, sw_ref = O.quantize_weight_rows(d["W"])
    assert np.array_equal(host(lin.CB), Wq_ref)
    Y = lin(dev(d["X"]))
    torch.cuda.synchronize()
    ref = O.linear_int8_mixed(d["X"], Wq_ref, sw_ref)
    assert y_err(host(Y), ref["Y"]) <= Y_TOL
    with pytest.raises(TypeError):
        lin(dev(d["X"]).float())


def test_gelu(gpu):
    note("gelu")
    rng = np.random.default_rng(8)
    X = synth.normal_f16(rng, (4099,), 3.0)
    # signed zero, the fp16 extremes and large magnitudes, in the 8-element
    # groups and in the partial last group (4099 = 512 * 8 + 3)
    X[[0, 1, 2, 3, 4096, 4097, 4098]] = np.array(
        [-0.0, 65504.0, -65504.0, -20.0, 20.0, -9.5, 1e-7], np.float32).astype(np.float16)
    Y = host(_ops(gpu).gelu_f16(dev(X)))
    ref = O.gelu_erf(X.astype(np.float64))
    ref16 = ref.astype(np.float16)
    # within one fp16 ulp of the correctly rounded fp64 value (the ulp of the
    # top binade at +-65504: finite, so the extremes are really checked)
    ulp = f16_ulp(ref16)
    assert np.all(np.isfinite(ulp))
    assert np.all(np.abs(Y.astype(np.float64) - ref16.astype(np.float64)) <= ulp + 1e-12)
    assert Y[1] == np.float16(65504.0) and Y[2] == 0.0


def test_int8_linear_save_load(gpu, tmp_path):
    """The quantized pair saved and loaded (file and state dict) gives the
    oracle's module: CB and SCB bit for bit equal to the oracle's quantization
    of W, the output of each reloaded module within the tolerance of the
    oracle's layer on those codes, the same output bits as the module it came
    from, and no second quantization ([HF-blog] "Saving 8-bit state dicts on
    the Hub")."""
    note("Int8Linear save/load")
    rng = np.random.default_rng(77)
    W = synth.normal_f16(rng, (96, 256), 0.05)
    b = synth.normal_f16(rng, (96,), 0.5)
    X = synth.normal_f16(rng, (40, 256), 1.0)
    X[:, 7] = 12.0
    Wq_ref, sw_ref = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq_ref, sw_ref, 6.0, b)
    assert ref["n"] >= 1

    def check_module(m):
        assert m.quantized
        assert np.array_equal(host(m.CB), Wq_ref)
        assert np.array_equal(host(m.SCB).view(np.uint32), sw_ref.view(np.uint32))
        Ym = host(m(dev(X)))
        assert y_err(Ym, ref["Y"]) <= Y_TOL
        return Ym

    lin = gpu.Int8Linear(256, 96, bias=True)
    lin.quantize_(dev(W), dev(b))
    Y0 = check_module(lin)
    p = str(tmp_path / "lin.safetensors")
    lin.save_int8(p)
    lin2 = gpu.Int8Linear.from_int8_file(p)
    assert np.array_equal(check_module(lin2).view(np.uint16), Y0.view(np.uint16))
    with pytest.raises(RuntimeError):
        lin2.quantize_(dev(W))
    sd = str(tmp_path / "lin.pt")
    torch.save(lin.state_dict(), sd)
    lin3 = gpu.Int8Linear(256, 96, bias=True)
    lin3.load_state_dict(torch.load(sd, weights_only=True))
    assert np.array_equal(check_module(lin3).view(np.uint16), Y0.view(np.uint16))


@pytest.mark.parametrize("M", [3, 40, 300])
def test_empty_k(gpu, M):
    """K == 0: every product is an empty sum ([Summary] "The full picture" with
    no hidden features). On each token path (few-token, GEMV range, tiled) the
    layer returns Y = bias exactly, with no outlier column and every row
    scale 0, as the oracle does; so do the fp16-weight layer and the step
    calls (weight scales 0, C = 0)."""
    note("empty K, M=%d" % M)
    ops = _ops(gpu)
    N = 150
    X = np.zeros((M, 0), np.float16)
    W = np.zeros((N, 0), np.float16)
    bias = synth.normal_f16(np.random.default_rng(41), (N,), 0.5)
    Wq, sw = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq, sw, 6.0, bias)
    assert ref["n"] == 0
    ref_bits = ref["Y"].astype(np.float16).view(np.uint16)
    Wqd, swd = ops.int8_quantize_colwise_weight(dev(W))
    ws = torch.empty((ops.workspace_bytes(M, 0),), dtype=torch.uint8, device="cuda")
    Y = ops.linear_int8_mixed(dev(X), Wqd, swd, dev(bias), 6.0, ws)
    torch.cuda.synchronize()
    assert tuple(Wqd.shape) == (N, 0)
    assert np.array_equal(host(swd).view(np.uint32), sw.view(np.uint32))
    assert np.array_equal(host(Y).view(np.uint16), ref_bits)
    views = ops.workspace_views(ws, M, 0)
    assert int(host(views["n"])[0]) == 0
    assert not host(views["sx"]).view(np.uint32).any()
    Yw = ops.linear_int8_mixed_fp16_weights(dev(X), dev(W), Wqd, swd, True, dev(bias), 6.0, ws)
    Xq, sx = ops.int8_quantize_rowwise(dev(X))
    _, _, n, _ = ops.outlier_detect_gather(dev(X), 6.0)
    Ys, C = ops.int8_mm_dequant(Xq, Wqd, sx, swd, bias=dev(bias), want_int32=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(Yw).view(np.uint16), ref_bits)
    assert not host(sx).view(np.uint32).any() and int(host(n)[0]) == 0
    assert np.array_equal(host(Ys).view(np.uint16), ref_bits)
    assert not host(C).any()


@pytest.mark.parametrize("case", ["small_tiles", "large_tiles"])
def test_outlier_columns_at_block_edges(gpu, case):
    """The first 16 outlier columns' weight codes are taken from the GEMM's
    staged k-blocks of 64 columns: columns sharing a k-block, on both sides
    of a k-block boundary, column 0, and the last column of a partial last
    k-block (K % 64 != 0); all 16 slots filled (small tiles) or 10 (large
    tiles). Intermediates bit for bit, C bit for bit (int32 step call), Y
    within the tolerance."""
    note("outlier columns at block edges %s" % case)
    rng = np.random.default_rng(900 + len(case))
    if case == "small_tiles":
        M, K, N = 300, 1040, 260
        cols = [0, 1, 15, 16, 63, 64, 65, 127, 128, 500, 511, 512, 1000, 1023, 1024, 1039]
    else:
        M, K, N = 4100, 528, 4100
        cols = [0, 1, 63, 64, 255, 256, 511, 512, 520, 527]
    X = np.clip(synth.normal_f16(rng, (M, K), 1.0).astype(np.float32), -5.0, 5.0).astype(np.float16)
    for c in cols:
        rows = rng.choice(M, size=max(1, M // 8), replace=False)
        X[rows, c] = (rng.uniform(7.0, 30.0, rows.size) * rng.choice([-1.0, 1.0], rows.size)).astype(np.float16)
    W = synth.normal_f16(rng, (N, K), 0.05)
    Wq, sw = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq, sw, 6.0)
    assert ref["cols"].tolist() == cols
    Y, views = _run_linear(gpu, X, Wq, sw, 6.0)
    _check_intermediates(gpu, views, X, ref)
    assert y_err(Y, ref["Y"]) <= Y_TOL
    ops = _ops(gpu)
    Y2, C = ops.int8_mm_dequant(views["Xq"], dev(Wq), views["sx"], dev(sw), views["Xo"],
                                views["cols"], views["n"], want_int32=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(C), O.int32_accumulators(ref["Xq"], Wq))
    assert np.array_equal(host(Y2).view(np.uint16), Y.view(np.uint16))


@pytest.mark.parametrize("shape", [(1, 528), (300, 4112), (2048, 4096)])
def test_outlier_detect_quantize(gpu, shape):
    """The activation side alone (detection, gather, row quantization) writes
    the oracle's intermediates, the same workspace bytes as the whole layer
    call, and int8_mm_dequant on that workspace gives the layer's Y bits and
    the oracle's int32 accumulators."""
    M, K = shape
    note("outlier_detect_quantize M=%d K=%d" % (M, K))
    ops = _ops(gpu)
    rng = np.random.default_rng(4000 + M)
    X = synth.normal_f16(rng, (M, K), 1.0)
    synth.plant_outlier_columns(rng, X, 7, 7.0, 30.0, 0.3)
    X[0, 5] = 6.0
    N = 160
    W = synth.normal_f16(rng, (N, K), 0.03)
    Wq, sw = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq, sw, 6.0)
    ws = ops.outlier_detect_quantize(dev(X), 6.0)
    torch.cuda.synchronize()
    v = ops.workspace_views(ws, M, K)
    _check_intermediates(gpu, v, X, ref)
    Y_l, v_l = _run_linear(gpu, X, Wq, sw, 6.0)
    lay = ops.workspace_layout(M, K)
    n = ref["n"]
    for key in ("bitmap", "n", "sx", "Xq"):
        assert np.array_equal(host(v[key]), host(v_l[key])), key
    # only the first n entries of cols are defined
    assert np.array_equal(host(v["cols"])[:n], host(v_l["cols"])[:n])
    ld = ops.outlier_ld(n)
    assert np.array_equal(host(v["Xo"])[: M * ld], host(v_l["Xo"])[: M * ld])
    Y, C = ops.int8_mm_dequant(v["Xq"], dev(Wq), v["sx"], dev(sw), v["Xo"], v["cols"], v["n"],
                               want_int32=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(C), O.int32_accumulators(ref["Xq"], Wq))
    assert y_err(host(Y), ref["Y"]) <= Y_TOL
    # the layer forms the same fp32 sums from the same intermediates (on the
    # few-token path too, whose single launch matches the separate kernels)
    assert np.array_equal(host(Y).view(np.uint16), Y_l.view(np.uint16))
    assert lay["total"] == ops.workspace_bytes(M, K)


def test_int8_linear_modules_share_one_workspace(gpu):
    """Modules of different shapes, called in turn on one stream, use one
    shared workspace (grown to the largest need) and each output is the
    oracle's."""
    note("Int8Linear shared workspace")
    from int8_quantized_matmul_absmax_amd import linear as L
    rng = np.random.default_rng(88)
    shapes = [(512, 96, 40), (1040, 300, 130), (512, 64, 7)]   # (in, out, tokens)
    mods, refs, xs = [], [], []
    for k, n, m in shapes:
        W = synth.normal_f16(rng, (n, k), 0.05)
        X = synth.normal_f16(rng, (m, k), 1.0)
        synth.plant_outlier_columns(rng, X, 20, 7.0, 30.0, 0.5)
        lin = gpu.Int8Linear(k, n)
        lin.quantize_(dev(W))
        Wq, sw = O.quantize_weight_rows(W)
        mods.append(lin)
        refs.append(O.linear_int8_mixed(X, Wq, sw, 6.0)["Y"])
        xs.append(dev(X))
    for _ in range(2):
        for lin, X, ref in zip(mods, xs, refs):
            Y = host(lin(X))
            assert y_err(Y, ref) <= Y_TOL
    key = (torch.device("cuda").index or 0, torch.cuda.current_stream().cuda_stream)
    ws = L._WORKSPACES[key]
    need = max(gpu.ops.workspace_bytes(m, k, n) for k, n, m in shapes)
    assert ws.numel() >= need
    assert sum(1 for (dev_i, _) in L._WORKSPACES if dev_i == key[0]) >= 1

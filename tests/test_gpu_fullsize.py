"""Parity at the full workload sizes, through the same calls the benchmark times.

Every intermediate the oracle can afford is compared in full and bit-exactly
(outlier set, activation codes and scales, weight codes and scales). The int32
accumulators and the fp16 outputs are compared on sampled rows (and, for the
175B-scale layer, sampled output features): each sampled output is computed by
the oracle from the full outlier set, the sampled row's codes and the sampled
feature's weight row, which is all it depends on.
"""

import numpy as np
import pytest
import torch

from int8_quantized_matmul_absmax_amd import synth
from oracle import llm_int8 as O
from tests.gpu_helpers import Y_TOL, dev, f16_ulp, host, note, sample_rows, y_err

pytestmark = pytest.mark.gpu


def _weight_rows_oracle(W, rows, chunk=2048):
    """Oracle weight quantization of the listed output rows (row-independent)."""
    Wq = np.empty((rows.size, W.shape[1]), np.int8)
    sw = np.empty(rows.size, np.float32)
    for s in range(0, rows.size, chunk):
        q, a = O.quantize_weight_rows(W[rows[s:s + chunk]])
        Wq[s:s + chunk], sw[s:s + chunk] = q, a
    return Wq, sw


def _full_layer_check(gpu, d, n_rows, n_feats=None, seed=0):
    ops = gpu.ops
    X, W = d["X"], d["W"]
    M, K = X.shape
    N = W.shape[0]
    note("%s: weight quantization" % d["name"])
    Wd = dev(W)
    Wq_g, sw_g = ops.int8_quantize_colwise_weight(Wd)
    del Wd
    feats = np.arange(N) if n_feats is None else np.sort(
        np.random.default_rng(seed + 1).choice(N, n_feats, replace=False))
    Wq_ref, sw_ref = _weight_rows_oracle(W, feats)
    idx = torch.from_numpy(feats).cuda()
    assert np.array_equal(host(Wq_g[idx]), Wq_ref)
    assert np.array_equal(host(sw_g[idx]).view(np.uint32), sw_ref.view(np.uint32))

    note("%s: layer call" % d["name"])
    Xd = dev(X)
    ws = torch.empty((ops.workspace_bytes(M, K),), dtype=torch.uint8, device="cuda")
    Y = ops.linear_int8_mixed(Xd, Wq_g, sw_g, None, 6.0, ws)
    torch.cuda.synchronize()
    v = ops.workspace_views(ws, M, K)

    cols = O.detect_outlier_columns(X, 6.0)
    n = cols.size
    assert int(host(v["n"])[0]) == n
    assert np.array_equal(host(v["cols"])[:n], cols)
    assert set(d["planted"].tolist()) <= set(cols.tolist())
    Xq_ref, sx_ref = O.quantize_activation_rows(X, cols)
    assert np.array_equal(host(v["Xq"]), Xq_ref)
    assert np.array_equal(host(v["sx"]).view(np.uint32), sx_ref.view(np.uint32))
    ld = ops.outlier_ld(n)
    Xo = host(v["Xo"][: M * ld]).reshape(M, ld)
    assert np.array_equal(Xo[:, :n].view(np.uint16), X[:, cols].view(np.uint16))

    rows = sample_rows(M, n_rows, seed, must=[int(np.argmax(np.abs(X[:, cols[0]])))] if n else ())
    ridx = torch.from_numpy(rows).cuda()

    note("%s: int32 accumulators on %d rows" % (d["name"], rows.size))
    C = ops.int8_mm_dequant(v["Xq"], Wq_g, v["sx"], sw_g, want_y=False, want_int32=True)
    C_s = host(C[ridx][:, idx])
    del C
    assert np.array_equal(C_s, O.int32_accumulators(Xq_ref[rows], Wq_ref))

    note("%s: outputs on %d rows x %d features" % (d["name"], rows.size, feats.size))
    ref = O.linear_int8_mixed(X, Wq_ref, sw_ref, 6.0, rows=rows)
    err = y_err(host(Y[ridx][:, idx]), ref["Y"])
    assert err <= Y_TOL, err
    return err


def test_opt_ffn_up_full(gpu):
    """OPT-6.7B FFN up-projection at prefill: 2048 x 4096 -> 16384, 6 outlier dims."""
    d = synth.opt_ffn_up()
    _full_layer_check(gpu, d, n_rows=96)


def test_ffn_175b_full(gpu):
    """175B-scale FFN layer: 4096 x 12288 -> 49152, 12 outlier dims (~0.1%)."""
    d = synth.ffn_175b()
    _full_layer_check(gpu, d, n_rows=48, n_feats=4096, seed=4)


@pytest.mark.parametrize("n_in", [0, 6, 32, 128, 512])
def test_mlp_sweep_per_layer(gpu, n_in):
    """Two-layer MLP block 4096 -> 16384 -> GELU -> 4096 with n_in planted input
    outlier columns. Layer 1 is checked in full; layer 2 is checked on the
    oracle's own GELU output (the same fp16 input on both sides), whose
    outlier set is emergent and grows with n_in up to all 16384 columns."""
    ops = gpu.ops
    d = synth.mlp_sweep(n_in)
    X, W1, W2 = d["X"], d["W1"], d["W2"]
    M = X.shape[0]

    note("mlp n_in=%d layer 1" % n_in)
    Wq1, sw1 = ops.int8_quantize_colwise_weight(dev(W1))
    Wq1_ref, sw1_ref = O.quantize_weight_rows(W1)
    assert np.array_equal(host(Wq1), Wq1_ref)
    ref1 = O.linear_int8_mixed(X, Wq1_ref, sw1_ref, 6.0)
    assert ref1["n"] >= n_in
    K1, N1 = X.shape[1], Wq1.shape[0]
    ws1 = torch.empty((ops.workspace_bytes(M, K1, N1),), dtype=torch.uint8, device="cuda")
    Y1 = ops.linear_int8_mixed(dev(X), Wq1, sw1, None, 6.0, ws1)
    torch.cuda.synchronize()
    assert y_err(host(Y1), ref1["Y"]) <= Y_TOL
    v1 = ops.workspace_views(ws1, M, K1)
    assert np.array_equal(host(v1["Xq"]), ref1["Xq"])
    rows1 = sample_rows(M, 64, 100 + n_in)
    note("mlp n_in=%d layer 1 int32 accumulators on %d rows" % (n_in, rows1.size))
    C1 = ops.int8_mm_dequant(v1["Xq"], Wq1, v1["sx"], sw1, want_y=False, want_int32=True)
    C1_s = host(C1[torch.from_numpy(rows1).cuda()])
    del C1
    assert np.array_equal(C1_s, O.int32_accumulators(ref1["Xq"][rows1], Wq1_ref))

    # GELU between the layers: the oracle's chain (fp16 layer-1 output, exact
    # GELU, fp16) defines layer 2's input.
    G_ref = O.gelu_erf(ref1["Y"].astype(np.float16).astype(np.float64)).astype(np.float16)
    G_gpu = host(ops.gelu_f16(dev(ref1["Y"].astype(np.float16))))
    ulp = f16_ulp(G_ref)
    assert np.all(np.abs(G_gpu.astype(np.float64) - G_ref.astype(np.float64)) <= ulp + 1e-12)

    note("mlp n_in=%d layer 2" % n_in)
    Wq2, sw2 = ops.int8_quantize_colwise_weight(dev(W2))
    Wq2_ref, sw2_ref = O.quantize_weight_rows(W2)
    assert np.array_equal(host(Wq2), Wq2_ref)
    K2 = G_ref.shape[1]
    N2 = Wq2.shape[0]
    ws = torch.empty((ops.workspace_bytes(M, K2, N2),), dtype=torch.uint8, device="cuda")
    Y2 = ops.linear_int8_mixed(dev(G_ref), Wq2, sw2, None, 6.0, ws)
    torch.cuda.synchronize()
    v = ops.workspace_views(ws, M, K2)
    cols2 = O.detect_outlier_columns(G_ref, 6.0)
    assert int(host(v["n"])[0]) == cols2.size
    assert np.array_equal(host(v["cols"])[: cols2.size], cols2)
    rows = sample_rows(M, 128, n_in)
    ref2 = O.linear_int8_mixed(G_ref, Wq2_ref, sw2_ref, 6.0, rows=rows)
    assert np.array_equal(host(v["Xq"])[rows], ref2["Xq"])
    # the gathered outlier activations and their zero pad on the same rows
    n2 = cols2.size
    ld2 = (n2 + 31) // 32 * 32
    Xo2 = host(v["Xo"])[: M * ld2].reshape(M, ld2)[rows].view(np.uint16)
    assert np.array_equal(Xo2[:, :n2], G_ref[rows][:, cols2].view(np.uint16))
    assert not Xo2[:, n2:].any()
    note("mlp n_in=%d layer 2 int32 accumulators on %d rows" % (n_in, rows.size))
    C2 = ops.int8_mm_dequant(v["Xq"], Wq2, v["sx"], sw2, want_y=False, want_int32=True)
    C2_s = host(C2[torch.from_numpy(rows).cuda()])
    del C2
    assert np.array_equal(C2_s, O.int32_accumulators(ref2["Xq"], Wq2_ref))
    err2 = y_err(host(Y2)[rows], ref2["Y"])
    assert err2 <= Y_TOL, err2
    print("n_in=%d: layer-1 outliers %d, layer-2 outliers %d" % (n_in, ref1["n"], cols2.size))

"""Seeded random shapes through the whole layer, against the oracle.

Each case draws the token count M (from 1 to 600, including the edges of
the few-token paths), K (a multiple of 16 up to 2096), N (1 to 699), a
number of planted outlier columns (0 to 59, on a random token fraction), the
threshold (6, or now and then 0 or +inf), an optional bias and the
workspace size (with or without the many-outlier region). Together they
reach the detection's row bands, the row pass's flag modes, the
single-launch few-token layer, the few-token GEMV, the tiled GEMM, both Wo
builders and the GEMM's pick-up of outlier weight codes, at ragged sizes.
Two more cases use the large GEMM tiles (2100 x 8200 outputs).

Against the oracle: the intermediates bit for bit and Y within the
tolerance, with either workspace. With at most 16 outlier columns, or on
the few-token paths (which do not use the region), the two workspaces give
the same Y bits; with more columns the tiled GEMM runs the outlier product
over the recovered weights with the region and as its dense loop over all
columns without it (different fp32 sums), each checked against the oracle.
"""

import numpy as np
import pytest
import torch

from int8_quantized_matmul_absmax_amd import synth
from oracle import llm_int8 as O
from tests.gpu_helpers import Y_TOL, dev, host, note, y_err
from tests.test_gpu_parity import _check_intermediates

pytestmark = pytest.mark.gpu

SMALL_CASES = 24
LARGE_CASES = 2


def _draw(seed):
    rng = np.random.default_rng(7000 + seed)
    if seed < SMALL_CASES:
        M = int(rng.choice([1, 2, 3, 5, 8, 9, 16, 40, 64, 65, 130, 257, 300, 600]))
        K = int(16 * rng.integers(1, 132))
        N = int(rng.integers(1, 700))
    else:
        M, N = 2100, 8200
        K = int(16 * rng.integers(1, 34))
    u = rng.random()
    tau = 0.0 if u < 0.08 else (float("inf") if u < 0.16 else 6.0)
    with_bias, big_ws = bool(rng.random() < 0.5), bool(rng.random() < 0.5)
    if seed >= SMALL_CASES:   # large tiles: threshold 6, each workspace size once
        tau, big_ws = 6.0, seed % 2 == 0
    return rng, M, K, N, tau, with_bias, big_ws


@pytest.mark.parametrize("seed", range(SMALL_CASES + LARGE_CASES))
def test_random_shape(gpu, seed):
    rng, M, K, N, tau, with_bias, big_ws = _draw(seed)
    note("random shape seed=%d M=%d K=%d N=%d tau=%s bias=%s big_ws=%s"
         % (seed, M, K, N, tau, with_bias, big_ws))
    X = synth.normal_f16(rng, (M, K), 1.0)
    n_plant = int(rng.integers(0, min(K, 60)))
    if n_plant:
        synth.plant_outlier_columns(rng, X, n_plant, 6.5, 40.0, (0.05, 1.0))
    W = synth.normal_f16(rng, (N, K), 0.05)
    bias = synth.normal_f16(rng, (N,), 0.5) if with_bias else None
    Wq, sw = O.quantize_weight_rows(W)
    ref = O.linear_int8_mixed(X, Wq, sw, tau, bias)

    ops = gpu.ops
    ws = torch.empty((ops.workspace_bytes(M, K, N if big_ws else None),), dtype=torch.uint8,
                     device="cuda")
    Xd, Wqd, swd = dev(X), dev(Wq), dev(sw)
    bd = None if bias is None else dev(bias)
    Y = ops.linear_int8_mixed(Xd, Wqd, swd, bd, tau, ws)
    torch.cuda.synchronize()
    _check_intermediates(gpu, ops.workspace_views(ws, M, K), X, ref)
    err = y_err(host(Y), ref["Y"])
    assert err <= Y_TOL, err
    if big_ws:
        ws_small = torch.empty((ops.workspace_bytes(M, K),), dtype=torch.uint8, device="cuda")
        Y2 = ops.linear_int8_mixed(Xd, Wqd, swd, bd, tau, ws_small)
        torch.cuda.synchronize()
        err2 = y_err(host(Y2), ref["Y"])
        assert err2 <= Y_TOL, err2
        if ref["n"] <= 16 or M <= 64:
            assert np.array_equal(host(Y).view(np.uint16), host(Y2).view(np.uint16))

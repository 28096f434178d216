"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print for a worked example (fixtures under tests/golden/ with their
citation), closed forms, invariants, special cases that reduce to a library
routine, and brute force on tiny inputs.
"""

import json
import os

import numpy as np
import pytest

from oracle import llm_int8 as O
from int8_quantized_matmul_absmax_amd import synth


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- printed examples

def test_worked_absmax_example(golden_dir):
    g = _load(golden_dir, "absmax_worked_example.json")
    codes, s, a = O.absmax_quantize_vector(np.array(g["input"], np.float64))
    assert codes.tolist() == g["codes"]
    assert float(a) == pytest.approx(g["absmax"], abs=1e-6)
    assert round(float(s), g["scale_printed_decimals"]) == g["scale_printed"]
    # the same codes from fp16 images of the decimals (the layer's input type)
    codes16, _, _ = O.absmax_quantize_vector(np.array(g["input"], np.float16))
    assert codes16.tolist() == g["codes"]


def test_scaled_round_example(golden_dir):
    g = _load(golden_dir, "scaled_round_example.json")
    # a vector with absmax 1.0 holding 0.3: scale 127, 0.3 -> 38.1 -> 38
    v = np.array([g["value"], g["absmax"], -g["absmax"]], np.float64)
    codes, s, a = O.absmax_quantize_vector(v)
    assert float(s) == 127.0
    assert int(codes[0]) == g["code"]
    assert round(float(g["value"]) * float(s), 1) == g["scaled_printed"]
    deq = O.absmax_dequantize(codes[0], a)
    assert round(float(deq), g["dequantized_printed_decimals"]) == g["dequantized_printed"]
    # the true error is 7.87e-4 (the page's 0.008 is not reproduced)
    assert abs(g["value"] - deq) == pytest.approx(0.3 - 38 / 127, rel=1e-9)


def _f16_in(lo, hi):
    """All fp16 values v with lo <= v <= hi (brute force over bit patterns)."""
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    pos = bits.view(np.float16).astype(np.float64)
    vals = np.concatenate([pos, -pos[1:]])
    sel = (vals >= lo) & (vals <= hi)
    return np.sort(vals[sel]).astype(np.float16)


def _scb_candidates(g):
    """fp16 absmax values consistent with the printed recovery.

    The printed recovered tensor equals CB[i, j] * S[j] / 127 within print
    rounding (the scale vector broadcast along the input axis of the square
    layer); S[j] is the absmax of output row j. Intersect the intervals over
    the visible rows and keep the fp16 values inside.
    """
    CB = np.array(g["codes_int8_printed"], np.float64)
    R = np.array(g["recovered_printed"], np.float64)
    h = g["print_half_width"]
    out = []
    for j in range(6):
        lo, hi = -np.inf, np.inf
        for i in range(6):
            a = (R[i, j] - h) * 127 / CB[i, j]
            b = (R[i, j] + h) * 127 / CB[i, j]
            lo, hi = max(lo, min(a, b)), min(hi, max(a, b))
        assert lo <= hi
        cands = _f16_in(lo, hi)
        assert cands.size >= 1
        out.append(cands)
    return out


def test_printed_weight_codes_follow_per_output_row_absmax(golden_dir):
    """The printed 64x64 weight before/after quantization (HF blog, 'Usage').

    Build a 64x64 fp16 weight holding the printed visible corners (nearest
    fp16 of each printed decimal) and, in a hidden column of each visible
    row, that row's absmax as pinned by the printed recovery. The oracle's
    weight quantization must reproduce the printed codes; a cell whose code
    the 4-decimal print cannot decide (checked by brute force over every fp16
    value that prints the same) may differ by one.
    """
    g = _load(golden_dir, "printed_weight_example.json")
    idx = g["visible_index"]
    Wp = np.array(g["weight_fp16_printed"], np.float64)
    CB = np.array(g["codes_int8_printed"], np.int64)
    h = g["print_half_width"]
    scb = _scb_candidates(g)

    W = np.zeros((64, 64), np.float16)
    for r in range(6):
        for c in range(6):
            W[idx[r], idx[c]] = np.float16(Wp[r, c])
        W[idx[r], 30] = scb[r][0]
    Wq, sw = O.quantize_weight_rows(W)
    for r in range(6):
        assert float(sw[idx[r]]) == float(scb[r][0])

    ambiguous = 0
    for r in range(6):
        for c in range(6):
            # every code the print allows for this cell under the per-row rule
            allowed = set()
            for w in _f16_in(Wp[r, c] - h, Wp[r, c] + h):
                for S in scb[r]:
                    row = np.zeros(64, np.float16)
                    row[0], row[1] = w, S
                    q, _ = O.quantize_weight_rows(row[None, :])
                    allowed.add(int(q[0, 0]))
            assert CB[r, c] in allowed, (r, c, allowed)
            got = int(Wq[idx[r], idx[c]])
            if len(allowed) == 1:
                assert got == CB[r, c], (r, c)
            else:
                ambiguous += 1
                assert abs(got - CB[r, c]) <= 1
    assert ambiguous <= 2

    # The pin discriminates: the transposed rule (absmax per input column)
    # fails many printed codes.
    Wq_t, _ = O.quantize_weight_rows(np.ascontiguousarray(W.T))
    wrong = sum(int(Wq_t[idx[c], idx[r]]) != CB[r, c] for r in range(6) for c in range(6))
    assert wrong >= 10


def test_printed_recovery_reading(golden_dir):
    """Reading of the recovery CB * SCB / 127 (HF blog, 'Usage').

    Per output row, the recovery stays within the absmax rounding bound
    absmax/254 of the printed fp16 weights (plus print rounding); the printed
    recovered values, which broadcast the scale along the other axis, do not.
    """
    g = _load(golden_dir, "printed_weight_example.json")
    Wp = np.array(g["weight_fp16_printed"], np.float64)
    CB = np.array(g["codes_int8_printed"], np.float64)
    R = np.array(g["recovered_printed"], np.float64)
    h = g["print_half_width"]
    S = np.array([float(c[0]) for c in _scb_candidates(g)])
    per_row = CB * S[:, None] / 127
    assert np.all(np.abs(per_row - Wp) <= S[:, None] / 254 + h + 1e-6)
    assert np.any(np.abs(R - Wp) > S[:, None] / 254 + 2 * h)
    # the oracle's recovery function gives the per-row values
    Wq = CB.astype(np.int8)
    Wo = O.recover_outlier_weights(Wq, S.astype(np.float32), np.arange(6))
    assert np.allclose(Wo.astype(np.float64), per_row, rtol=2 ** -10, atol=0)


# ---------------------------------------------------------------- invariants

def test_row_max_maps_to_127_and_back_exactly():
    rng = np.random.default_rng(7)
    W = synth.normal_f16(rng, (64, 96), 0.02)
    Wq, sw = O.quantize_weight_rows(W)
    Wf = W.astype(np.float32)
    for j in range(W.shape[0]):
        k = int(np.argmax(np.abs(Wf[j])))
        assert abs(int(Wq[j, k])) == 127
        assert np.sign(Wq[j, k]) == np.sign(Wf[j, k])
        # the dequantized row maximum is exact: fl(fl(127 * a) / 127) == a
        a = np.float32(sw[j])
        assert np.float32(np.float32(127 * a) / np.float32(127)) == a
    assert Wq.min() >= -127 and Wq.max() <= 127


def test_absmax_error_bound_symmetry_monotone():
    rng = np.random.default_rng(11)
    X = synth.normal_f16(rng, (32, 128), 1.0)
    Xq, sx = O.quantize_activation_rows(X, np.zeros(0, np.int32))
    Xf = X.astype(np.float64)
    err = np.abs(Xf - Xq.astype(np.float64) * sx[:, None].astype(np.float64) / 127)
    assert np.all(err <= sx[:, None] / 254 * (1 + 1e-6))
    Xn = (-X.astype(np.float32)).astype(np.float16)
    Xqn, sxn = O.quantize_activation_rows(Xn, np.zeros(0, np.int32))
    assert np.array_equal(Xqn, -Xq) and np.array_equal(sxn, sx)
    for i in range(X.shape[0]):
        order = np.argsort(Xf[i], kind="stable")
        assert np.all(np.diff(Xq[i][order].astype(np.int64)) >= 0)


def test_round_half_to_even_ties():
    # absmax 127/32 (exact in fp16, below 6) gives the exact scale 32
    a = np.float16(127 / 32)
    assert float(a) == 3.96875
    row = np.array([a, 0.078125, 0.109375, -0.078125, 0.046875], np.float16)
    Xq, sx = O.quantize_activation_rows(row[None, :], np.zeros(0, np.int32))
    assert float(O.absmax_scale(sx)[0]) == 32.0
    # 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, 1.5 -> 2
    assert Xq[0].tolist() == [127, 2, 4, -2, 2]
    # weight side: absmax 127 gives scale 1; 2.5 -> 2 and 0.5 -> 0
    w = np.array([[127.0, 2.5, 0.5, -3.5]], np.float16)
    Wq, sw = O.quantize_weight_rows(w)
    assert Wq[0].tolist() == [127, 2, 0, -4]


def test_zero_rows():
    X = np.zeros((3, 64), np.float16)
    X[1, 5] = 9.0          # row 1: its only nonzero is in an outlier column
    X[2, :] = 0.25
    X[2, 5] = -7.5
    cols = O.detect_outlier_columns(X, 6.0)
    assert cols.tolist() == [5]
    Xq, sx = O.quantize_activation_rows(X, cols)
    assert sx[0] == 0 and sx[1] == 0 and np.all(Xq[:2] == 0)
    assert sx[2] == np.float32(0.25) and np.all(Xq[2, np.arange(64) != 5] == 127)
    assert Xq[2, 5] == 0
    Wq, sw = O.quantize_weight_rows(np.zeros((2, 32), np.float16))
    assert np.all(Wq == 0) and np.all(sw == 0)


# ---------------------------------------------------------------- outlier detection

def _detect_brute(X, tau):
    M, K = X.shape
    out = []
    for k in range(K):
        for i in range(M):
            if abs(float(X[i, k])) >= tau:
                out.append(k)
                break
    return out


def test_outlier_detection_brute_force_and_edges():
    rng = np.random.default_rng(3)
    X = synth.normal_f16(rng, (9, 70), 2.5)
    X[4, 13] = 6.0            # exactly the threshold: flagged (>=)
    X[2, 14] = -6.0
    X[0, 15] = np.float16(5.99609375)   # largest fp16 below 6: not flagged by itself
    for tau in (6.0, 3.0, 0.5):
        assert O.detect_outlier_columns(X, tau).tolist() == _detect_brute(X, tau)
    got = O.detect_outlier_columns(X, 6.0).tolist()
    assert 13 in got and 14 in got
    assert O.detect_outlier_columns(X, np.inf).tolist() == []
    assert O.detect_outlier_columns(X, 0.0).tolist() == list(range(70))
    assert O.detect_outlier_columns(np.zeros((0, 70), np.float16), 6.0).tolist() == []
    with pytest.raises(ValueError):
        O.detect_outlier_columns(X, float("nan"))


def test_nan_and_inf_columns_are_outlier_columns():
    X = np.full((3, 48), 0.5, np.float16)
    X[1, 7] = np.float16(np.nan)
    X[2, 20] = np.float16(-np.inf)
    X[0, 30] = 6.0
    assert O.detect_outlier_columns(X, 6.0).tolist() == [7, 20, 30]
    assert O.detect_outlier_columns(X, np.inf).tolist() == [7, 20]
    Xq, sx = O.quantize_activation_rows(X, O.detect_outlier_columns(X, 6.0))
    assert np.all(np.isfinite(sx)) and np.all(sx == np.float32(0.5))


def test_planted_columns_are_found_and_scales_below_threshold():
    d = synth.tiny()
    cols = O.detect_outlier_columns(d["X"], 6.0)
    assert set(d["planted"].tolist()) <= set(cols.tolist())
    Xf = np.abs(d["X"].astype(np.float32))
    for k in cols:
        assert Xf[:, k].max() >= 6.0
    Xq, sx = O.quantize_activation_rows(d["X"], cols)
    assert np.all(sx < 6.0)
    assert np.all(Xq[:, cols] == 0)
    bm = O.outlier_bitmap(cols, d["X"].shape[1])
    back = [k for k in range(d["X"].shape[1]) if (int(bm[k // 32]) >> (k % 32)) & 1]
    assert back == cols.tolist()


# ---------------------------------------------------------------- int32 accumulators

def test_int32_accumulators_brute_force_tiny():
    rng = np.random.default_rng(5)
    Xq = synth.random_codes(1, (4, 8))
    Wq = synth.random_codes(2, (8, 8))
    C = O.int32_accumulators(Xq, Wq)
    for i in range(4):
        for j in range(8):
            s = 0
            for k in range(8):
                s += int(Xq[i, k]) * int(Wq[j, k])
            assert int(C[i, j]) == s
    # extreme codes: every product 127*127 (the int32 bound with margin)
    K = 2048
    C = O.int32_accumulators(np.full((2, K), 127, np.int8), np.full((3, K), -127, np.int8))
    assert np.all(C == -K * 127 * 127)
    assert C.dtype == np.int32


def test_int32_accumulators_vs_int64_einsum():
    Xq = synth.random_codes(3, (16, 256))
    Wq = synth.random_codes(4, (256, 256))
    C = O.int32_accumulators(Xq, Wq)
    ref = np.einsum("ik,jk->ij", Xq.astype(np.int64), Wq.astype(np.int64))
    assert np.array_equal(C.astype(np.int64), ref)


# ---------------------------------------------------------------- end to end

def test_exactly_representable_construction():
    """X = qx / 32 with row absmax 127/32, W = qw / 64 with row absmax 127/64.

    Every value is exact in fp16 and below the threshold, the scales are the
    exact powers of two 32 and 64, so Xq = qx, Wq = qw, and the method's
    output equals X . W^T exactly: this pins the 1/127^2 dequantization and
    the storage of the absmax scales end to end.
    """
    rng = np.random.default_rng(9)
    M, K, N = 8, 64, 24
    qx = rng.integers(-127, 128, size=(M, K))
    qw = rng.integers(-127, 128, size=(N, K))
    qx[:, 0] = 127
    qw[:, 1] = -127
    X = (qx / 32.0).astype(np.float16)
    W = (qw / 64.0).astype(np.float16)
    assert np.array_equal(X.astype(np.float64) * 32, qx)
    Wq, sw = O.quantize_weight_rows(W)
    assert np.array_equal(Wq.astype(np.int64), qw)
    r = O.linear_int8_mixed(X, Wq, sw, 6.0)
    assert r["n"] == 0
    assert np.array_equal(r["Xq"].astype(np.int64), qx)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.array_equal(r["Y"], exact)


def test_threshold_infinity_is_pure_vector_wise_int8():
    """tau = +inf: no outlier columns; Y is the sum over k of the dequantized
    products (q_x a_x / 127) (q_w a_w / 127), written here as a brute-force
    loop."""
    d = synth.tiny(M=4, K=32, N=6)
    Wq, sw = O.quantize_weight_rows(d["W"])
    r = O.linear_int8_mixed(d["X"], Wq, sw, np.inf)
    assert r["n"] == 0
    Xq, sx = r["Xq"], r["sx"]
    for i in range(4):
        for j in range(6):
            s = 0.0
            for k in range(32):
                s += (int(Xq[i, k]) * float(sx[i]) / 127) * (int(Wq[j, k]) * float(sw[j]) / 127)
            assert r["Y"][i, j] == pytest.approx(s, rel=1e-12, abs=1e-12)


def test_threshold_zero_is_fp16_matmul_of_recovered_weights():
    """tau = 0: every column is an outlier, every int8 code is 0, and the
    layer is the plain matmul of X with the fp16 weights recovered per output
    row; compared with numpy's float64 matmul."""
    d = synth.tiny(M=5, K=48, N=7)
    Wq, sw = O.quantize_weight_rows(d["W"])
    r = O.linear_int8_mixed(d["X"], Wq, sw, 0.0)
    assert r["n"] == 48 and np.all(r["Xq"] == 0) and np.all(r["C"] == 0)
    assert np.all(r["sx"] == 0)
    Wrec = (Wq.astype(np.float64) * sw.astype(np.float64)[:, None] / 127).astype(np.float16)
    ref = d["X"].astype(np.float64) @ Wrec.astype(np.float64).T
    assert np.allclose(r["Y"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", [(4, 8, 8), (16, 256, 256)])
def test_error_bound_vs_unquantized(shape):
    """Brute force in fp64: the method's output stays within the absmax
    rounding bound of the unquantized X . W^T, elementwise."""
    M, K, N = shape
    d = synth.tiny(M=M, K=K, N=N)
    X, W = d["X"], d["W"]
    if K == 8:
        X[:, 3] = np.float16(12.5)
    Wq, sw = O.quantize_weight_rows(W)
    r = O.linear_int8_mixed(X, Wq, sw, 6.0)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    Xa = np.abs(X.astype(np.float64))
    What = Wq.astype(np.float64) * sw.astype(np.float64)[:, None] / 127
    mask = np.zeros(K, bool)
    mask[r["cols"]] = True
    bound = np.zeros((M, N))
    for i in range(M):
        for j in range(N):
            b = 0.0
            for k in range(K):
                if mask[k]:
                    b += Xa[i, k] * (float(sw[j]) / 254 + 2.0 ** -11 * abs(What[j, k]))
                else:
                    b += Xa[i, k] * float(sw[j]) / 254 + abs(What[j, k]) * float(r["sx"][i]) / 254
            bound[i, j] = b * (1 + 1e-5) + 1e-12
    assert np.all(np.abs(r["Y"] - exact) <= bound)
    # and the decomposition matters: the planted columns are found
    assert set(d["planted"].tolist()) <= set(r["cols"].tolist()) or K == 8


# ------------------------------------------- weight kept in fp16 (f16 mode)

def test_fp16_weights_threshold_zero_is_fp16_matmul_of_original_weights():
    """tau = 0 with the weight kept in fp16: every column is an outlier and
    the layer is the plain matmul of X with the original fp16 W (numpy's
    float64 matmul). The recovered-weight mode differs from it by the weight
    rounding error, so this separates the two weight sources."""
    d = synth.tiny(M=5, K=48, N=7)
    r = O.linear_int8_mixed_fp16_weights(d["X"], d["W"], 0.0)
    assert r["n"] == 48 and np.all(r["C"] == 0)
    ref = d["X"].astype(np.float64) @ d["W"].astype(np.float64).T
    assert np.allclose(r["Y"], ref, rtol=1e-12, atol=1e-12)
    Wq, sw = O.quantize_weight_rows(d["W"])
    rec = O.linear_int8_mixed(d["X"], Wq, sw, 0.0)
    assert np.max(np.abs(rec["Y"] - ref)) > 1e-6


def test_fp16_weights_threshold_infinity_equals_int8_weights_mode():
    """tau = +inf: no outlier columns, so the weight source of the outlier
    part never matters and both modes give the same result exactly."""
    d = synth.tiny(M=6, K=64, N=9)
    Wq, sw = O.quantize_weight_rows(d["W"])
    a = O.linear_int8_mixed_fp16_weights(d["X"], d["W"], np.inf)
    b = O.linear_int8_mixed(d["X"], Wq, sw, np.inf)
    assert a["n"] == 0
    assert np.array_equal(a["Y"], b["Y"])


def test_fp16_weights_exact_construction_agrees_with_recovery():
    """W = qw / 64 with every row absmax 127/64: the recovery
    fp16(q * sw / 127) reproduces W exactly, so with outlier columns present
    the two modes must agree bit for bit (and the outlier columns taken from
    W equal the recovered ones)."""
    rng = np.random.default_rng(11)
    M, K, N = 6, 64, 10
    qw = rng.integers(-127, 128, size=(N, K))
    qw[:, 2] = 127
    W = (qw / 64.0).astype(np.float16)
    X = (rng.standard_normal((M, K)) * 0.5).astype(np.float16)
    X[1, 5] = np.float16(9.0)
    X[3, 40] = np.float16(-7.25)
    a = O.linear_int8_mixed_fp16_weights(X, W, 6.0)
    Wq, sw = O.quantize_weight_rows(W)
    b = O.linear_int8_mixed(X, Wq, sw, 6.0)
    assert a["cols"].tolist() == [5, 40]
    assert np.array_equal(a["Wo"], b["Wo"])
    assert np.array_equal(a["Y"], b["Y"])


@pytest.mark.parametrize("shape", [(4, 8, 8), (16, 256, 256)])
def test_fp16_weights_error_bound_vs_unquantized(shape):
    """With the original fp16 weight columns the outlier part carries no
    weight rounding: the error against X . W^T is bounded by the absmax terms
    of the normal columns alone (brute force in fp64)."""
    M, K, N = shape
    d = synth.tiny(M=M, K=K, N=N)
    X, W = d["X"], d["W"]
    if K == 8:
        X[:, 3] = np.float16(12.5)
    r = O.linear_int8_mixed_fp16_weights(X, W, 6.0)
    assert r["n"] > 0
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    Xa = np.abs(X.astype(np.float64))
    What = r["Wq"].astype(np.float64) * r["sw"].astype(np.float64)[:, None] / 127
    normal = np.ones(K, bool)
    normal[r["cols"]] = False
    for i in range(M):
        for j in range(N):
            b = 0.0
            for k in np.nonzero(normal)[0]:
                b += Xa[i, k] * float(r["sw"][j]) / 254 + abs(What[j, k]) * float(r["sx"][i]) / 254
            assert abs(r["Y"][i, j] - exact[i, j]) <= b * (1 + 1e-5) + 1e-12


def test_fp16_weights_given_codes_match_per_call_quantization():
    d = synth.tiny(M=7, K=96, N=12)
    a = O.linear_int8_mixed_fp16_weights(d["X"], d["W"], 6.0)
    Wq, sw = O.quantize_weight_rows(d["W"])
    b = O.linear_int8_mixed_fp16_weights(d["X"], d["W"], 6.0, Wq=Wq, sw=sw)
    assert np.array_equal(a["Wq"], Wq) and np.array_equal(a["sw"], sw)
    assert np.array_equal(a["Y"], b["Y"])


def test_rows_subset_matches_full():
    d = synth.tiny()
    Wq, sw = O.quantize_weight_rows(d["W"])
    full = O.linear_int8_mixed(d["X"], Wq, sw)
    rows = np.array([0, 5, 15])
    part = O.linear_int8_mixed(d["X"], Wq, sw, rows=rows)
    assert np.array_equal(part["cols"], full["cols"])
    assert np.array_equal(part["Xq"], full["Xq"][rows])
    assert np.array_equal(part["C"], full["C"][rows])
    assert np.array_equal(part["Y"], full["Y"][rows])


def test_bias_is_added():
    d = synth.tiny(M=3, K=32, N=5)
    Wq, sw = O.quantize_weight_rows(d["W"])
    b = np.array([1.0, -2.0, 0.5, 0.0, 3.25], np.float16)
    r0 = O.linear_int8_mixed(d["X"], Wq, sw)
    r1 = O.linear_int8_mixed(d["X"], Wq, sw, bias=b)
    assert np.allclose(r1["Y"] - r0["Y"], b.astype(np.float64)[None, :], rtol=0, atol=1e-12)


def test_gelu_closed_forms():
    """GELU(x) = x * Phi(x) with Phi the standard normal CDF: textbook table
    values of Phi, the odd-part identity GELU(x) - GELU(-x) = x, and the tails."""
    # Phi(1) and Phi(1.96) from standard normal tables (16 digits).
    assert abs(O.gelu_erf(1.0) - 0.8413447460685429) < 1e-14
    assert abs(O.gelu_erf(1.96) - 1.96 * 0.9750021048517795) < 1e-14
    assert O.gelu_erf(0.0) == 0.0
    x = np.linspace(-9, 9, 181)
    assert np.allclose(O.gelu_erf(x) - O.gelu_erf(-x), x, rtol=0, atol=1e-13)
    assert abs(O.gelu_erf(12.0) - 12.0) < 1e-12 and abs(O.gelu_erf(-12.0)) < 1e-12


def test_max_abs_rel_error_definition():
    ref = np.array([[1.0, -4.0], [2.0, 0.0]])
    test = ref + np.array([[0.0, 0.02], [-0.04, 0.01]])
    assert abs(O.max_abs_rel_error(test, ref) - 0.01) < 1e-15
    assert O.max_abs_rel_error(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0

"""The oracle pins have power: plausible mistakes planted in the oracle (on the
CPU, in this process only) make at least one pin fail."""

import numpy as np
import pytest

from oracle import llm_int8 as O
from tests import test_oracle_pins as P

# the unpatched functions, for mutants built from other oracle steps
O_ORIG_QUANTIZE = O.quantize_weight_rows
O_ORIG_RECOVER = O.recover_outlier_weights


def _half_away_codes(x_f32, scale_f32):
    prod = np.multiply(np.asarray(x_f32, np.float32), np.asarray(scale_f32, np.float32),
                       dtype=np.float32)
    q = np.sign(prod) * np.floor(np.abs(prod) + np.float32(0.5))
    return np.clip(q, -127, 127).astype(np.int8)


def _strict_detect(X16, threshold=6.0):
    X = np.asarray(X16).astype(np.float32)
    if X.shape[0] == 0:
        return np.zeros(0, np.int32)
    return np.nonzero(np.any(np.abs(X) > np.float32(threshold), axis=0))[0].astype(np.int32)


def _per_column_weight(W16):
    W = np.asarray(W16).astype(np.float32)
    sw = np.max(np.abs(W), axis=0).astype(np.float32)
    s = O.absmax_scale(sw)
    return O.absmax_codes(W, s[None, :]), sw


def _dequant_one_127(C, sx, sw, Yo, bias=None):
    return (np.asarray(C, np.float64) * np.asarray(sx, np.float64)[:, None]
            * np.asarray(sw, np.float64)[None, :] / 127.0 + Yo)


def _absmax_includes_outliers(X16, cols, rows=None):
    X = np.asarray(X16)
    if rows is not None:
        X = X[np.asarray(rows)]
    Xf = X.astype(np.float32)
    sx = np.max(np.abs(Xf), axis=1).astype(np.float32)
    Xq = O.absmax_codes(Xf, O.absmax_scale(sx)[:, None])
    Xq[:, np.asarray(cols, np.int64)] = 0
    return Xq, sx


def _recover_per_column(Wq, sw, cols):
    cols = np.asarray(cols, np.int64)
    q = np.asarray(Wq)[:, cols].astype(np.float32)
    t = np.multiply(q, np.asarray(sw, np.float32)[cols][None, :], dtype=np.float32)
    return np.divide(t, np.float32(127), dtype=np.float32).astype(np.float16)


def _outlier_product_dropped(X16, cols, Wo, rows=None):
    X = np.asarray(X16)
    if rows is not None:
        X = X[np.asarray(rows)]
    return np.zeros((X.shape[0], np.asarray(Wo).shape[0]))


def _fp16_columns_recovered(W16, cols):
    Wq, sw = O_ORIG_QUANTIZE(W16)
    return O_ORIG_RECOVER(Wq, sw, cols)


def _scale_times_absmax(absmax):
    a = np.asarray(absmax, dtype=np.float32)
    s = np.zeros_like(a)
    nz = a != 0
    s[nz] = np.float32(1.0) / a[nz] * np.float32(126)
    return s


MUTANTS = {
    "round_half_away": ("absmax_codes", _half_away_codes),
    "strict_threshold": ("detect_outlier_columns", _strict_detect),
    "per_column_weight_scale": ("quantize_weight_rows", _per_column_weight),
    "dequant_by_127": ("dequantize_merge", _dequant_one_127),
    "absmax_over_outliers": ("quantize_activation_rows", _absmax_includes_outliers),
    "recovery_wrong_axis": ("recover_outlier_weights", _recover_per_column),
    "outlier_part_dropped": ("outlier_product", _outlier_product_dropped),
    "range_126": ("absmax_scale", _scale_times_absmax),
    "fp16_mode_uses_recovered_weights": ("fp16_weight_columns", _fp16_columns_recovered),
}

PINS = [
    (P.test_worked_absmax_example, ("golden",)),
    (P.test_scaled_round_example, ("golden",)),
    (P.test_printed_weight_codes_follow_per_output_row_absmax, ("golden",)),
    (P.test_printed_recovery_reading, ("golden",)),
    (P.test_row_max_maps_to_127_and_back_exactly, ()),
    (P.test_round_half_to_even_ties, ()),
    (P.test_zero_rows, ()),
    (P.test_outlier_detection_brute_force_and_edges, ()),
    (P.test_planted_columns_are_found_and_scales_below_threshold, ()),
    (P.test_exactly_representable_construction, ()),
    (P.test_threshold_zero_is_fp16_matmul_of_recovered_weights, ()),
    (P.test_fp16_weights_threshold_zero_is_fp16_matmul_of_original_weights, ()),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, monkeypatch, golden_dir):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin, args in PINS:
        try:
            pin(*[golden_dir for _ in args])
        except (AssertionError, ValueError, IndexError, TypeError):
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name

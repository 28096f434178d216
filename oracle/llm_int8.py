"""Plain CPU oracle for the LLM.int8() mixed-precision int8 linear layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check of the repository
entry point and the CPU-baseline leg of the benchmark may import this module.
The product path (the HIP library and its Python binding) never imports or
calls it, and this module imports nothing from the product path.

Pages cited (by title and section; the reader has the pages themselves):

  [HF-blog]  Hugging Face blog, "A Gentle Introduction to 8-bit Matrix
             Multiplication for transformers at scale using Hugging Face
             Transformers, Accelerate and bitsandbytes" (Chinese translation).
  [Summary]  Paper summary page "LLM.int8(): 8-Bit Matrix Multiplication for
             Transformers at Scale" (Dettmers, Lewis, Belkada, Zettlemoyer).

What the method computes for Y = X . W^T (X fp16 [M, K] tokens x hidden,
W fp16 [N, K] in nn.Linear layout, Y [M, N]):

  1. outlier columns: every hidden dimension k for which some token has
     abs(X[i, k]) >= threshold (6.0)           [HF-blog "Inside the MatMul"],
                                               [Summary "The full picture" step 1]
  2. split X and W along those columns          [Summary "The full picture" step 2]
  3a. outlier part: an fp16 matmul of the outlier columns of X against the
      matching fp16 weight columns             [HF-blog "Inside the MatMul"]
  3b. normal part: absmax-quantize each row of X and each output row of W
      (a column of B = W^T) to int8, int8 matmul with int32 accumulation,
      dequantize by the outer product of the two absmax vectors
                                               [HF-blog "Introduction to model
                                               quantization"], [Summary "First
                                               innovation", "The full picture" step 3]
  4. add the two parts                         [Summary "The full picture" step 4]

Readings taken where the pages are open:
  * threshold test is abs(x) >= tau ("6 or greater" in "Inside the MatMul");
    a column holding NaN also counts as an outlier column;
  * scale s = fl32(127 / absmax) once per vector, code = rne(fl32(x * s))
    (the worked example of "Introduction to model quantization" divides 127
    by the absmax and multiplies the vector by the result); ties round to
    even; codes are symmetric in [-127, 127];
  * an all-zero vector (absmax 0) gets scale 0 and all-zero codes;
  * the X row absmax runs over the non-outlier columns only (the normal part
    is what gets quantized); the W row absmax runs over the full row, once,
    when the weight is placed on the device ("Usage": quantization happens on
    .to(device));
  * the fp16 weight columns of the outlier matmul are recovered from the int8
    weight as fp16(CB * SCB / 127) with SCB broadcast per output row
    ("Usage": recovery of fp16 weights for the outlier matmul);
  * with the weight kept in fp16 (has_fp16_weights=True, "Usage") the
    outlier matmul takes the original fp16 columns instead, and the int8
    codes of W are those of this call's weight (quantized per call, or the
    caller's codes of the same weight);
  * the outlier set is the union over all rows of one call, listed ascending;
  * sums of the fp16 outlier product and the dequantized result are formed in
    fp64 here (the reference value); the kernel forms them in fp32 and rounds
    the output once to fp16.

fp16 values are numpy float16 arrays (IEEE binary16; numpy's conversion to
binary32 is exact and its conversion from binary32 rounds to nearest even).
The scale arithmetic is IEEE binary32, one operation at a time, as numpy does
it element-wise (no fused multiply-add, no extended precision).
"""

import numpy as np

# [HF-blog "Inside the MatMul"]: extracting all outliers of magnitude 6 or more
# recovered full inference quality; [HF-blog "accelerate is all you need"]:
# the module-replacement helper defaults to threshold=6.0.
DEFAULT_THRESHOLD = 6.0

# [HF-blog "Introduction to model quantization"]: the int8 target range of
# absmax quantization is [-127, 127].
QMAX = 127


def _as_f16(a):
    a = np.asarray(a)
    if a.dtype != np.float16:
        raise TypeError("fp16 input required, got %s" % a.dtype)
    return a


def absmax_scale(absmax):
    """Per-vector quantization constant 127 / absmax in binary32.

    [HF-blog "Introduction to model quantization"], worked example: the scale
    is 127 divided by the absolute maximum (127 / 5.4 ~ 23.5). A zero absmax
    (all-zero vector) has no such constant; its scale is 0 so that every code
    is 0 (reading: zero vector).
    """
    a = np.asarray(absmax, dtype=np.float32)
    s = np.zeros_like(a, dtype=np.float32)
    nz = a != 0
    s[nz] = np.float32(QMAX) / a[nz]          # one correctly rounded fp32 divide
    return s


def absmax_codes(x_f32, scale_f32):
    """int8 codes rne(fl32(x * s)) clamped to [-127, 127].

    [HF-blog "Introduction to model quantization"]: multiply the vector by the
    scale and round; [Summary "How quantization works"]: round to the nearest
    integer. Ties go to even (numpy rint).
    """
    prod = np.multiply(np.asarray(x_f32, np.float32), np.asarray(scale_f32, np.float32),
                       dtype=np.float32)
    q = np.rint(prod)
    q = np.clip(q, -QMAX, QMAX)
    return q.astype(np.int8)


def absmax_quantize_vector(v):
    """Absmax quantization of one vector: returns (codes int8, scale fp32, absmax fp32).

    [HF-blog "Introduction to model quantization"]: take the absolute maximum,
    scale = 127 / absmax, codes = round(v * scale). Input is converted to
    binary32 first (decimal literals or fp16 values both work).
    """
    v32 = np.asarray(v, dtype=np.float32)
    a = np.max(np.abs(v32)) if v32.size else np.float32(0)
    s = absmax_scale(np.array([a], np.float32))[0]
    return absmax_codes(v32, s), s, np.float32(a)


def absmax_dequantize(codes, absmax):
    """Inverse map q * absmax / 127 in fp64 (reference value, not a kernel)."""
    return np.asarray(codes, np.float64) * np.float64(absmax) / QMAX


def quantize_weight_rows(W16):
    """Step a4: per-output-row absmax quantization of W [N, K] fp16.

    [HF-blog "Introduction to model quantization"]: vector-wise quantization
    takes the absmax of every column of B in A*B; with Y = X . W^T, B = W^T so
    each column of B is an output row of W. [HF-blog "Inside the MatMul"]: the
    weight matrix is quantized column-wise (columns of B). [HF-blog "Usage"]:
    this happens once, when the weight is moved to the device, over the whole
    row. Returns (Wq int8 [N, K], sw fp32 [N]) with sw the row absmax (the SCB
    statistic) so that W ~ Wq * sw[:, None] / 127.
    """
    W = _as_f16(W16).astype(np.float32)
    sw = np.max(np.abs(W), axis=1) if W.shape[1] else np.zeros(W.shape[0], np.float32)
    sw = sw.astype(np.float32)
    s = absmax_scale(sw)
    Wq = absmax_codes(W, s[:, None])
    return Wq, sw


def detect_outlier_columns(X16, threshold=DEFAULT_THRESHOLD):
    """Step a1: ascending int32 list of columns k with some abs(X[i, k]) >= threshold.

    [HF-blog "A gentle summary of LLM.int8()" step 1]: outliers are extracted
    column-wise from the input hidden states; [HF-blog "Inside the MatMul"]:
    magnitude 6 or greater; [Summary "The full picture" step 1]: a feature
    dimension is an outlier when at least one value in it reaches the
    threshold in magnitude. The set is the union over all M rows of the call.
    The comparison is made on exact binary32 images of the fp16 values.
    Reading (the pages do not cover NaN): a column holding a NaN is an
    outlier column too, so NaN never enters the int8 path and propagates
    through the fp16 outlier product instead.
    """
    X = _as_f16(X16).astype(np.float32)
    tau = np.float32(threshold)
    if np.isnan(tau):
        raise ValueError("threshold is NaN")
    if X.shape[0] == 0:
        return np.zeros(0, np.int32)
    flagged = np.any((np.abs(X) >= tau) | np.isnan(X), axis=0)
    return np.nonzero(flagged)[0].astype(np.int32)


def outlier_bitmap(cols, K):
    """K-bit column flag map, bit (k % 32) of uint32 word k // 32."""
    words = np.zeros((K + 31) // 32, np.uint32)
    for k in np.asarray(cols, np.int64):
        words[k // 32] |= np.uint32(1) << np.uint32(k % 32)
    return words


def quantize_activation_rows(X16, cols, rows=None):
    """Step a3: row-wise absmax quantization of the normal part of X.

    [HF-blog "Inside the MatMul"]: the hidden states are quantized row-wise;
    [Summary "Second innovation"] and [Summary "The full picture" step 3]:
    only the normal (non-outlier) part goes through int8. So the absmax of row
    i runs over the columns not in `cols`, the codes of the outlier columns
    are 0, and sx[i] is that absmax. `rows` optionally restricts the rows
    evaluated (a subset of the outputs, same arithmetic).
    Returns (Xq int8 [R, K], sx fp32 [R]).
    """
    X = _as_f16(X16)
    if rows is not None:
        X = X[np.asarray(rows)]
    Xf = X.astype(np.float32)
    normal = np.ones(Xf.shape[1], bool)
    normal[np.asarray(cols, np.int64)] = False
    Xn = np.where(normal[None, :], Xf, np.float32(0))
    sx = (np.max(np.abs(Xn), axis=1) if Xf.shape[1] else
          np.zeros(Xf.shape[0], np.float32)).astype(np.float32)
    s = absmax_scale(sx)
    Xq = absmax_codes(Xn, s[:, None])
    Xq[:, ~normal] = 0
    return Xq, sx


def int32_accumulators(Xq, Wq):
    """Step a5: C[i, j] = sum_k Xq[i, k] * Wq[j, k] with int32 accumulation.

    [Summary "The full picture" step 3]: an Int8 matmul with an Int32 result.
    The sum is formed with a float64 matrix product: every product of two
    int8 codes and every partial sum is an integer below 2**53 in magnitude,
    so the float64 sum is the exact integer sum in any order. The result is
    checked against the int32 range (abs(C) <= K * 127**2).
    """
    Xq = np.asarray(Xq)
    Wq = np.asarray(Wq)
    K = Xq.shape[1]
    if K * QMAX * QMAX >= 2 ** 53:
        raise ValueError("K too large for exact float64 accumulation")
    C = np.asarray(Xq, np.float64) @ np.asarray(Wq, np.float64).T
    Ci = C.astype(np.int64)
    if Ci.size and np.max(np.abs(Ci)) > 2 ** 31 - 1:
        raise OverflowError("int32 accumulator overflow")
    return Ci.astype(np.int32)


def recover_outlier_weights(Wq, sw, cols):
    """fp16 weight columns for the outlier matmul, from the int8 weight.

    [HF-blog "Usage"]: in inference mode (has_fp16_weights=False) the fp16
    weights for the outlier matmul are recovered as CB * SCB / 127, where CB
    is the int8 weight and SCB the per-output-row absmax; the scale is applied
    per output row. Arithmetic: fp16(fl32(fl32(q * sw[j]) / 127)).
    Returns Wo fp16 [N, n].
    """
    cols = np.asarray(cols, np.int64)
    q = np.asarray(Wq)[:, cols].astype(np.float32)
    t = np.multiply(q, np.asarray(sw, np.float32)[:, None], dtype=np.float32)
    t = np.divide(t, np.float32(QMAX), dtype=np.float32)
    return t.astype(np.float16)


def outlier_product(X16, cols, Wo, rows=None):
    """Step a6: Yo = X[:, cols] . Wo^T with fp16 operands, summed in fp64.

    [HF-blog "Inside the MatMul"]: the outlier part is a classic fp16 matmul;
    [Summary "The full picture" step 3]: the outlier part is multiplied in
    full 16-bit precision. Each fp16 x fp16 product is exact in fp64.
    """
    X = _as_f16(X16)
    if rows is not None:
        X = X[np.asarray(rows)]
    Xo = X[:, np.asarray(cols, np.int64)].astype(np.float64)
    return Xo @ np.asarray(Wo, np.float16).astype(np.float64).T


def dequantize_merge(C, sx, sw, Yo, bias=None):
    """Step a7: Y = C * (sx[i] * sw[j]) / 127**2 + Yo (+ bias), in fp64.

    [HF-blog "Introduction to model quantization"]: denormalize by the outer
    product of the two absmax vectors; each absmax carries a factor 1/127 of
    its own scale, hence 1/127**2. [HF-blog "A gentle summary" step 3] and
    [Summary "The full picture" step 4]: add the outlier result; the layer
    output is fp16 (the kernel rounds once at the end; this value is kept in
    fp64 as the reference).
    """
    Y = (np.asarray(C, np.float64)
         * (np.asarray(sx, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :])
         / float(QMAX * QMAX))
    Y = Y + np.asarray(Yo, np.float64)
    if bias is not None:
        Y = Y + _as_f16(bias).astype(np.float64)[None, :]
    return Y


def linear_int8_mixed(X16, Wq, sw, threshold=DEFAULT_THRESHOLD, bias=None, rows=None):
    """Whole layer, steps a1-a3 and a5-a7, for a weight already quantized (a4).

    Returns a dict with the intermediates: cols, n, Xq, sx, C, Wo, Yo, Y.
    With `rows`, the outlier set is still taken over all rows of X (it is a
    property of the whole call), and the per-row results are evaluated only
    for the listed rows.
    """
    cols = detect_outlier_columns(X16, threshold)
    Xq, sx = quantize_activation_rows(X16, cols, rows)
    C = int32_accumulators(Xq, Wq)
    Wo = recover_outlier_weights(Wq, sw, cols)
    Yo = outlier_product(X16, cols, Wo, rows)
    Y = dequantize_merge(C, sx, sw, Yo, bias)
    return {"cols": cols, "n": int(cols.size), "Xq": Xq, "sx": sx, "C": C,
            "Wo": Wo, "Yo": Yo, "Y": Y}


def fp16_weight_columns(W16, cols):
    """fp16 weight columns for the outlier matmul, from the fp16 weight.

    [HF-blog "Usage"]: has_fp16_weights=True (the default, meant for mixed
    Int8/FP16 training) keeps the weight in fp16 inside the module, so the
    outlier matmul takes the weight columns matching the outlier columns of X
    as they are ([HF-blog "Inside the MatMul"]: the outlier part is an fp16
    matmul of those columns); no CB * SCB / 127 recovery is involved.
    Returns W[:, cols] fp16 [N, n].
    """
    return _as_f16(W16)[:, np.asarray(cols, np.int64)]


def linear_int8_mixed_fp16_weights(X16, W16, threshold=DEFAULT_THRESHOLD, bias=None,
                                   rows=None, Wq=None, sw=None):
    """Whole layer with the weight kept in fp16 (has_fp16_weights=True).

    Steps a1-a7 as in `linear_int8_mixed`, with two differences that follow
    from the module holding W in fp16 ([HF-blog "Usage"]): the int8 normal
    part uses W quantized per output row at this call (step a4; a caller that
    still holds the codes of the same W may pass them as Wq, sw), and the
    outlier part multiplies the original fp16 weight columns.
    Returns the same dict as `linear_int8_mixed`, plus Wq and sw.
    """
    if Wq is None or sw is None:
        Wq, sw = quantize_weight_rows(W16)
    cols = detect_outlier_columns(X16, threshold)
    Xq, sx = quantize_activation_rows(X16, cols, rows)
    C = int32_accumulators(Xq, Wq)
    Wo = fp16_weight_columns(W16, cols)
    Yo = outlier_product(X16, cols, Wo, rows)
    Y = dequantize_merge(C, sx, sw, Yo, bias)
    return {"cols": cols, "n": int(cols.size), "Xq": Xq, "sx": sx, "C": C,
            "Wo": Wo, "Yo": Yo, "Y": Y, "Wq": Wq, "sw": sw}


def gelu_erf(x64):
    """Exact-erf GELU, x * (1 + erf(x / sqrt 2)) / 2, in fp64.

    Not part of the method; it is the activation between the two linear
    layers of the two-layer MLP workload.
    """
    from scipy.special import erf
    x = np.asarray(x64, np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def max_abs_rel_error(Y_test, Y_ref):
    """max |Y_test - Y_ref| / max |Y_ref| (the parity metric for fp outputs)."""
    Yt = np.asarray(Y_test, np.float64)
    Yr = np.asarray(Y_ref, np.float64)
    if Yr.size == 0:
        return 0.0
    den = np.max(np.abs(Yr))
    num = np.max(np.abs(Yt - Yr))
    if den == 0:
        return float(num)
    return float(num / den)

"""Plain CPU baselines for the accuracy ablations of LLM.int8().

TEST AND MEASUREMENT INFRASTRUCTURE ONLY, like the rest of this package: only
the tests and the benchmark's ablation report use it; the product path never
does. These are the quantization schemes the pages compare LLM.int8() with,
not steps of the method; the GPU path implements the method (and, with an
infinite threshold, vector-wise quantization without the decomposition).

Pages cited (by title and section):
  [HF-blog]  Hugging Face blog, "A Gentle Introduction to 8-bit Matrix
             Multiplication for transformers at scale using Hugging Face
             Transformers, Accelerate and bitsandbytes" (Chinese translation).
  [Summary]  Paper summary page "LLM.int8(): 8-Bit Matrix Multiplication for
             Transformers at Scale".

Schemes, for Y = X . W^T with X fp16 [M, K] and W fp16 [N, K]:
  tensor-wise absmax  one absmax scale for all of X and one for all of W
                      ([HF-blog] "Introduction to model quantization": divide
                      by the tensor's absolute maximum, times 127; [Summary]
                      "First innovation": one scale for the whole tensor, which
                      one outlier spoils);
  zero-point          asymmetric codes over the full int8 range [-128, 127] per
                      tensor, with 0 exactly representable ([HF-blog] same
                      section: subtract the minimum and scale by the range,
                      keeping the value 0 on an integer; [Summary] "How
                      quantization works": shifts the distribution so that
                      asymmetric ranges use the whole range);
  vector-wise         per-row absmax of X and per-output-row absmax of W with
                      no outlier decomposition: `llm_int8.linear_int8_mixed`
                      with threshold +inf ([Summary] "First innovation").

Readings where the pages give no formula: zero-point uses the binary32 scale
nd = fl32(255 / (max - min)), zero point zp = rne(-min * nd) - 128 (so min
maps to -128 and 0 to the integer zp), codes q = clamp(rne(fl32(x * nd)) +
zp, -128, 127), dequantized as (q - zp) / nd; a constant tensor (max == min)
gets nd = 0 and codes zp = -128 ... the same arithmetic as absmax's zero
vector: every code equal, dequantizing to 0. Products are summed exactly
(integer codes, fp64 sums); the outputs are fp64.
"""

import numpy as np

from . import llm_int8 as O


def tensorwise_absmax(A16):
    """Codes and absmax of one absmax scale over the whole tensor."""
    A = np.asarray(A16, np.float16).astype(np.float32)
    a = np.float32(np.max(np.abs(A))) if A.size else np.float32(0)
    s = O.absmax_scale(np.array([a], np.float32))[0]
    return O.absmax_codes(A, s), a


def tensorwise_absmax_linear(X16, W16):
    """Y = (Xq . Wq^T) * aX * aW / 127^2 with one scale per tensor."""
    Xq, ax = tensorwise_absmax(X16)
    Wq, aw = tensorwise_absmax(W16)
    C = np.asarray(Xq, np.float64) @ np.asarray(Wq, np.float64).T
    return C * (float(ax) * float(aw)) / float(O.QMAX * O.QMAX)


def zeropoint_quantize(A16):
    """Asymmetric int8 codes of a tensor: (codes int16 in [-128, 127], nd, zp)."""
    A = np.asarray(A16, np.float16).astype(np.float32)
    lo = np.float32(np.min(A)) if A.size else np.float32(0)
    hi = np.float32(np.max(A)) if A.size else np.float32(0)
    span = np.float32(hi - lo)
    nd = np.divide(np.float32(255), span, dtype=np.float32) if span > 0 else np.float32(0)
    zp = int(np.rint(-np.float64(np.float32(lo * nd)))) - 128
    y = np.multiply(A, nd, dtype=np.float32)
    q = np.clip(np.rint(y).astype(np.int64) + zp, -128, 127)
    return q.astype(np.int16), nd, zp


def zeropoint_dequantize(q, nd, zp):
    if nd == 0:
        return np.zeros(np.shape(q), np.float64)
    return (np.asarray(q, np.float64) - zp) / float(nd)


def zeropoint_linear(X16, W16):
    """Y = sum_k (qx - zx)(qw - zw) / (ndX * ndW), the products exact."""
    qx, ndx, zx = zeropoint_quantize(X16)
    qw, ndw, zw = zeropoint_quantize(W16)
    if ndx == 0 or ndw == 0:
        return np.zeros((np.shape(X16)[0], np.shape(W16)[0]))
    C = (qx.astype(np.float64) - zx) @ (qw.astype(np.float64) - zw).T
    return C / (float(ndx) * float(ndw))


def vectorwise_linear(X16, Wq, sw):
    """Vector-wise int8 without the decomposition (threshold +inf)."""
    return O.linear_int8_mixed(X16, Wq, sw, np.inf)["Y"]


def relative_errors(Y, Y_exact):
    """(max |Y - Y_exact| / max |Y_exact|, mean |Y - Y_exact| / mean |Y_exact|)."""
    d = np.abs(np.asarray(Y, np.float64) - Y_exact)
    return float(d.max() / np.abs(Y_exact).max()), float(d.mean() / np.abs(Y_exact).mean())

"""Torch-tensor wrappers of the C ABI, one per entry point, with the same names.

Argument marshalling only: every step of the layer runs in the HIP kernels of
libi8mm.so. torch provides device memory and the current stream. Inputs must
be contiguous tensors on one gfx950 GPU; outputs are allocated here with torch
unless passed in.

Pages cited: [HF-blog] Hugging Face blog "A Gentle Introduction to 8-bit Matrix
Multiplication for transformers at scale using Hugging Face Transformers,
Accelerate and bitsandbytes"; [Summary] paper summary page "LLM.int8(): 8-Bit
Matrix Multiplication for Transformers at Scale".
"""

import ctypes
import math

import torch

from . import _lib

DEFAULT_THRESHOLD = 6.0  # [HF-blog] "Inside the MatMul": magnitude 6 or more


def outlier_ld(n):
    """Row stride (in halfs) of the gathered outlier columns: n rounded up to 32."""
    return (int(n) + 31) // 32 * 32


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU (the path runs on the GPU only)" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %d" % (name, ndim, t.dim()))


def _flatten_tokens(X):
    """[..., K] -> [M, K] (tokens of all leading dims are the rows)."""
    if X.dim() < 2:
        raise ValueError("X must be at least 2-D")
    return X.reshape(math.prod(X.shape[:-1]), X.shape[-1])   # (-1 is ambiguous when K == 0)


def int8_quantize_colwise_weight(W, Wq=None, sw=None):
    """Per-output-row absmax quantization of W [N, K] fp16 -> (Wq int8 [N, K], sw fp32 [N])."""
    lib = _lib.load_library()
    _need(W, "W", torch.float16, 2)
    N, K = W.shape
    Wq = Wq if Wq is not None else torch.empty((N, K), dtype=torch.int8, device=W.device)
    sw = sw if sw is not None else torch.empty((N,), dtype=torch.float32, device=W.device)
    _need(Wq, "Wq", torch.int8, 2)
    _need(sw, "sw", torch.float32, 1)
    _lib.check(lib.int8_quantize_colwise_weight(_ptr(W), N, K, _ptr(Wq), _ptr(sw),
                                                _stream(W.device)))
    return Wq, sw


def int8_quantize_rowwise(X, outlier_bitmap=None, Xq=None, sx=None):
    """Row-wise absmax quantization of X [M, K] fp16 over its non-outlier columns
    -> (Xq int8 [M, K], sx fp32 [M])."""
    lib = _lib.load_library()
    _need(X, "X", torch.float16)
    X2 = _flatten_tokens(X)
    M, K = X2.shape
    if outlier_bitmap is not None:
        _need(outlier_bitmap, "outlier_bitmap", torch.int32, 1)
        if outlier_bitmap.numel() < (K + 31) // 32:
            raise ValueError("outlier_bitmap too small")
    Xq = Xq if Xq is not None else torch.empty((M, K), dtype=torch.int8, device=X.device)
    sx = sx if sx is not None else torch.empty((M,), dtype=torch.float32, device=X.device)
    _lib.check(lib.int8_quantize_rowwise(_ptr(X2), M, K, _ptr(outlier_bitmap), _ptr(Xq), _ptr(sx),
                                         _stream(X.device)))
    return Xq, sx


def outlier_detect_gather(X, threshold=DEFAULT_THRESHOLD, gather=True):
    """Outlier columns of X [M, K] fp16.

    Returns (bitmap int32 [ceil(K/32)] (bit patterns of the uint32 words),
    cols int32 [K] (first n valid, ascending), n int32 [1] on the device,
    Xo fp16 flat buffer of capacity M * outlier_ld(K) holding [M, outlier_ld(n)]
    or None).
    """
    lib = _lib.load_library()
    _need(X, "X", torch.float16)
    X2 = _flatten_tokens(X)
    M, K = X2.shape
    dev = X.device
    bitmap = torch.empty(((K + 31) // 32,), dtype=torch.int32, device=dev)
    cols = torch.empty((max(K, 1),), dtype=torch.int32, device=dev)
    n = torch.empty((1,), dtype=torch.int32, device=dev)
    Xo = torch.empty((max(M * outlier_ld(K), 1),), dtype=torch.float16, device=dev) if gather else None
    _lib.check(lib.outlier_detect_gather(_ptr(X2), M, K, float(threshold), _ptr(bitmap), _ptr(cols),
                                         _ptr(n), _ptr(Xo), _stream(dev)))
    return bitmap, cols, n, Xo


def int8_mm_dequant(Xq, Wq, sx, sw, Xo=None, cols=None, n=None, bias=None, want_y=True,
                    want_int32=False):
    """int8 GEMM (int32 accumulation) with the fused dequantization, fp16 outlier
    product and bias. Returns Y fp16 [M, N] and/or C int32 [M, N]."""
    lib = _lib.load_library()
    _need(Xq, "Xq", torch.int8, 2)
    _need(Wq, "Wq", torch.int8, 2)
    _need(sx, "sx", torch.float32, 1)
    _need(sw, "sw", torch.float32, 1)
    M, K = Xq.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or sx.numel() != M or sw.numel() != N:
        raise ValueError("shape mismatch")
    if bias is not None:
        _need(bias, "bias", torch.float16, 1)
        if bias.numel() != N:
            raise ValueError("bias must have N entries")
    dev = Xq.device
    Y = torch.empty((M, N), dtype=torch.float16, device=dev) if want_y else None
    C = torch.empty((M, N), dtype=torch.int32, device=dev) if want_int32 else None
    _lib.check(lib.int8_mm_dequant(_ptr(Xq), _ptr(Wq), _ptr(sx), _ptr(sw), M, N, K, _ptr(Xo),
                                   _ptr(cols), _ptr(n), _ptr(bias), _ptr(Y), _ptr(C),
                                   _stream(dev)))
    if want_y and want_int32:
        return Y, C
    return Y if want_y else C


def workspace_bytes(M, K, N=None):
    """Workspace bytes of linear_int8_mixed for M tokens and K features; with N
    (output features) given, the size that also enables the fast path for
    many outlier columns."""
    lib = _lib.load_library()
    if N is None:
        return int(lib.linear_int8_mixed_workspace_bytes(int(M), int(K)))
    return int(lib.linear_int8_mixed_workspace_bytes_many_outliers(int(M), int(K), int(N)))


def workspace_offsets(M, K):
    """Byte offsets of bitmap, cols, n, sx, Xq, Xo in the workspace, and its size."""
    lib = _lib.load_library()
    off = (ctypes.c_int64 * 7)()
    _lib.check(lib.i8mm_workspace_offsets(int(M), int(K), off))
    keys = ("bitmap", "cols", "n", "sx", "Xq", "Xo", "total")
    return dict(zip(keys, [int(v) for v in off]))


def linear_int8_mixed(X, Wq, sw, bias=None, threshold=DEFAULT_THRESHOLD, workspace=None, out=None):
    """The whole layer: Y = X . W^T with outlier decomposition, for an int8 weight
    (Wq, sw) from int8_quantize_colwise_weight. X [..., K] fp16 -> Y [..., N] fp16."""
    lib = _lib.load_library()
    _need(X, "X", torch.float16)
    _need(Wq, "Wq", torch.int8, 2)
    _need(sw, "sw", torch.float32, 1)
    lead = X.shape[:-1]
    X2 = _flatten_tokens(X)
    M, K = X2.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or sw.numel() != N:
        raise ValueError("shape mismatch")
    if bias is not None:
        _need(bias, "bias", torch.float16, 1)
    dev = X.device
    if workspace is None:
        need = workspace_bytes(M, K, N)
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(Y, "out", torch.float16)
    _lib.check(lib.linear_int8_mixed(_ptr(X2), M, K, _ptr(Wq), _ptr(sw), N, _ptr(bias),
                                     float(threshold), _ptr(Y), _ptr(workspace),
                                     workspace.numel(), _stream(dev)))
    return Y.reshape(*lead, N)


def linear_int8_mixed_fp16_weights(X, W, Wq, sw, quantize_weight=True, bias=None,
                                   threshold=DEFAULT_THRESHOLD, workspace=None, out=None):
    """The whole layer for a weight kept in fp16 (has_fp16_weights=True).
    W [N, K] fp16; Wq [N, K] int8 and sw [N] fp32 are caller-owned buffers that
    receive W's codes when quantize_weight (else they must already hold them).
    The outlier product uses W's own columns. X [..., K] fp16 -> Y [..., N]."""
    lib = _lib.load_library()
    _need(X, "X", torch.float16)
    _need(W, "W", torch.float16, 2)
    _need(Wq, "Wq", torch.int8, 2)
    _need(sw, "sw", torch.float32, 1)
    lead = X.shape[:-1]
    X2 = _flatten_tokens(X)
    M, K = X2.shape
    N = W.shape[0]
    if W.shape[1] != K or tuple(Wq.shape) != (N, K) or sw.numel() != N:
        raise ValueError("shape mismatch")
    if bias is not None:
        _need(bias, "bias", torch.float16, 1)
    dev = X.device
    if workspace is None:
        need = workspace_bytes(M, K, N)
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(Y, "out", torch.float16)
    _lib.check(lib.linear_int8_mixed_fp16_weights(
        _ptr(X2), M, K, _ptr(W), N, _ptr(Wq), _ptr(sw), 1 if quantize_weight else 0, _ptr(bias),
        float(threshold), _ptr(Y), _ptr(workspace), workspace.numel(), _stream(dev)))
    return Y.reshape(*lead, N)


def gelu_f16(X, out=None):
    """Exact-erf GELU in fp32 on an fp16 tensor (glue between MLP layers)."""
    lib = _lib.load_library()
    _need(X, "X", torch.float16)
    Y = out if out is not None else torch.empty_like(X)
    _lib.check(lib.i8mm_gelu_f16(_ptr(X), X.numel(), _ptr(Y), _stream(X.device)))
    return Y


def workspace_views(workspace, M, K, N=None):
    """Typed views of the intermediates inside a linear_int8_mixed workspace.
    Given N and a workspace of workspace_bytes(M, K, N), also "Wo": the fp16
    outlier weight columns the tiled path materializes with more than 16
    outlier columns, N rows outlier_ld(n) halfs apart (flat, capacity
    N * outlier_ld(K))."""
    off = workspace_offsets(M, K)
    w = workspace
    views = {
        "bitmap": w[off["bitmap"]:off["bitmap"] + ((K + 31) // 32) * 4].view(torch.int32),
        "cols": w[off["cols"]:off["cols"] + K * 4].view(torch.int32),
        "n": w[off["n"]:off["n"] + 4].view(torch.int32),
        "sx": w[off["sx"]:off["sx"] + M * 4].view(torch.float32),
        "Xq": w[off["Xq"]:off["Xq"] + M * K].view(torch.int8).view(M, K),
        "Xo": w[off["Xo"]:off["Xo"] + M * outlier_ld(K) * 2].view(torch.float16),
    }
    if N is not None:
        end = off["total"] + int(N) * outlier_ld(K) * 2
        if workspace.numel() < end:
            raise ValueError("workspace has no outlier weight region for N=%d" % N)
        views["Wo"] = w[off["total"]:end].view(torch.float16)
    return views

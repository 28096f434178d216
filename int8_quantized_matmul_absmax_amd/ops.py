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


def _need(t, name, dtype, ndim=None, shape=None, min_numel=None):
    """Type, dtype, contiguity and size of one tensor argument (no device check:
    _on_gpu does that for all arguments of a call together)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %d" % (name, ndim, t.dim()))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s must hold at least %d elements, got %d" % (name, min_numel, t.numel()))


def _on_gpu(**tensors):
    """Every given tensor (None = absent) is on one GPU; returns that device.
    The path runs on the GPU only: a host tensor is an error, not a fallback."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("%s must be on a GPU (the path runs on the GPU only)" % name)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, the other arguments on %s" % (name, t.device, dev))
    return dev


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
    if Wq is not None:
        _need(Wq, "Wq", torch.int8, shape=(N, K))
    if sw is not None:
        _need(sw, "sw", torch.float32, shape=(N,))
    dev = _on_gpu(W=W, Wq=Wq, sw=sw)
    Wq = Wq if Wq is not None else torch.empty((N, K), dtype=torch.int8, device=dev)
    sw = sw if sw is not None else torch.empty((N,), dtype=torch.float32, device=dev)
    _lib.check(lib.int8_quantize_colwise_weight(_ptr(W), N, K, _ptr(Wq), _ptr(sw),
                                                _stream(dev)))
    return Wq, sw


def int8_quantize_rowwise(X, outlier_bitmap=None, Xq=None, sx=None):
    """Row-wise absmax quantization of X [M, K] fp16 over its non-outlier columns
    -> (Xq int8 [M, K], sx fp32 [M])."""
    lib = _lib.load_library()
    _need(X, "X", torch.float16)
    X2 = _flatten_tokens(X)
    M, K = X2.shape
    if outlier_bitmap is not None:
        _need(outlier_bitmap, "outlier_bitmap", torch.int32, 1, min_numel=(K + 31) // 32)
    if Xq is not None:
        _need(Xq, "Xq", torch.int8, shape=(M, K))
    if sx is not None:
        _need(sx, "sx", torch.float32, shape=(M,))
    dev = _on_gpu(X=X, outlier_bitmap=outlier_bitmap, Xq=Xq, sx=sx)
    Xq = Xq if Xq is not None else torch.empty((M, K), dtype=torch.int8, device=dev)
    sx = sx if sx is not None else torch.empty((M,), dtype=torch.float32, device=dev)
    _lib.check(lib.int8_quantize_rowwise(_ptr(X2), M, K, _ptr(outlier_bitmap), _ptr(Xq), _ptr(sx),
                                         _stream(dev)))
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
    dev = _on_gpu(X=X)
    bitmap = torch.empty(((K + 31) // 32,), dtype=torch.int32, device=dev)
    cols = torch.empty((max(K, 1),), dtype=torch.int32, device=dev)
    n = torch.empty((1,), dtype=torch.int32, device=dev)
    Xo = torch.empty((max(M * outlier_ld(K), 1),), dtype=torch.float16, device=dev) if gather else None
    _lib.check(lib.outlier_detect_gather(_ptr(X2), M, K, float(threshold), _ptr(bitmap), _ptr(cols),
                                         _ptr(n), _ptr(Xo), _stream(dev)))
    return bitmap, cols, n, Xo


def outlier_detect_quantize(X, threshold=DEFAULT_THRESHOLD, workspace=None):
    """The activation side of linear_int8_mixed alone (detection, gather and
    row quantization, the same two kernels) into a layer workspace. Returns
    the workspace; workspace_views(workspace, M, K) gives bitmap, cols, n, sx,
    Xq and Xo, which int8_mm_dequant takes."""
    lib = _lib.load_library()
    _need(X, "X", torch.float16)
    X2 = _flatten_tokens(X)
    M, K = X2.shape
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1, min_numel=workspace_bytes(M, K))
    dev = _on_gpu(X=X, workspace=workspace)
    if workspace is None:
        workspace = torch.empty((max(workspace_bytes(M, K), 1),), dtype=torch.uint8, device=dev)
    _lib.check(lib.outlier_detect_quantize(_ptr(X2), M, K, float(threshold), _ptr(workspace),
                                           workspace.numel(), _stream(dev)))
    return workspace


def int8_mm_dequant(Xq, Wq, sx, sw, Xo=None, cols=None, n=None, bias=None, want_y=True,
                    want_int32=False, out=None):
    """int8 GEMM (int32 accumulation) with the fused dequantization, fp16 outlier
    product and bias. Returns Y fp16 [M, N] and/or C int32 [M, N].

    Xo, cols, n come together (from outlier_detect_gather or a layer
    workspace): Xo fp16 of capacity >= M * outlier_ld(K) (the count n is only
    known on the device, so room for every column is required), cols int32
    with >= K entries, n int32 [1] on the device."""
    lib = _lib.load_library()
    _need(Xq, "Xq", torch.int8, 2)
    M, K = Xq.shape
    _need(Wq, "Wq", torch.int8, 2)
    N = Wq.shape[0]
    _need(Wq, "Wq", torch.int8, shape=(N, K))
    _need(sx, "sx", torch.float32, shape=(M,))
    _need(sw, "sw", torch.float32, shape=(N,))
    given = [t is not None for t in (Xo, cols, n)]
    if any(given) and not all(given):
        raise ValueError("Xo, cols and n must be given together")
    if Xo is not None:
        _need(Xo, "Xo", torch.float16, min_numel=M * outlier_ld(K))
        _need(cols, "cols", torch.int32, min_numel=K)
        _need(n, "n", torch.int32, shape=(1,))
    if bias is not None:
        _need(bias, "bias", torch.float16, shape=(N,))
    if out is not None:
        _need(out, "out", torch.float16, shape=(M, N))
    if not (want_y or want_int32):
        raise ValueError("nothing requested: want_y and want_int32 are both False")
    dev = _on_gpu(Xq=Xq, Wq=Wq, sx=sx, sw=sw, Xo=Xo, cols=cols, n=n, bias=bias, out=out)
    Y = None
    if want_y:
        Y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
    C = torch.empty((M, N), dtype=torch.int32, device=dev) if want_int32 else None
    _lib.check(lib.int8_mm_dequant(_ptr(Xq), _ptr(Wq), _ptr(sx), _ptr(sw), M, N, K, _ptr(Xo),
                                   _ptr(cols), _ptr(n), _ptr(bias), _ptr(Y), _ptr(C),
                                   _stream(dev)))
    if want_y and want_int32:
        return Y, C
    return Y if want_y else C


def workspace_bytes(M, K, N=None):
    """Workspace bytes of linear_int8_mixed for M tokens and K features; with N
    (output features) given, the size with a region of recovered outlier
    weights with room for 512 columns, which speeds up 17 to 512 outlier
    columns; without it every outlier count still takes a second GEMM loop.
    Any larger workspace has room for floor(extra / (2 N) / 32) * 32 columns
    (see workspace_bytes_all_outliers)."""
    lib = _lib.load_library()
    if N is None:
        return int(lib.linear_int8_mixed_workspace_bytes(int(M), int(K)))
    return int(lib.linear_int8_mixed_workspace_bytes_many_outliers(int(M), int(K), int(N)))


def workspace_bytes_all_outliers(M, K, N):
    """Workspace bytes whose outlier weight region has room for every outlier
    count (K columns): the fastest layer at any count, for N * outlier_ld(K)
    * 2 extra bytes."""
    base = workspace_bytes(M, K)
    return base + int(N) * outlier_ld(int(K)) * 2 if base else 0


def outlier_region_cols(workspace_bytes_, M, K, N):
    """Outlier columns a workspace of workspace_bytes_ bytes has room for in
    its recovered-weight region (0 means none)."""
    extra = int(workspace_bytes_) - workspace_bytes(M, K)
    if extra <= 0 or N <= 0:
        return 0
    return min(extra // (2 * int(N)) // 32 * 32, outlier_ld(int(K)))


def workspace_layout(M, K):
    """Byte offsets of bitmap, cols, n, sx, Xq, Xo in the workspace, and its size."""
    lib = _lib.load_library()
    off = (ctypes.c_int64 * 7)()
    _lib.check(lib.i8mm_workspace_layout(int(M), int(K), off))
    keys = ("bitmap", "cols", "n", "sx", "Xq", "Xo", "total")
    return dict(zip(keys, [int(v) for v in off]))


def _layer_buffers(X, N, bias, workspace, out, K_w, W_name):
    """Shared argument checks of the two layer calls; returns (X2, M, K, dev,
    workspace, Y, lead)."""
    lead = X.shape[:-1]
    X2 = _flatten_tokens(X)
    M, K = X2.shape
    if K_w != K:
        raise ValueError("%s has %d input features, X has %d" % (W_name, K_w, K))
    if bias is not None:
        _need(bias, "bias", torch.float16, shape=(N,))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1, min_numel=workspace_bytes(M, K))
    if out is not None:
        _need(out, "out", torch.float16)
        if out.numel() != M * N:
            raise ValueError("out must hold M * N = %d elements, got %d" % (M * N, out.numel()))
    return X2, M, K, lead


def linear_int8_mixed(X, Wq, sw, bias=None, threshold=DEFAULT_THRESHOLD, workspace=None, out=None):
    """The whole layer: Y = X . W^T with outlier decomposition, for an int8 weight
    (Wq, sw) from int8_quantize_colwise_weight. X [..., K] fp16 -> Y [..., N] fp16.
    Without a workspace, one of workspace_bytes(M, K, N) bytes is allocated."""
    lib = _lib.load_library()
    _need(X, "X", torch.float16)
    _need(Wq, "Wq", torch.int8, 2)
    N = Wq.shape[0]
    _need(sw, "sw", torch.float32, shape=(N,))
    X2, M, K, lead = _layer_buffers(X, N, bias, workspace, out, Wq.shape[1], "Wq")
    dev = _on_gpu(X=X, Wq=Wq, sw=sw, bias=bias, workspace=workspace, out=out)
    if workspace is None:
        workspace = torch.empty((max(workspace_bytes(M, K, N), 1),), dtype=torch.uint8, device=dev)
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
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
    N, K_w = W.shape
    _need(Wq, "Wq", torch.int8, shape=(N, K_w))
    _need(sw, "sw", torch.float32, shape=(N,))
    X2, M, K, lead = _layer_buffers(X, N, bias, workspace, out, K_w, "W")
    dev = _on_gpu(X=X, W=W, Wq=Wq, sw=sw, bias=bias, workspace=workspace, out=out)
    if workspace is None:
        workspace = torch.empty((max(workspace_bytes(M, K, N), 1),), dtype=torch.uint8, device=dev)
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
    _lib.check(lib.linear_int8_mixed_fp16_weights(
        _ptr(X2), M, K, _ptr(W), N, _ptr(Wq), _ptr(sw), 1 if quantize_weight else 0, _ptr(bias),
        float(threshold), _ptr(Y), _ptr(workspace), workspace.numel(), _stream(dev)))
    return Y.reshape(*lead, N)


def gelu_f16(X, out=None):
    """Exact-erf GELU in fp32 on an fp16 tensor (glue between MLP layers)."""
    lib = _lib.load_library()
    _need(X, "X", torch.float16)
    if out is not None:
        _need(out, "out", torch.float16, min_numel=X.numel())
    dev = _on_gpu(X=X, out=out)
    Y = out if out is not None else torch.empty_like(X)
    _lib.check(lib.i8mm_gelu_f16(_ptr(X), X.numel(), _ptr(Y), _stream(dev)))
    return Y


OUTLIER_REGION_COLS = 512   # I8MM_OUTLIER_REGION_COLS


def workspace_views(workspace, M, K, N=None):
    """Typed views of the intermediates inside a linear_int8_mixed workspace.
    Given N and a workspace larger than workspace_bytes(M, K), also "Wo": the
    region of fp16 outlier weight columns the tiled path materializes when
    16 < n <= outlier_region_cols(...), N rows outlier_ld(n) halfs apart
    (flat, the region's whole room)."""
    off = workspace_layout(M, K)
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
        room = outlier_region_cols(workspace.numel(), M, K, N)
        if room == 0:
            raise ValueError("workspace has no outlier weight region for N=%d" % N)
        end = off["total"] + int(N) * room * 2
        views["Wo"] = w[off["total"]:end].view(torch.float16)
    return views

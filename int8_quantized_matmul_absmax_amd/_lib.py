"""ctypes loader of libi8mm.so and the prototypes of its C ABI (include/i8mm.h)."""

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libi8mm.so")

I8MM_OK = 0
I8MM_EINVAL = -1
I8MM_EALIGN = -2
I8MM_EWORKSPACE = -3
I8MM_ENODEVICE = -4
I8MM_ELAUNCH = -5
I8MM_ERANGE = -6
I8MM_MAX_K = 133144
I8MM_NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol include/i8mm.h declares.
EXPORTS = (
    "int8_quantize_colwise_weight",
    "int8_quantize_rowwise",
    "outlier_detect_gather",
    "outlier_detect_quantize",
    "int8_mm_dequant",
    "linear_int8_mixed",
    "linear_int8_mixed_noalloc",
    "linear_int8_mixed_fp16_weights",
    "linear_int8_mixed_workspace_bytes",
    "linear_int8_mixed_workspace_bytes_many_outliers",
    "i8mm_workspace_layout",
    "i8mm_gelu_f16",
    "i8mm_last_error",
    "i8mm_status_string",
)

_lock = threading.Lock()
_lib = None


class I8mmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (%d): %s" % (_status_name(status), status, message))
        self.status = status


def _status_name(status):
    names = {0: "I8MM_OK", -1: "I8MM_EINVAL", -2: "I8MM_EALIGN", -3: "I8MM_EWORKSPACE",
             -4: "I8MM_ENODEVICE", -5: "I8MM_ELAUNCH", -6: "I8MM_ERANGE"}
    return names.get(status, "I8MM_UNKNOWN")


def _declare(lib):
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    sig = {
        "int8_quantize_colwise_weight": ([vp, i64, i64, vp, vp, vp], i32),
        "int8_quantize_rowwise": ([vp, i64, i64, vp, vp, vp, vp], i32),
        "outlier_detect_gather": ([vp, i64, i64, f32, vp, vp, vp, vp, vp], i32),
        "outlier_detect_quantize": ([vp, i64, i64, f32, vp, ctypes.c_size_t, vp], i32),
        "int8_mm_dequant": ([vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp], i32),
        "linear_int8_mixed": ([vp, i64, i64, vp, vp, i64, vp, f32, vp, vp, ctypes.c_size_t, vp],
                              i32),
        "linear_int8_mixed_noalloc": ([vp, i64, i64, vp, vp, i64, vp, f32, vp, vp], i32),
        "linear_int8_mixed_fp16_weights": ([vp, i64, i64, vp, i64, vp, vp, i32, vp, f32, vp, vp,
                                            ctypes.c_size_t, vp], i32),
        "linear_int8_mixed_workspace_bytes": ([i64, i64], ctypes.c_size_t),
        "linear_int8_mixed_workspace_bytes_many_outliers": ([i64, i64, i64], ctypes.c_size_t),
        "i8mm_workspace_layout": ([i64, i64, ctypes.POINTER(ctypes.c_int64)], i32),
        "i8mm_gelu_f16": ([vp, i64, vp, vp], i32),
        "i8mm_last_error": ([], ctypes.c_char_p),
        "i8mm_status_string": ([i32], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res


def load_library(path=None):
    """Load libi8mm.so (once). Raises ImportError if it is not built.

    torch is imported first so that the library binds to the HIP runtime
    torch already loaded (same soname): device pointers and streams handed
    over from torch are then valid in the library.
    """
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise ImportError("libi8mm.so is not built (expected at %s); build it with "
                              "python -m int8_quantized_matmul_absmax_amd.build" % p)
        import torch  # noqa: F401
        lib = ctypes.CDLL(p)
        _declare(lib)
        _lib = lib
        return lib


def check(status):
    if status != I8MM_OK:
        msg = _lib.i8mm_last_error()
        raise I8mmError(status, msg.decode() if msg else "")
    return status

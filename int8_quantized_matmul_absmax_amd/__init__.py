"""LLM.int8() mixed-precision int8 linear layer for AMD Instinct MI355X (gfx950).

The compute runs in hand-written HIP kernels (libi8mm.so, C ABI declared in
include/i8mm.h); this package is the Python binding. Loading is lazy: importing
the package does not need a GPU, calling an op does, and an op raises if the
library is not built or no gfx950 GPU is current.
"""

from ._lib import EXPORTS, I8mmError, LIB_PATH, load_library  # noqa: F401


def ensure_built():
    """Load libi8mm.so, building it first only if it does not exist."""
    import os
    if not os.path.exists(LIB_PATH):
        from .build import build_library
        build_library()
    return load_library()


def __getattr__(name):
    # ops and the module are imported on first use (they import torch)
    if name in ("ops", "linear", "synth"):
        import importlib
        return importlib.import_module("." + name, __name__)
    if name == "Int8Linear":
        from .linear import Int8Linear
        return Int8Linear
    from . import ops as _ops
    if hasattr(_ops, name):
        return getattr(_ops, name)
    raise AttributeError(name)

"""group_limited_top_amd -- forward pass of a group-limited top-k sparse-MoE
layer on one AMD Instinct MI355X (gfx950), as hand-written HIP kernels behind
the C ABI in include/moe.h.

The binding (``group_limited_top_amd._lib``) is imported lazily so that the
input generators (``synth``) and the build script work without the built
library; calling any entry point without libmoe.so raises ImportError.
"""
__all__ = ["lib", "synth"]


def lib():
    """The ctypes binding of libmoe (raises ImportError when it is not built)."""
    from . import _lib
    return _lib

"""Fused tiled self-attention for AMD Instinct MI355X (gfx950).

The computation lives in libattn.so (hand-written HIP kernels behind the C ABI
of include/attn.h); ``tiled_attention_08_amd._lib`` is its ctypes binding.
This package root stays import-light so that the build step can import it
before the library exists.
"""

__all__ = ["load"]


def load():
    """Return the binding module; raises ImportError if libattn.so is not built."""
    from . import _lib
    return _lib

"""CacheGen KV-cache codec for AMD Instinct MI355X (gfx950).

The codec lives in a C-ABI shared library of hand-written HIP kernels
(``libcachegen_mi355x.so``, declared in ``include/cachegen.h``). The binding in
:mod:`kv_cache_compression_layer_amd.cachegen` marshals torch device tensors
into it. Importing this package loads nothing; the library is loaded on first
use of the binding and a missing library is an error, never a fallback.
"""

__all__ = ["cachegen", "synth"]

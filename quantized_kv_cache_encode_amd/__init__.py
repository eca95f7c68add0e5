"""Attention computed directly from quantized key-cache codes on AMD MI355X.

The computation runs in libkvq.so (hand-written HIP for gfx950, C ABI in
include/kvq.h); ``quantized_kv_cache_encode_amd.kvq`` is its Python binding.
Importing the binding fails if the library has not been built
(``python -m quantized_kv_cache_encode_amd.build``).
"""
import importlib

__all__ = ["kvq"]


def __getattr__(name):
    # Only the binding and the names it defines are resolved here; anything else (the `build` submodule
    # in particular) is left to the import system, so building never needs the library to exist.
    if name == "kvq":
        return importlib.import_module(".kvq", __name__)
    if name.startswith(("kvq_", "KVQ_", "Kvq")):
        mod = importlib.import_module(".kvq", __name__)
        if hasattr(mod, name):
            return getattr(mod, name)
    raise AttributeError(name)

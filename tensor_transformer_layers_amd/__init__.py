"""MI355X-native tensor-parallel linear pair (column -> activation -> row).

The compute lives in the HIP library ``libtp.so`` (C ABI, declared in
include/tp.h).  ``tensor_transformer_layers_amd.tp`` is the thin ctypes
binding; importing this package does not load the library.
"""
__all__ = ["configs", "inputs"]

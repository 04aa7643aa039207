"""MI355X-native VDN-H3 dual-branch hybrid attention layer.

The compute path is the HIP library ``libhybattn.so`` (C-ABI declared in
``include/hyb_attn.h``); ``api`` is a thin ctypes binding over it.  Importing
this package does not load the library; ``api.load()`` does, and raises if it
is missing.
"""
__all__ = ["inputs", "api"]

"""log_linear_token_amd: the log-linear (Fenwick-tree) token mixer on MI355X.

The compute lives in the HIP library ``libloglin.so`` (C ABI declared in
``include/loglin.h``); ``log_linear_token_amd.loglin`` is the thin ctypes
binding with the same entry-point names.  Importing this package loads
nothing; ``loglin`` loads the library on first use and raises if it is
missing.
"""
__all__ = ["inputs", "loglin"]

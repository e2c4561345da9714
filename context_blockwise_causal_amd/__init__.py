"""libringattn: one context-parallel rank's share of blockwise causal ring attention on MI355X.

The compute path is the HIP library ``libringattn.so`` (C ABI in ``include/ra.h``); ``api``
is its torch-facing binding and ``_lib`` the raw ctypes layer.  Importing this package does not
load the library; the first call that needs it does, and fails loudly if it is not built.
"""
__all__ = ["api", "inputs", "workloads"]

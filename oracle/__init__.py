"""FP64 CPU oracle (test infrastructure only; never imported by the product path).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP library or its binding.
"""
from . import attn64  # noqa: F401

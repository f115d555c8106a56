"""Plain float64 CPU oracle for quantization-aware attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""
from . import fp8, qat_attention  # noqa: F401

"""MI355X-native quantization-aware attention (fake-quant FP8 attention with a
straight-through backward).  Hand-written HIP kernels for gfx950 behind the C
ABI declared in ``include/qat_attn.h``; this package holds the ctypes binding
(``ops``) and the seeded synthetic workloads (``workloads``).

Submodules are imported lazily so that host-only code (workload generation)
does not need the built library.
"""
import importlib

__all__ = ["ops", "workloads", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)

"""MI355X-native quantization-aware attention (fake-quant FP8 attention with a
straight-through backward).  Hand-written HIP kernels for gfx950 behind the C
ABI declared in ``include/qat_attn.h``; this package holds the ctypes binding
(``ops``) and the seeded synthetic workloads (``workloads``).

The binding is imported lazily so that host-only code (workload generation)
does not need the built library.
"""
__all__ = ["ops", "workloads"]


def __getattr__(name):
    if name == "ops":
        from . import ops
        return ops
    if name == "workloads":
        from . import workloads
        return workloads
    raise AttributeError(name)

"""QK4V8 attention for MI355X (gfx950): MXFP4 Q/K, FP8 E4M3 V, FP32 online
softmax, behind the C ABI declared in include/qk4v8.h.

Importing the package does not load the native library; ``ops`` does, on
first use, and raises if it is missing (there is no CPU fallback).
"""

__all__ = ["ops", "synth"]


def __getattr__(name):
    if name in ("ops", "synth"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)

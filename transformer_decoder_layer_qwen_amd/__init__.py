"""One Qwen-style pre-norm decoder layer (forward) on AMD Instinct MI355X (gfx950).

The compute lives in ``libqlayer.so`` (hand-written HIP kernels behind the C ABI
of ``include/qlayer.h``); ``binding`` is a thin ctypes layer over it.
"""
from . import configs  # noqa: F401

__all__ = ["configs", "synth", "binding", "build"]

"""Sampled-softmax cross-entropy LM-head step for AMD Instinct MI355X (gfx950).

The compute path lives in the HIP library ``libsampledce.so`` (C ABI declared in
``include/sampled_ce.h``); ``binding`` is a thin ctypes layer that passes device
pointers and the current HIP stream. ``synth`` draws seeded synthetic inputs.
Importing the package loads nothing; the library is loaded on first use and a
missing library is an error, never a fallback.
"""
__all__ = ["binding", "synth"]

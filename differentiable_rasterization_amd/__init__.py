"""MI355X-native 3D Gaussian-splatting training step.

The compute lives in ``libgsmi.so`` (hand-written HIP kernels for gfx950 behind
a C ABI, declared in ``include/gs.h``).  ``binding`` marshals torch tensors to
that ABI; ``scenes`` generates seeded synthetic inputs.  Importing this package
does not load the library; ``binding`` does, and fails loudly if it is missing.
"""
__all__ = ["scenes", "binding", "memory"]

"""MI355X-native speculative-sampling verify (modified rejection sampling).

Submodules:
  synth    seeded synthetic inputs (no verify arithmetic)
  binding  ctypes binding of the C-ABI library libspec_softmax.so (HIP, gfx950)
  build    compiles libspec_softmax.so with hipcc

Nothing is loaded at import time; ``binding`` loads the HIP library on first
use and raises if it is missing.
"""

__all__ = ["synth", "binding", "build"]

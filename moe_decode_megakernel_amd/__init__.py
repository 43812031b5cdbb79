"""MI355X (gfx950) speculative-verify MoE layer kernel.

Submodules:
  msk    thin ctypes binding of libmsk.so (include/msk.h); loads the library on
         first use and raises if it is missing
  synth  seeded synthetic workloads (host and device fillers)
  build  compiles the native libraries in place
"""
__all__ = ["msk", "synth", "build"]

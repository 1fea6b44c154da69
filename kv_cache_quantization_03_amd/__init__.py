"""TurboQuant KV-cache and vector codec for AMD MI355X (gfx950).

The compute path is libtq.so (hand-written HIP kernels behind a C ABI, see
include/tq.h); ``binding`` is its thin ctypes wrapper and raises on import
when the library has not been built.  ``inputs`` holds the seeded synthetic
workloads.
"""
__all__ = ["binding", "inputs", "build"]

"""MI355X-native forward of the FLUX.3 Image Klein parallel DiT block.

The compute path is a C-ABI shared library of HIP kernels for gfx950
(``csrc/``); ``ops`` is a thin ctypes binding over it that only marshals
arguments.  ``configs`` and ``inputs`` hold shapes and seeded input draws.
"""
__all__ = ["configs", "inputs"]

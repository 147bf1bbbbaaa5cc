"""MI355X-native Fathom bit-plane key scan.

The work happens in ``libfathom.so`` (hand-written HIP kernels for gfx950 behind a C-ABI
declared in ``include/fathom.h``).  ``bit_plane_kv_amd.fathom`` is the thin ctypes
binding with the same call names; ``bit_plane_kv_amd.synth`` draws seeded synthetic
inputs.  Importing this package loads nothing; the library is loaded on first use and
the binding raises if it is missing -- there is no CPU fallback.
"""
__all__ = ["fathom", "synth"]

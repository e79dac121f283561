"""MI355X-native DualQuant dual-scale quantizer (block-coordinate descent).

The solver itself lives in a C-ABI shared library of hand-written HIP for
gfx950 (``csrc/``, declared in ``include/dq.h``). ``dq`` is the thin ctypes
binding with the same entry-point names; ``synth`` draws seeded inputs.
Importing this package loads nothing; the library is loaded on first use
and a missing build is an error, never a fallback.
"""

__all__ = ["dq", "synth"]

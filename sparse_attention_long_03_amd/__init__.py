"""MI355X-native DeepSeek Sparse Attention (DSA) hot path.

The compute lives in a HIP library for gfx950 (``csrc/``) behind a C ABI
(``include/dsa.h``); :mod:`.binding` is a thin ctypes layer over it that only
marshals arguments.  Importing this package does not load the library; the
first call into :mod:`.binding` does, and fails loudly if it is missing.
"""

__all__ = ["binding", "inputs"]

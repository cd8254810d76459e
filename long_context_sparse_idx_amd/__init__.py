"""MI355X-native sparse-index hot path: lightning-indexer scoring, per-row
top-k, cross-layer index reuse (F/S layers) and sparse gather attention.

The compute lives in ``liblcsi.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/lcsi.h``); ``long_context_sparse_idx_amd.lcsi`` is the
thin ctypes binding.  ``inputs`` holds the seeded synthetic workloads.
"""
__version__ = "0.1.0"

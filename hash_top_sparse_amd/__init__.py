"""hash_top_sparse_amd -- HATA decode-step hot path for MI355X (gfx950).

The compute lives in ``libhata.so`` (hand-written HIP kernels behind a C ABI
declared in ``include/hata.h``); ``binding`` is a thin ctypes layer over it
that marshals torch tensors and streams.  Importing this package loads
nothing: call ``binding.load()`` (or any binding function) on a GPU machine.
``synth`` holds the seeded input generators.
"""

__all__ = ["binding", "synth", "build"]

"""Fused chunked top-K KL distillation loss for AMD Instinct MI355X (gfx950).

The compute path is ``libfkl.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fkl.h``); ``sparse_top_kl_amd.fkl`` is a thin ctypes
binding over it and ``sparse_top_kl_amd.synth`` draws seeded synthetic inputs.
The binding loads the library on first use and raises if it is missing: there
is no CPU fallback.
"""

__all__ = ["fkl", "synth"]

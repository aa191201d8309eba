"""Fused chunked top-K KL distillation loss for AMD Instinct MI355X (gfx950).

The compute path is ``libfkl.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fkl.h``); ``sparse_top_kl_amd.fkl`` is a thin ctypes
binding over it and ``sparse_top_kl_amd.synth`` draws seeded synthetic inputs.
The binding loads the library on first use and raises if it is missing: there
is no CPU fallback.

What the library offers (``fkl``):
  * ``fused_chunked_kl`` — the loss with autograd (fused chunked method; with
    ``keep_logits`` the forward-chunked variant; ``row_weight``, ``labels``
    and ``alpha`` for masks, means and the hard-label cross-entropy mixture);
  * ``fkl_forward`` / ``fkl_backward`` (and ``_keep`` / ``_ex`` variants) — the
    C entry points one to one;
  * ``fkl_teacher_topk`` / ``fkl_teacher_topk_ex`` — the teacher top-K cache
    (and the teacher's full-vocabulary lse for the tail-bucket option).
"""

__all__ = ["fkl", "synth"]

"""Seeded synthetic inputs for the fused chunked top-K KL loss.

This module is the only code shared by the HIP path's tests/benchmark and the
CPU oracle. It holds none of the loss arithmetic: it draws hidden states, an
LM-head weight, a teacher top-K id list and teacher logits with the shapes of
the workloads the pages describe, and nothing else. It imports nothing from
the rest of the package.

Stand-ins (no model weights, training data or evaluation suite is used):
  * ``tiny``            512 tokens, d=512, V=8192, fp32 (oracle-sized case)
  * ``llama3b_8k``      8192 tokens at a 3B-student shape (d=3072), Llama
                        vocabulary (128256): the student/teacher experiment of
                        "Multiverse Computing ..." (iitak.ru), fourth paragraph
  * ``long32k``         the isolated 32K-token loss test of the same page,
                        fifth paragraph, at T=2 with Zipf-skewed teacher ids
  * ``gptoss20b_32k``   gpt-oss-20B student shape (d=2880, V=201088) at
                        32768 tokens: same page, first paragraph
  * ``stress_b4_32k`` / ``stress_b1_64k``
                        batch 4 x 32K at the gpt-oss vocabulary (the ~50 GB
                        teacher-tensor example of the malakhovai.ru page) and a
                        65536-token run (the dense loss no longer runs at 64K,
                        iitak.ru fifth paragraph)

Teacher side (inputs of the top-K cache producer; ``TEACHER_WORKLOADS``):
  * ``teacher_tiny``    512 tokens, d=256, V=4096, fp32 (oracle-sized case)
  * ``teacher_llama8b_32k``
                        32768 tokens through a Llama-3.1-8B-shaped teacher
                        head (d=4096, V=128256): the teacher of the student
                        experiment on the iitak.ru page, fourth paragraph
  * ``teacher_gptoss120b_b4_32k``
                        batch 4 x 32K through a gpt-oss-120b-shaped head
                        (d=2880, V=201088): the malakhovai.ru page's
                        teacher-tensor example
  Streams t = 4 (teacher hidden) and 5 (teacher weight); "normal" values as
  for the student (N(0, 1) and N(0, 1/d)), or "integer" values drawn
  uniformly from {-2, ..., 2} for both, so every logit is an exact small
  integer in fp32 and in fp64 (and many logits tie).

Recipe (fixed; tests depend on it):
  * streams ``numpy.random.default_rng([seed, t])`` with t = 0 hidden,
    1 weight, 2 ids, 3 teacher logits;
  * hidden ~ N(0, 1), weight ~ N(0, 1/d), drawn in fp32 in storage order
    (weight stored [V, d]); for bf16 workloads both are rounded to the nearest
    bf16 (ties to even) and returned as fp32 arrays holding bf16 values;
  * ids: K distinct per row, in draw order; uniform over [0, V), or Zipf(1.1)
    over ranks 1..V (P(rank) ~ rank^-1.1, id = rank - 1), drawn with
    replacement and discarding repeats (sequential sampling without
    replacement);
  * teacher logits: K Gumbel(0, 1) draws per row, sorted descending, plus 3,
    so the first-drawn id carries the largest logit.
"""

from __future__ import annotations

import dataclasses

import numpy as np

GENERATOR_VERSION = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    d: int
    V: int
    K: int
    T: float
    dtype: str          # "fp32" or "bf16"
    chunk: int
    ids: str            # "uniform" or "zipf"
    seed: int

    @property
    def N(self) -> int:
        return self.B * self.S


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, 512, 512, 8192, 100, 1.0, "fp32", 128, "uniform", 1001),
        Workload("llama3b_8k", 1, 8192, 3072, 128256, 100, 1.0, "bf16", 1024, "uniform", 1002),
        Workload("long32k", 1, 32768, 3072, 128256, 100, 2.0, "bf16", 2048, "zipf", 1003),
        Workload("gptoss20b_32k", 1, 32768, 2880, 201088, 100, 1.0, "bf16", 2048, "uniform", 1004),
        Workload("stress_b4_32k", 4, 32768, 2880, 201088, 100, 1.0, "bf16", 4096, "zipf", 1005),
        Workload("stress_b1_64k", 1, 65536, 2880, 201088, 100, 1.0, "bf16", 4096, "zipf", 1006),
    ]
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); fp32 result."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    out = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return out.view(np.float32)


def _rng(seed: int, t: int) -> np.random.Generator:
    return np.random.default_rng([seed, t])


def _distinct_in_draw_order(draw, n_rows: int, k: int, batch: int) -> np.ndarray:
    """K distinct values per row, keeping draw order; ``draw(rows, m)`` -> ints."""
    out = np.empty((n_rows, k), dtype=np.int64)
    pending = np.arange(n_rows)
    cand = draw(pending.size, batch)
    while True:
        order = np.argsort(cand, axis=1, kind="stable")
        srt = np.take_along_axis(cand, order, axis=1)
        first_sorted = np.ones_like(srt, dtype=bool)
        first_sorted[:, 1:] = srt[:, 1:] != srt[:, :-1]
        first = np.empty_like(first_sorted)
        np.put_along_axis(first, order, first_sorted, axis=1)
        n_distinct = first.sum(axis=1)
        ok = n_distinct >= k
        if ok.any():
            sel = first[ok] & (np.cumsum(first[ok], axis=1) <= k)
            out[pending[ok]] = cand[ok][sel].reshape(-1, k)
        if ok.all():
            return out
        cand = np.concatenate([cand[~ok], draw(int((~ok).sum()), batch)], axis=1)
        pending = pending[~ok]


def _uniform_ids(rng, n_rows, V, K):
    return _distinct_in_draw_order(
        lambda r, m: rng.integers(0, V, size=(r, m), dtype=np.int64), n_rows, K,
        batch=K + 16)


def zipf_cdf(V: int, a: float = 1.1) -> np.ndarray:
    w = np.arange(1, V + 1, dtype=np.float64) ** (-a)
    c = np.cumsum(w)
    return c / c[-1]


def _zipf_ids(rng, n_rows, V, K, a=1.1):
    cdf = zipf_cdf(V, a)

    def draw(r, m):
        u = rng.random((r, m))
        return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int64)

    return _distinct_in_draw_order(draw, n_rows, K, batch=4 * K)


def _teacher_logits(rng, n_rows, K):
    u = rng.random((n_rows, K))
    u = np.clip(u, np.finfo(np.float64).tiny, 1.0 - 2.0 ** -53)
    g = -np.log(-np.log(u))
    g = -np.sort(-g, axis=1)
    return (g + 3.0).astype(np.float32)


def make_hidden(w: Workload, n_rows: int | None = None) -> np.ndarray:
    n = w.N if n_rows is None else n_rows
    h = _rng(w.seed, 0).standard_normal((n, w.d), dtype=np.float32)
    return round_to_bf16(h) if w.dtype == "bf16" else h


def make_weight(w: Workload) -> np.ndarray:
    W = _rng(w.seed, 1).standard_normal((w.V, w.d), dtype=np.float32)
    W *= np.float32(1.0 / np.sqrt(w.d))
    return round_to_bf16(W) if w.dtype == "bf16" else W


def make_teacher(w: Workload, n_rows: int | None = None):
    n = w.N if n_rows is None else n_rows
    rng = _rng(w.seed, 2)
    if w.ids == "zipf":
        idx = _zipf_ids(rng, n, w.V, w.K)
    else:
        idx = _uniform_ids(rng, n, w.V, w.K)
    logit = _teacher_logits(_rng(w.seed, 3), n, w.K)
    return idx.astype(np.int32), logit


def make_inputs(name_or_workload, n_rows: int | None = None) -> dict:
    """All inputs of a workload; ``n_rows`` truncates/extends the token count.

    Row r of a shorter draw equals row r of the full draw for hidden states
    and teacher logits (same stream, same order); ids match too for uniform
    draws whenever no redraw happened, which is not guaranteed, so callers
    that need identical rows generate the full set and slice.
    """
    w = WORKLOADS[name_or_workload] if isinstance(name_or_workload, str) else name_or_workload
    idx, logit = make_teacher(w, n_rows)
    return {
        "workload": w,
        "hidden": make_hidden(w, n_rows),
        "weight": make_weight(w),
        "topk_idx": idx,
        "topk_logit": logit,
        "T": w.T,
        "chunk": w.chunk,
        "dtype": w.dtype,
    }


def make_loss_options(w: Workload, seed: int = 99) -> dict:
    """Inputs of the loss options at a workload's size: a hard label per row
    (uniform over the vocabulary, stream ``default_rng(seed)``), the mixing
    weight 0.5, and a teacher full-vocabulary log-sum-exp at T per row chosen
    so that the cached entries hold half of the teacher's mass (the log-sum-exp
    of the cached logits / T over the K entries, plus ln 2, in fp64, rounded
    to fp32). Only input data; the loss itself is computed elsewhere."""
    y = np.random.default_rng(seed).integers(0, w.V, size=w.N).astype(np.int32)
    logit = _teacher_logits(_rng(w.seed, 3), w.N, w.K)
    a = logit.astype(np.float64) / w.T
    mx = a.max(axis=1)
    tlse = (mx + np.log(np.exp(a - mx[:, None]).sum(axis=1)) + np.log(2.0)).astype(np.float32)
    return {"labels": y, "alpha": 0.5, "teacher_lse": tlse}


def small_workload(name="small", n=300, d=64, V=1000, K=100, T=1.0, dtype="fp32",
                   chunk=128, ids="uniform", seed=7) -> Workload:
    """A custom (usually tiny) workload with the same recipe."""
    return Workload(name, 1, n, d, V, K, T, dtype, chunk, ids, seed)


@dataclasses.dataclass(frozen=True)
class TeacherWorkload:
    name: str
    B: int
    S: int
    d: int
    V: int
    K: int
    dtype: str          # "fp32" or "bf16"
    chunk: int
    seed: int
    values: str = "normal"   # "normal" or "integer"

    @property
    def N(self) -> int:
        return self.B * self.S


TEACHER_WORKLOADS = {
    w.name: w
    for w in [
        TeacherWorkload("teacher_tiny", 1, 512, 256, 4096, 100, "fp32", 128, 2001),
        TeacherWorkload("teacher_llama8b_32k", 1, 32768, 4096, 128256, 100, "bf16", 2048, 2002),
        TeacherWorkload("teacher_gptoss120b_b4_32k", 4, 32768, 2880, 201088, 100, "bf16", 4096,
                        2003),
    ]
}


def make_teacher_inputs(w: TeacherWorkload, n_rows: int | None = None) -> dict:
    """Teacher hidden states [N, d] and teacher LM head [V, d] (fp32 arrays;
    bf16 workloads hold bf16-representable values)."""
    n = w.N if n_rows is None else n_rows
    if w.values == "integer":
        h = _rng(w.seed, 4).integers(-2, 3, size=(n, w.d)).astype(np.float32)
        W = _rng(w.seed, 5).integers(-2, 3, size=(w.V, w.d)).astype(np.float32)
    else:
        h = _rng(w.seed, 4).standard_normal((n, w.d), dtype=np.float32)
        W = _rng(w.seed, 5).standard_normal((w.V, w.d), dtype=np.float32)
        W *= np.float32(1.0 / np.sqrt(w.d))
        if w.dtype == "bf16":
            h, W = round_to_bf16(h), round_to_bf16(W)
    return {"workload": w, "hidden": h, "weight": W, "K": w.K, "chunk": w.chunk,
            "dtype": w.dtype}


def small_teacher_workload(name="teacher_small", n=300, d=64, V=1000, K=100, dtype="fp32",
                           chunk=128, seed=9, values="normal") -> TeacherWorkload:
    """A custom (usually tiny) teacher workload with the same recipe."""
    return TeacherWorkload(name, 1, n, d, V, K, dtype, chunk, seed, values)

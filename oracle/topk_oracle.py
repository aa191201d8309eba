"""fp64 reference of the teacher top-K cache (the step before the loss).

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
imports this module and this module never imports the HIP library.

What is computed, and where it comes from
-----------------------------------------
The pages' first system change is offline distillation: the teacher is run
once over the data and, for every position, only its 100 most probable
tokens are stored; the cache then replaces the teacher during student
training ("Эффективная дистилляция знаний ..." (malakhovai.ru), second
paragraph; "Multiverse Computing ... (iitak.ru)", third paragraph;
"Wissensdestillation mit deutlich weniger GPU-Speicher", section
"Teacher-Ausgaben einmalig zwischenspeichern", which says the 100 most
probable logits per token are stored).

The softmax at any temperature is increasing in the logit, so the K most
probable tokens are the K largest logits. Per row r:

    l_r     = h_r . W_store^T           (teacher LM head stored [V, d])
    topk_r  = the K ids with the largest l_rv, ordered by l_rv descending;
              among equal logits the lower id comes first
    values  = l_r at those ids

The tie rule and the order are readings (the pages do not say how ties are
broken or whether the cache is sorted); both make the output a unique
function of the logits.
"""

from __future__ import annotations

import numpy as np


def teacher_logits(hidden, w_store) -> np.ndarray:
    """l = hidden . W in fp64, with W given in its stored [V, d] layout."""
    return np.asarray(hidden, dtype=np.float64) @ np.asarray(w_store, dtype=np.float64).T


def topk_rows(logits, K: int):
    """Per row, the K largest entries ordered by value descending, ties by the
    lower column index first. Returns (ids int32 [R, K], values float64 [R, K]).

    np.lexsort sorts by its last key first: -value ascending (value
    descending), then the column index ascending among equal values.
    """
    z = np.asarray(logits, dtype=np.float64)
    R, V = z.shape
    if not 1 <= K <= V:
        raise ValueError(f"K must be in [1, {V}] (got {K})")
    cols = np.arange(V)
    ids = np.empty((R, K), dtype=np.int32)
    vals = np.empty((R, K), dtype=np.float64)
    for r in range(R):
        order = np.lexsort((cols, -z[r]))[:K]
        ids[r] = order
        vals[r] = z[r, order]
    return ids, vals


def teacher_topk(hidden, w_store, K: int):
    """The cached teacher entries: (ids int32 [N, K], logits float64 [N, K])."""
    return topk_rows(teacher_logits(hidden, w_store), K)

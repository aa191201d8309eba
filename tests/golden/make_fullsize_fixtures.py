#!/usr/bin/env python3
"""Write the oracle's expected values for the full-size workloads.

Calls only ``oracle`` (the fp64 definition of the loss) and the seeded input
generator ``sparse_top_kl_amd.synth``; nothing from the HIP library is
imported or run. For each full-size workload (and the loss options on the
32K-token workload) it runs ``oracle.forward_backward`` once over all rows
and stores, in ``tests/golden/fullsize_<case>.npz``:

  * ``lse`` and ``row_loss`` for every row, rounded to fp32 (relative
    rounding 6e-8, four orders below the 1e-3 loss tolerance), and the
    ``math.fsum`` total ``loss`` in fp64;
  * full rows of grad_W for four groups of vocabulary ids, each compared with
    its own largest magnitude by the GPU test: ``hot`` (the ids with the most
    (row, entry) pairs in the teacher cache), ``cold`` (ids with the fewest
    pairs, none where such ids exist: their gradient is the dense softmax
    term alone), ``tail`` (the last ids of the vocabulary: the ragged last
    tile) and ``random`` (uniform ids); rounded to fp32;
  * the workload's parameters and the generator version, which the test
    checks before comparing.

Per-row values that need only their own row (grad_hidden, the logits at the
teacher ids) are computed by the test itself from the oracle on sampled rows.

Usage: python tests/golden/make_fullsize_fixtures.py [case ...]
(at about 0.3 fp64 TFLOP/s the six cases take about an hour together).
"""

from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from sparse_top_kl_amd import synth  # noqa: E402

# case name -> (workload, with loss options)
CASES = {
    "llama3b_8k": ("llama3b_8k", False),
    "long32k": ("long32k", False),
    "gptoss20b_32k": ("gptoss20b_32k", False),
    "stress_b1_64k": ("stress_b1_64k", False),
    "stress_b4_32k": ("stress_b4_32k", False),
    "long32k-options": ("long32k", True),
}
N_HOT, N_COLD, N_TAIL, N_RANDOM = 12, 12, 4, 4
VOCAB_SEED = 20261203


def fixture_path(case: str) -> str:
    return os.path.join(HERE, f"fullsize_{case}.npz")


def vocab_groups(idx: np.ndarray, V: int) -> dict:
    """Vocabulary ids to check, chosen from the teacher cache's id counts."""
    count = np.bincount(idx.ravel(), minlength=V)
    order = np.argsort(-count, kind="stable")
    hot = np.sort(order[:N_HOT])
    rng = np.random.default_rng(VOCAB_SEED)
    least = count.min()
    pool = np.flatnonzero(count == least)
    if pool.size < N_COLD:
        pool = np.argsort(count, kind="stable")[:4 * N_COLD]
    cold = np.sort(rng.choice(pool, size=N_COLD, replace=False))
    tail = np.arange(V - N_TAIL, V)
    rand = np.sort(rng.choice(V, size=N_RANDOM, replace=False))
    return {"hot": hot, "cold": cold, "tail": tail, "random": rand,
            "hot_pairs": count[hot], "cold_pairs": count[cold]}


def make(case: str, block_rows: int = 512) -> str:
    name, with_options = CASES[case]
    w = synth.WORKLOADS[name]
    t0 = time.perf_counter()
    inp = synth.make_inputs(w)
    opts = synth.make_loss_options(w) if with_options else {}
    print(f"[{case}] inputs N={w.N} d={w.d} V={w.V} ({time.perf_counter() - t0:.0f} s)",
          flush=True)
    t1 = time.perf_counter()
    ref = oracle.forward_backward(inp["hidden"], inp["weight"], inp["topk_idx"],
                                  inp["topk_logit"], w.T, block_rows=block_rows, **opts)
    print(f"[{case}] oracle {time.perf_counter() - t1:.0f} s, loss {ref['loss']!r}", flush=True)
    groups = vocab_groups(inp["topk_idx"], w.V)
    out = {
        "case": np.array(case),
        "workload": np.array(name),
        "params": np.array([w.B, w.S, w.d, w.V, w.K, w.chunk, w.seed], dtype=np.int64),
        "T": np.float64(w.T),
        "dtype": np.array(w.dtype),
        "ids": np.array(w.ids),
        "generator_version": np.int64(synth.GENERATOR_VERSION),
        "options": np.bool_(with_options),
        "loss": np.float64(ref["loss"]),
        "lse": ref["lse"].astype(np.float32),
        "row_loss": ref["row_loss"].astype(np.float32),
    }
    for g in ("hot", "cold", "tail", "random"):
        out[f"vocab_{g}"] = groups[g].astype(np.int64)
        out[f"grad_w_{g}"] = ref["grad_w"][groups[g]].astype(np.float32)
    out["pairs_hot"] = groups["hot_pairs"]
    out["pairs_cold"] = groups["cold_pairs"]
    path = fixture_path(case)
    np.savez_compressed(path, **out)
    print(f"[{case}] wrote {path} ({os.path.getsize(path) / 1e6:.2f} MB, "
          f"{time.perf_counter() - t0:.0f} s total)", flush=True)
    return path


def main(argv):
    cases = argv or list(CASES)
    for c in cases:
        if c not in CASES:
            raise SystemExit(f"unknown case {c}; known: {', '.join(CASES)}")
    for c in cases:
        make(c)


if __name__ == "__main__":
    main(sys.argv[1:])

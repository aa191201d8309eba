"""The stored full-size oracle values (tests/golden/fullsize_*.npz) against
the oracle itself, on CPU: the fixtures were made for the current workload
parameters and input generator, a few rows recomputed here agree with them,
and the vocabulary groups are what their names say (hot ids carry the most
teacher-cache pairs, cold ids the fewest, tail ids end the vocabulary).
Full grad_W rows need every row of the batch, so only the per-row values are
recomputed here; the GPU test compares everything."""

from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from sparse_top_kl_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CASES = {"llama3b_8k": ("llama3b_8k", False), "long32k": ("long32k", False),
         "gptoss20b_32k": ("gptoss20b_32k", False), "stress_b1_64k": ("stress_b1_64k", False),
         "stress_b4_32k": ("stress_b4_32k", False), "long32k-options": ("long32k", True)}


def _load(case):
    path = os.path.join(GOLDEN, f"fullsize_{case}.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}: run tests/golden/make_fullsize_fixtures.py {case}")
    with np.load(path, allow_pickle=False) as f:
        return {k: f[k] for k in f.files}


@pytest.mark.parametrize("case", list(CASES))
def test_fixture_metadata_and_groups(case):
    name, options = CASES[case]
    w = synth.WORKLOADS[name]
    fx = _load(case)
    assert np.array_equal(fx["params"], [w.B, w.S, w.d, w.V, w.K, w.chunk, w.seed])
    assert float(fx["T"]) == w.T and int(fx["generator_version"]) == synth.GENERATOR_VERSION
    assert bool(fx["options"]) == options
    assert fx["lse"].shape == (w.N,) and fx["row_loss"].shape == (w.N,)
    assert np.isfinite(fx["lse"]).all() and np.isfinite(fx["row_loss"]).all()
    # per-row KL terms are >= 0; the stored total is their sum
    assert fx["row_loss"].min() >= -1e-6 * np.abs(fx["row_loss"]).max()
    assert abs(float(fx["loss"]) - fx["row_loss"].astype(np.float64).sum()) <= \
        1e-6 * abs(float(fx["loss"]))
    # lse is close to its statistical closed form ln V + |h|^2 / (2 d T^2) ~ ln V + 1/(2 T^2)
    assert abs(float(np.median(fx["lse"])) - (np.log(w.V) + 1 / (2 * w.T ** 2))) < 0.05
    assert fx["pairs_hot"].min() >= fx["pairs_cold"].max()
    assert np.array_equal(fx["vocab_tail"], np.arange(w.V - len(fx["vocab_tail"]), w.V))
    for g in ("hot", "cold", "tail", "random"):
        assert fx[f"grad_w_{g}"].shape == (len(fx[f"vocab_{g}"]), w.d)
        assert np.isfinite(fx[f"grad_w_{g}"]).all()
    if w.ids == "zipf":  # cold ids are in no row's top-K
        assert fx["pairs_cold"].max() == 0


@pytest.mark.slow
@pytest.mark.parametrize("case", ["llama3b_8k", "long32k-options"])
def test_fixture_rows_match_the_oracle(case):
    name, options = CASES[case]
    w = synth.WORKLOADS[name]
    fx = _load(case)
    inp = synth.make_inputs(w)
    opts = synth.make_loss_options(w) if options else {}
    rows = np.array([0, 1, w.chunk, w.N // 2, w.N - 1])
    sub = {k: v[rows] for k, v in opts.items() if k != "alpha"}
    if options:
        sub["alpha"] = opts["alpha"]
    ref = oracle.forward_backward(inp["hidden"][rows], inp["weight"], inp["topk_idx"][rows],
                                  inp["topk_logit"][rows], w.T, want_grads=False, **sub)
    np.testing.assert_allclose(fx["lse"][rows], ref["lse"], rtol=1e-7)
    np.testing.assert_allclose(fx["row_loss"][rows], ref["row_loss"], rtol=1e-6, atol=1e-6)

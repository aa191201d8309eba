"""The seeded input generator: recipe, reproducibility and distributions."""

import numpy as np
import pytest
import torch

from sparse_top_kl_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000)).astype(np.float32)
    # include exact ties
    x[:4] = np.array([1.00390625, 1.01171875, -1.00390625, 3.0], np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(synth.round_to_bf16(x), ref)


@pytest.mark.parametrize("ids", ["uniform", "zipf"])
def test_ids_distinct_in_range_and_reproducible(ids):
    w = synth.small_workload(n=2000, d=8, V=5000, K=100, ids=ids, seed=11)
    idx, logit = synth.make_teacher(w)
    assert idx.dtype == np.int32 and idx.shape == (2000, 100)
    assert idx.min() >= 0 and idx.max() < 5000
    s = np.sort(idx, axis=1)
    assert np.all(s[:, 1:] != s[:, :-1])
    idx2, logit2 = synth.make_teacher(w)
    np.testing.assert_array_equal(idx, idx2)
    np.testing.assert_array_equal(logit, logit2)


def test_teacher_logits_sorted_descending_gumbel_plus_3():
    w = synth.small_workload(n=4000, d=8, V=1000, K=100, seed=12)
    _, logit = synth.make_teacher(w)
    assert logit.dtype == np.float32
    assert np.all(np.diff(logit, axis=1) <= 0)
    # mean of Gumbel(0,1) is the Euler-Mascheroni constant
    assert abs(logit.mean() - (3.0 + 0.5772156649)) < 0.01


def test_zipf_head_frequency():
    """P(id 0) for the first draw is 1 / H_{V,1.1}; the first column is draw 1."""
    V = 128256
    w = synth.small_workload(n=20000, d=8, V=V, K=100, ids="zipf", seed=13)
    idx, _ = synth.make_teacher(w)
    p0 = 1.0 / np.sum(np.arange(1, V + 1, dtype=np.float64) ** -1.1)
    freq = np.mean(idx[:, 0] == 0)
    assert abs(freq - p0) < 5 * np.sqrt(p0 * (1 - p0) / 20000)
    # id 0 appears in most rows once 100 distinct draws are made
    assert np.mean((idx == 0).any(axis=1)) > 0.9


def test_hidden_and_weight_recipe():
    w = synth.small_workload(n=512, d=256, V=4096, K=10, dtype="bf16", seed=14)
    h = synth.make_hidden(w)
    W = synth.make_weight(w)
    np.testing.assert_array_equal(h, synth.round_to_bf16(h))
    np.testing.assert_array_equal(W, synth.round_to_bf16(W))
    assert abs(h.std() - 1.0) < 0.01
    assert abs(W.std() * np.sqrt(256) - 1.0) < 0.01
    np.testing.assert_array_equal(h, synth.make_hidden(w))


def test_workloads_have_the_stated_shapes():
    W = synth.WORKLOADS
    assert W["tiny"].N == 512 and W["tiny"].dtype == "fp32" and W["tiny"].chunk == 128
    assert (W["llama3b_8k"].N, W["llama3b_8k"].d, W["llama3b_8k"].V) == (8192, 3072, 128256)
    assert W["long32k"].T == 2.0 and W["long32k"].ids == "zipf"
    assert (W["gptoss20b_32k"].d, W["gptoss20b_32k"].V) == (2880, 201088)
    assert W["stress_b4_32k"].N == 131072 and W["stress_b1_64k"].N == 65536


def test_teacher_workloads_and_recipe():
    w = synth.TEACHER_WORKLOADS["teacher_llama8b_32k"]
    assert (w.N, w.d, w.V, w.K, w.dtype) == (32768, 4096, 128256, 100, "bf16")
    w = synth.TEACHER_WORKLOADS["teacher_gptoss120b_b4_32k"]
    assert (w.N, w.d, w.V) == (131072, 2880, 201088)
    small = synth.small_teacher_workload(n=40, d=32, V=300, dtype="bf16")
    a = synth.make_teacher_inputs(small)
    b = synth.make_teacher_inputs(small)
    assert a["hidden"].shape == (40, 32) and a["weight"].shape == (300, 32)
    np.testing.assert_array_equal(a["weight"], b["weight"])          # seeded
    np.testing.assert_array_equal(synth.round_to_bf16(a["hidden"]), a["hidden"])
    ints = synth.make_teacher_inputs(synth.small_teacher_workload(n=40, d=32, V=300,
                                                                  values="integer"))
    assert set(np.unique(ints["hidden"])) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
    assert set(np.unique(ints["weight"])) <= {-2.0, -1.0, 0.0, 1.0, 2.0}

"""Pins of the teacher top-K oracle against things other than itself: a
hand-worked example, pure-Python sorting, heapq, the softmax order, ties,
K = V and vocabulary permutations."""

import heapq

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def test_hand_worked_example():
    # logits row 0 = [1, 2, 3, 3], row 1 = [0, -1, -1, -2] (worked out by hand)
    hidden = np.array([[1.0, 2.0], [0.0, -1.0]])
    w = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-1.0, 2.0]])
    np.testing.assert_array_equal(oracle.teacher_logits(hidden, w),
                                  [[1, 2, 3, 3], [0, -1, -1, -2]])
    ids, vals = oracle.teacher_topk(hidden, w, 3)
    np.testing.assert_array_equal(ids, [[2, 3, 1], [0, 1, 2]])   # equal 3s: id 2 before 3
    np.testing.assert_array_equal(vals, [[3, 3, 2], [0, -1, -1]])


def _python_topk(row, K):
    pairs = sorted(((-float(v), i) for i, v in enumerate(row)))[:K]
    return [i for _, i in pairs], [-v for v, _ in pairs]


@pytest.mark.parametrize("seed", range(5))
def test_matches_pure_python_sort_with_ties(seed):
    rng = np.random.default_rng(seed)
    z = rng.integers(-4, 5, size=(7, 40)).astype(np.float64)  # many equal values
    for K in (1, 5, 17, 40):
        ids, vals = oracle.topk_rows(z, K)
        for r in range(z.shape[0]):
            pi, pv = _python_topk(z[r], K)
            assert ids[r].tolist() == pi
            assert vals[r].tolist() == pv


def test_matches_heapq_nlargest():
    rng = np.random.default_rng(11)
    z = np.round(rng.normal(size=(5, 300)), 1)   # rounding creates ties
    ids, _ = oracle.topk_rows(z, 25)
    for r in range(5):
        best = heapq.nlargest(25, range(300), key=lambda i: (z[r, i], -i))
        assert ids[r].tolist() == best


def test_most_probable_tokens_at_any_temperature():
    """Distinct logits: the K largest logits are the K most probable tokens of
    the teacher softmax, at every temperature, in the same order."""
    rng = np.random.default_rng(3)
    hidden = rng.normal(size=(4, 16))
    w = rng.normal(size=(200, 16))
    ids, _ = oracle.teacher_topk(hidden, w, 12)
    z = hidden @ w.T
    for T in (0.5, 1.0, 3.0):
        p = softmax(z / T, axis=1)
        np.testing.assert_array_equal(ids, np.argsort(-p, axis=1, kind="stable")[:, :12])


def test_all_equal_logits_give_the_lowest_ids():
    ids, vals = oracle.teacher_topk(np.ones((3, 8)), np.zeros((50, 8)), 10)
    np.testing.assert_array_equal(ids, np.tile(np.arange(10), (3, 1)))
    assert np.all(vals == 0.0)


def test_k_equal_v_is_a_sorted_permutation():
    rng = np.random.default_rng(5)
    z = rng.normal(size=(3, 64))
    ids, vals = oracle.topk_rows(z, 64)
    for r in range(3):
        assert sorted(ids[r].tolist()) == list(range(64))
        assert np.all(np.diff(vals[r]) <= 0)
        np.testing.assert_array_equal(vals[r], z[r, ids[r]])


def test_vocabulary_permutation_maps_the_ids():
    rng = np.random.default_rng(8)
    hidden = rng.normal(size=(6, 10))
    w = rng.normal(size=(120, 10))
    perm = rng.permutation(120)          # new row j holds old row perm[j]
    ids, vals = oracle.teacher_topk(hidden, w, 30)
    ids_p, vals_p = oracle.teacher_topk(hidden, w[perm], 30)
    np.testing.assert_array_equal(perm[ids_p], ids)
    np.testing.assert_allclose(vals_p, vals, rtol=0, atol=1e-12)


def test_rejects_k_out_of_range():
    with pytest.raises(ValueError):
        oracle.topk_rows(np.zeros((2, 5)), 6)
    with pytest.raises(ValueError):
        oracle.topk_rows(np.zeros((2, 5)), 0)

"""Pins of the fp64 oracle against things other than itself.

Library routines (scipy logsumexp, torch kl_div / cross_entropy / autograd),
closed forms, a hand-derived worked example, central finite differences,
pure-Python brute force, and invariants of the definition (KL >= 0, teacher
shift/permutation invariance, the temperature-scaling identity, zero column
sums of grad_W). Each is chosen so that a plausible slip in the oracle (a
dropped T factor, a wrong sign, a transposed weight, an index off by one)
fails at least one of them; ``test_planted_mistakes_are_caught`` checks that
claim on mutated copies of the oracle.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import kl_oracle
from sparse_top_kl_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(seed, n=5, d=6, v=13, k=4, dup=False, scale=1.0):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((n, d))
    w = rng.standard_normal((v, d)) * scale / math.sqrt(d)
    if dup:
        idx = rng.integers(0, v, size=(n, k))
    else:
        idx = np.stack([rng.permutation(v)[:k] for _ in range(n)])
    logit = rng.gumbel(size=(n, k)) + 3.0
    return h, w, idx.astype(np.int32), logit


def _run(*args, **kw):
    return oracle.forward_backward(*args, **kw)


# ---------------------------------------------------------------- library pins

def test_logsumexp_matches_scipy():
    rng = np.random.default_rng(0)
    u = rng.standard_normal((7, 33)) * 30.0
    np.testing.assert_allclose(oracle.logsumexp_rows(u),
                               scipy.special.logsumexp(u, axis=1), rtol=1e-14)


def test_lse_matches_torch_logsumexp():
    h, w, idx, logit = _rand_problem(1, n=6, d=8, v=40, k=5)
    T = 1.7
    out = _run(h, w, idx, logit, T)
    ref = torch.logsumexp(torch.from_numpy(h) @ torch.from_numpy(w).T / T, dim=1)
    np.testing.assert_allclose(out["lse"], ref.numpy(), rtol=1e-13)


@pytest.mark.parametrize("T", [1.0, 2.0, 0.7])
def test_full_vocab_teacher_equals_torch_kl_div(T):
    """K = V (ids a permutation): the loss is T^2 KL(softmax(l/T) || softmax(z/T))."""
    rng = np.random.default_rng(3)
    n, d, v = 4, 5, 9
    h = rng.standard_normal((n, d))
    w = rng.standard_normal((v, d))
    idx = np.stack([rng.permutation(v) for _ in range(n)]).astype(np.int32)
    logit = rng.standard_normal((n, v)) * 2.0
    out = _run(h, w, idx, logit, T)
    z = torch.from_numpy(h) @ torch.from_numpy(w).T
    dense_teacher = torch.empty(n, v, dtype=torch.float64)
    dense_teacher.scatter_(1, torch.from_numpy(idx).long(), torch.from_numpy(logit))
    ref = torch.nn.functional.kl_div(torch.log_softmax(z / T, 1),
                                     torch.log_softmax(dense_teacher / T, 1),
                                     log_target=True, reduction="sum") * T * T
    assert out["loss"] == pytest.approx(ref.item(), rel=1e-12)


@pytest.mark.parametrize("T", [1.0, 3.0])
def test_single_entry_teacher_equals_cross_entropy(T):
    """K = 1: p_t is one-hot, so the loss is T^2 times cross entropy at T."""
    rng = np.random.default_rng(4)
    n, d, v = 6, 7, 21
    h = rng.standard_normal((n, d))
    w = rng.standard_normal((v, d))
    idx = rng.integers(0, v, size=(n, 1)).astype(np.int32)
    logit = rng.standard_normal((n, 1))
    out = _run(h, w, idx, logit, T)
    z = torch.from_numpy(h) @ torch.from_numpy(w).T
    ref = torch.nn.functional.cross_entropy(z / T, torch.from_numpy(idx[:, 0]).long(),
                                            reduction="sum") * T * T
    assert out["loss"] == pytest.approx(ref.item(), rel=1e-12)


def test_gradients_match_torch_autograd():
    """Autograd of the dense KL written with library log_softmax."""
    h, w, idx, logit = _rand_problem(5, n=5, d=6, v=17, k=6)
    T, s = 1.3, 0.37
    out = _run(h, w, idx, logit, T, grad_scale=s)
    H = torch.tensor(h, requires_grad=True)
    W = torch.tensor(w, requires_grad=True)
    ls = torch.log_softmax(H @ W.T / T, dim=1)
    lp = torch.log_softmax(torch.from_numpy(logit) / T, dim=1)
    loss = (lp.exp() * (lp - ls.gather(1, torch.from_numpy(idx).long()))).sum() * T * T
    (loss * s).backward()
    np.testing.assert_allclose(out["grad_hidden"], H.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(out["grad_w"], W.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-12)


# ---------------------------------------------------------------- closed forms

def test_two_token_worked_example():
    with open(os.path.join(GOLDEN, "two_token_worked_example.json")) as f:
        g = json.load(f)
    out = _run(np.array(g["hidden"]), np.array(g["w_store"]), np.array(g["topk_idx"]),
               np.array(g["topk_logit"]), g["T"])
    e = g["expected"]
    assert out["loss"] == pytest.approx(0.5 * math.log(4.0 / 3.0), rel=1e-14)
    assert out["loss"] == pytest.approx(e["loss"], rel=1e-14)
    assert out["lse"][0] == pytest.approx(e["lse"], rel=1e-14)
    np.testing.assert_allclose(out["grad_hidden"], e["grad_hidden"], rtol=1e-14)
    np.testing.assert_allclose(out["grad_w"], e["grad_w"], rtol=1e-14, atol=1e-15)


def test_two_token_worked_example_at_T2():
    """Same example at T=2, derived by hand: z/T = [ln(3)/2, 0]."""
    r3 = math.sqrt(3.0)
    ps = [r3 / (r3 + 1.0), 1.0 / (r3 + 1.0)]
    kl = 0.5 * math.log(0.5 / ps[0]) + 0.5 * math.log(0.5 / ps[1])
    out = _run(np.array([[1.0]]), np.array([[math.log(3.0)], [0.0]]),
               np.array([[0, 1]]), np.array([[0.0, 0.0]]), 2.0)
    assert out["loss"] == pytest.approx(4.0 * kl, rel=1e-14)
    # G = T (q - p), grad_h = G . W
    G = [2.0 * (ps[0] - 0.5), 2.0 * (ps[1] - 0.5)]
    assert out["grad_hidden"][0, 0] == pytest.approx(G[0] * math.log(3.0), rel=1e-13)
    np.testing.assert_allclose(out["grad_w"][:, 0], G, rtol=1e-13)


@pytest.mark.parametrize("T", [1.0, 2.0])
def test_uniform_student_and_teacher_closed_form(T):
    """W = 0 and equal teacher logits: loss = N T^2 log(V/K), lse = log V,
    grad_hidden = 0, grad_W = s T H^T (1/V - P) with P = 1/K at the ids."""
    rng = np.random.default_rng(6)
    n, d, v, k, s = 5, 4, 50, 10, 0.6
    h = rng.standard_normal((n, d))
    w = np.zeros((v, d))
    idx = np.stack([rng.permutation(v)[:k] for _ in range(n)]).astype(np.int32)
    logit = np.full((n, k), 1.25)
    out = _run(h, w, idx, logit, T, grad_scale=s)
    assert out["loss"] == pytest.approx(n * T * T * math.log(v / k), rel=1e-13)
    np.testing.assert_allclose(out["lse"], math.log(v) / 1.0, rtol=1e-14)
    np.testing.assert_allclose(out["grad_hidden"], 0.0, atol=1e-15)
    expect = np.zeros((v, d))
    for r in range(n):
        for c in range(v):
            g = s * T * (1.0 / v - (1.0 / k if c in idx[r] else 0.0))
            expect[c] += g * h[r]
    np.testing.assert_allclose(out["grad_w"], expect, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- brute force / FD

@pytest.mark.parametrize("dup", [False, True])
def test_vectorised_matches_brute_force(dup):
    h, w, idx, logit = _rand_problem(7, n=4, d=5, v=11, k=4, dup=dup)
    logit[1, 2] = -np.inf
    T, s = 1.9, 1.4
    out = _run(h, w, idx, logit, T, grad_scale=s, block_rows=3)
    bf = oracle.brute_force(h, w, idx, logit, T, grad_scale=s)
    assert out["loss"] == pytest.approx(bf["loss"], rel=1e-12)
    for key in ["row_loss", "lse", "grad_hidden", "grad_w"]:
        np.testing.assert_allclose(out[key], bf[key], rtol=1e-11, atol=1e-13)


def _fd_grad(f, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("T", [1.0, 2.0])
def test_gradients_match_finite_differences(T):
    h, w, idx, logit = _rand_problem(8, n=3, d=4, v=9, k=5)
    s = 0.8
    out = _run(h, w, idx, logit, T, grad_scale=s)

    def f():
        return s * _run(h, w, idx, logit, T, want_grads=False)["loss"]

    gh = _fd_grad(f, h)
    gw = _fd_grad(f, w)
    np.testing.assert_allclose(out["grad_hidden"], gh, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(out["grad_w"], gw, rtol=1e-6, atol=1e-8)


# ---------------------------------------------------------------- invariants

def test_kl_is_nonnegative_per_row():
    h, w, idx, logit = _rand_problem(9, n=64, d=16, v=300, k=100, scale=3.0)
    out = _run(h, w, idx, logit, 1.0)
    assert np.all(out["row_loss"] >= -1e-12)


def test_block_size_invariance():
    """Splitting rows into blocks (the chunking) does not change the result."""
    h, w, idx, logit = _rand_problem(10, n=23, d=8, v=60, k=7)
    ref = _run(h, w, idx, logit, 1.5, block_rows=1)
    for b in (4, 7, 64):
        out = _run(h, w, idx, logit, 1.5, block_rows=b)
        assert out["loss"] == pytest.approx(ref["loss"], rel=1e-13)
        for key in ["row_loss", "lse", "grad_hidden", "grad_w"]:
            np.testing.assert_allclose(out[key], ref[key], rtol=1e-12, atol=1e-14)


def test_teacher_shift_and_pair_permutation_invariance():
    h, w, idx, logit = _rand_problem(11, n=6, d=5, v=30, k=8)
    ref = _run(h, w, idx, logit, 1.0)
    shifted = _run(h, w, idx, logit + 3.0, 1.0)
    perm = np.random.default_rng(0).permutation(8)
    permuted = _run(h, w, idx[:, perm], logit[:, perm], 1.0)
    for out in (shifted, permuted):
        assert out["loss"] == pytest.approx(ref["loss"], rel=1e-12)
        np.testing.assert_allclose(out["grad_hidden"], ref["grad_hidden"], rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(out["grad_w"], ref["grad_w"], rtol=1e-11, atol=1e-14)


def test_id_shift_is_a_negative_control():
    """Moving one id by +1 must change that row's loss by far more than tolerance."""
    h, w, idx, logit = _rand_problem(12, n=4, d=8, v=40, k=5)
    ref = _run(h, w, idx, logit, 1.0)
    idx2 = idx.copy()
    idx2[2, 0] = (idx2[2, 0] + 1) % 40
    if idx2[2, 0] in idx2[2, 1:]:
        idx2[2, 0] = (idx2[2, 0] + 1) % 40
    out = _run(h, w, idx2, logit, 1.0)
    assert abs(out["row_loss"][2] - ref["row_loss"][2]) > 1e-3 * abs(ref["row_loss"][2])
    np.testing.assert_allclose(out["row_loss"][[0, 1, 3]], ref["row_loss"][[0, 1, 3]], rtol=1e-14)


def test_minus_inf_teacher_entries_equal_dropping_them():
    h, w, idx, logit = _rand_problem(13, n=3, d=5, v=20, k=6)
    logit2 = logit.copy()
    logit2[:, 4:] = -np.inf
    out = _run(h, w, idx, logit2, 1.3)
    ref = _run(h, w, idx[:, :4], logit[:, :4], 1.3)
    assert np.isfinite(out["loss"])
    assert out["loss"] == pytest.approx(ref["loss"], rel=1e-13)
    np.testing.assert_allclose(out["grad_w"], ref["grad_w"], rtol=1e-12, atol=1e-14)


def test_temperature_scaling_identity():
    """L(H, W, l; T) = T^2 L(H, W/T, l/T; 1); grad_H scales by T^2, grad_W by T."""
    h, w, idx, logit = _rand_problem(14, n=5, d=6, v=25, k=7)
    T = 2.0
    a = _run(h, w, idx, logit, T)
    b = _run(h, w / T, idx, logit / T, 1.0)
    assert a["loss"] == pytest.approx(T * T * b["loss"], rel=1e-12)
    np.testing.assert_allclose(a["grad_hidden"], T * T * b["grad_hidden"], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(a["grad_w"], T * b["grad_w"], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=1e-13)


def test_grad_w_column_sums_vanish():
    """sum_v G_rv = 0 when the teacher sums to one, so sum_v grad_W[v, :] = 0."""
    h, w, idx, logit = _rand_problem(15, n=9, d=7, v=50, k=10)
    out = _run(h, w, idx, logit, 1.0)
    assert np.abs(out["grad_w"].sum(axis=0)).max() < 1e-13 * np.abs(out["grad_w"]).max() * 50


def test_lse_statistical_closed_form():
    """For W ~ N(0, 1/d): lse_r ~= log V + |h_r|^2 / (2 d T^2) within a few sd."""
    w = synth.small_workload(n=64, d=256, V=20000, K=10, T=1.0, seed=3)
    inp = synth.make_inputs(w)
    out = _run(inp["hidden"], inp["weight"], inp["topk_idx"], inp["topk_logit"], 1.0,
               want_grads=False)
    hn = (inp["hidden"].astype(np.float64) ** 2).sum(1)
    pred = math.log(w.V) + hn / (2 * w.d)
    sigma2 = hn / w.d
    sd = np.sqrt((np.exp(sigma2) - 1) / w.V)
    assert np.all(np.abs(out["lse"] - pred) < 8 * sd + 1e-3)


# ---------------------------------------------------------------- mutation check

def _mutants():
    """Plausible slips, each a patched copy of the oracle's row computation."""
    base = kl_oracle.forward_backward

    def dropped_t2(*a, **k):
        out = base(*a, **k)
        T = a[4]
        out = dict(out)
        out["loss"] /= T * T
        return out

    def transposed_weight_grad(*a, **k):
        out = dict(base(*a, **k))
        if "grad_w" in out:
            gw = out["grad_w"]
            out["grad_w"] = gw[::-1].copy()
        return out

    def wrong_sign_grad(*a, **k):
        out = dict(base(*a, **k))
        if "grad_hidden" in out:
            out["grad_hidden"] = -out["grad_hidden"]
        return out

    def student_renormalised_over_k(h, w, idx, logit, T, grad_scale=1.0, want_grads=True,
                                    block_rows=128):
        hh = np.asarray(h, np.float64)
        z = hh @ np.asarray(w, np.float64).T
        zk = np.take_along_axis(z, np.asarray(idx), 1) / T
        out = dict(base(h, w, idx, logit, T, grad_scale, want_grads, block_rows))
        lp, p = kl_oracle.teacher_log_probs(logit, T)
        lsk = zk - scipy.special.logsumexp(zk, axis=1, keepdims=True)
        out["row_loss"] = T * T * (p * (lp - lsk)).sum(1)
        out["loss"] = float(out["row_loss"].sum())
        return out

    def id_off_by_one(h, w, idx, logit, T, **k):
        v = np.asarray(w).shape[0]
        return base(h, w, (np.asarray(idx) + 1) % v, logit, T, **k)

    return [dropped_t2, transposed_weight_grad, wrong_sign_grad,
            student_renormalised_over_k, id_off_by_one]


def _pin_suite(fb):
    """A subset of the pins above, as booleans, for a candidate oracle ``fb``."""
    ok = []
    # kl_div pin at T = 2
    rng = np.random.default_rng(3)
    n, d, v = 4, 5, 9
    h = rng.standard_normal((n, d))
    w = rng.standard_normal((v, d))
    idx = np.stack([rng.permutation(v) for _ in range(n)]).astype(np.int32)
    logit = rng.standard_normal((n, v)) * 2.0
    T = 2.0
    out = fb(h, w, idx, logit, T)
    z = torch.from_numpy(h) @ torch.from_numpy(w).T
    dense = torch.empty(n, v, dtype=torch.float64)
    dense.scatter_(1, torch.from_numpy(idx).long(), torch.from_numpy(logit))
    ref = torch.nn.functional.kl_div(torch.log_softmax(z / T, 1), torch.log_softmax(dense / T, 1),
                                     log_target=True, reduction="sum") * T * T
    ok.append(math.isclose(out["loss"], ref.item(), rel_tol=1e-10))
    # finite differences at T = 1.5 on a K < V problem
    h, w, idx, logit = _rand_problem(8, n=3, d=4, v=9, k=5)
    out = fb(h, w, idx, logit, 1.5)

    def f():
        return fb(h, w, idx, logit, 1.5, want_grads=False)["loss"]

    ok.append(np.allclose(out["grad_hidden"], _fd_grad(f, h), rtol=1e-5, atol=1e-7))
    ok.append(np.allclose(out["grad_w"], _fd_grad(f, w), rtol=1e-5, atol=1e-7))
    # brute force
    bf = oracle.brute_force(h, w, idx, logit, 1.5)
    ok.append(math.isclose(out["loss"], bf["loss"], rel_tol=1e-10))
    return ok


def test_pins_accept_the_oracle():
    assert all(_pin_suite(kl_oracle.forward_backward))


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_mistakes_are_caught(mutant):
    assert not all(_pin_suite(mutant))


# ------------------------------------------- options: row weights, hard labels

def _labels(seed, n, v, ignore=()):
    y = np.random.default_rng(seed).integers(0, v, size=n).astype(np.int32)
    for r in ignore:
        y[r] = -1
    return y


@pytest.mark.parametrize("T", [1.0, 2.5])
def test_pure_hard_label_term_equals_torch_cross_entropy(T):
    """alpha = 0: only the cross-entropy at temperature 1 remains, whatever T."""
    h, w, idx, logit = _rand_problem(21, n=6, d=5, v=17, k=4)
    y = _labels(3, 6, 17)
    out = _run(h, w, idx, logit, T, labels=y, alpha=0.0)
    ht = torch.tensor(h, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    ref = torch.nn.functional.cross_entropy(ht @ wt.T, torch.tensor(y, dtype=torch.long),
                                            reduction="sum")
    ref.backward()
    assert out["loss"] == pytest.approx(ref.item(), rel=1e-12)
    np.testing.assert_allclose(out["grad_hidden"], ht.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["grad_w"], wt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["lse1"], torch.logsumexp(ht @ wt.T, 1).detach().numpy(),
                               rtol=1e-13)


@pytest.mark.parametrize("T", [1.0, 2.0])
def test_options_match_brute_force(T):
    h, w, idx, logit = _rand_problem(22, n=5, d=4, v=11, k=4, dup=True)
    wr = np.array([1.0, 0.0, 0.25, 2.0, 1.0])
    y = _labels(4, 5, 11, ignore=(3,))
    kw = dict(row_weight=wr, labels=y, alpha=0.3, grad_scale=-0.7)
    out = _run(h, w, idx, logit, T, **kw)
    bf = kl_oracle.brute_force(h, w, idx, logit, T, **kw)
    assert out["loss"] == pytest.approx(bf["loss"], rel=1e-12)
    for key in ("row_loss", "grad_hidden", "grad_w"):
        np.testing.assert_allclose(out[key], bf[key], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("T", [1.0, 3.0])
def test_option_gradients_match_finite_differences(T):
    h, w, idx, logit = _rand_problem(23, n=3, d=4, v=9, k=5)
    kw = dict(row_weight=np.array([0.5, 1.5, 1.0]), labels=_labels(5, 3, 9), alpha=0.6)
    out = _run(h, w, idx, logit, T, **kw)

    def f():
        return _run(h, w, idx, logit, T, want_grads=False, **kw)["loss"]

    np.testing.assert_allclose(out["grad_hidden"], _fd_grad(f, h), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(out["grad_w"], _fd_grad(f, w), rtol=1e-6, atol=1e-8)


def test_zero_weight_rows_contribute_nothing_even_if_padding():
    h, w, idx, logit = _rand_problem(24, n=4, d=5, v=12, k=3)
    logit = logit.copy()
    logit[2, :] = -np.inf                      # a padding row: no teacher entry at all
    wr = np.array([1.0, 1.0, 0.0, 1.0])
    out = _run(h, w, idx, logit, 1.5, row_weight=wr, labels=np.array([1, 2, -1, 3]), alpha=0.5)
    assert out["row_loss"][2] == 0.0 and np.all(out["grad_hidden"][2] == 0.0)
    keep = [0, 1, 3]
    sub = _run(h[keep], w, idx[keep], logit[keep], 1.5, labels=np.array([1, 2, 3]), alpha=0.5)
    assert out["loss"] == pytest.approx(sub["loss"], rel=1e-13)
    np.testing.assert_allclose(out["grad_w"], sub["grad_w"], rtol=1e-12, atol=1e-15)


def test_weights_one_over_n_give_the_mean_and_neutral_options_change_nothing():
    h, w, idx, logit = _rand_problem(25, n=6, d=5, v=14, k=4)
    base = _run(h, w, idx, logit, 2.0)
    mean = _run(h, w, idx, logit, 2.0, row_weight=np.full(6, 1 / 6))
    assert mean["loss"] == pytest.approx(base["loss"] / 6, rel=1e-13)
    np.testing.assert_allclose(mean["grad_w"], base["grad_w"] / 6, rtol=1e-12)
    alpha_one = _run(h, w, idx, logit, 2.0, labels=_labels(6, 6, 14), alpha=1.0)
    no_labels = _run(h, w, idx, logit, 2.0, alpha=0.2)     # alpha ignored without labels
    for o in (alpha_one, no_labels):
        assert o["loss"] == pytest.approx(base["loss"], rel=1e-13)
        np.testing.assert_allclose(o["grad_hidden"], base["grad_hidden"], rtol=1e-12, atol=1e-15)


def _option_mutants():
    """Plausible slips in the options, each a wrapper around the oracle."""
    base = kl_oracle.forward_backward

    def swapped_mixture(h, w, idx, logit, T, labels=None, alpha=1.0, **k):
        return base(h, w, idx, logit, T, labels=labels,
                    alpha=(1.0 - alpha) if labels is not None else alpha, **k)

    def weights_on_loss_only(h, w, idx, logit, T, row_weight=None, **k):
        out = dict(base(h, w, idx, logit, T, row_weight=row_weight, **k))
        if k.get("want_grads", True):
            plain = base(h, w, idx, logit, T, **k)
            out["grad_hidden"], out["grad_w"] = plain["grad_hidden"], plain["grad_w"]
        return out

    def ce_at_temperature_t(h, w, idx, logit, T, labels=None, alpha=1.0, **k):
        out = dict(base(h, w, idx, logit, T, labels=labels, alpha=alpha, **k))
        if labels is not None:
            kl = base(h, w, idx, logit, T, want_grads=False)["loss"]
            ce_t = base(np.asarray(h) / T, w, idx, logit, 1.0, labels=labels, alpha=0.0,
                        want_grads=False)["loss"]
            out["loss"] = alpha * kl + (1.0 - alpha) * ce_t
        return out

    return [swapped_mixture, weights_on_loss_only, ce_at_temperature_t]


def _option_pin_suite(fb):
    ok = []
    h, w, idx, logit = _rand_problem(21, n=6, d=5, v=17, k=4)
    y = _labels(3, 6, 17)
    out = fb(h, w, idx, logit, 2.5, labels=y, alpha=0.0)
    ref = torch.nn.functional.cross_entropy(torch.tensor(h) @ torch.tensor(w).T,
                                            torch.tensor(y, dtype=torch.long), reduction="sum")
    ok.append(math.isclose(out["loss"], ref.item(), rel_tol=1e-10))
    h, w, idx, logit = _rand_problem(23, n=3, d=4, v=9, k=5)
    kw = dict(row_weight=np.array([0.5, 1.5, 1.0]), labels=_labels(5, 3, 9), alpha=0.6)
    out = fb(h, w, idx, logit, 3.0, **kw)

    def f():
        return fb(h, w, idx, logit, 3.0, want_grads=False, **kw)["loss"]

    ok.append(np.allclose(out["grad_hidden"], _fd_grad(f, h), rtol=1e-5, atol=1e-7))
    bf = oracle.brute_force(h, w, idx, logit, 3.0, **kw)
    ok.append(math.isclose(out["loss"], bf["loss"], rel_tol=1e-10))
    return ok


def test_option_pins_accept_the_oracle():
    assert all(_option_pin_suite(kl_oracle.forward_backward))


@pytest.mark.parametrize("mutant", _option_mutants(), ids=lambda f: f.__name__)
def test_planted_option_mistakes_are_caught(mutant):
    assert not all(_option_pin_suite(mutant))


# ------------------------------------------------------------- teacher tail

def _teacher_with_tail(seed, n=5, d=6, v=40, k=7, T=1.5):
    """A full teacher (V logits per row) cached as its top-K plus its lse at T."""
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((n, d))
    w = rng.standard_normal((v, d)) / math.sqrt(d)
    full = rng.standard_normal((n, v)) * 2.0
    idx = np.argsort(-full, axis=1)[:, :k].astype(np.int32)
    logit = np.take_along_axis(full, idx.astype(np.int64), axis=1)
    tlse = scipy.special.logsumexp(full / T, axis=1)
    return h, w, idx, logit, tlse, full


@pytest.mark.parametrize("T", [1.0, 2.0])
def test_tail_bucket_equals_scipy_relative_entropy(T):
    h, w, idx, logit, tlse, full = _teacher_with_tail(31, T=T)
    out = _run(h, w, idx, logit, T, teacher_lse=tlse)
    pt = scipy.special.softmax(full / T, axis=1)
    qs = scipy.special.softmax((h @ w.T) / T, axis=1)
    ii = idx.astype(np.int64)
    P = np.concatenate([np.take_along_axis(pt, ii, 1), 1 - np.take_along_axis(pt, ii, 1).sum(1,
                        keepdims=True)], axis=1)
    Q = np.concatenate([np.take_along_axis(qs, ii, 1), 1 - np.take_along_axis(qs, ii, 1).sum(1,
                        keepdims=True)], axis=1)
    ref = T * T * scipy.special.rel_entr(P, Q).sum(axis=1)
    np.testing.assert_allclose(out["row_loss"], ref, rtol=1e-10)


def test_tail_bucket_with_the_whole_vocabulary_is_the_full_kl():
    rng = np.random.default_rng(32)
    n, d, v, T = 4, 5, 9, 1.7
    h, w = rng.standard_normal((n, d)), rng.standard_normal((v, d))
    idx = np.stack([rng.permutation(v) for _ in range(n)]).astype(np.int32)
    logit = rng.standard_normal((n, v)) * 2.0
    tlse = scipy.special.logsumexp(logit / T, axis=1)
    out = _run(h, w, idx, logit, T, teacher_lse=tlse)
    z = torch.from_numpy(h) @ torch.from_numpy(w).T
    dense = torch.empty(n, v, dtype=torch.float64)
    dense.scatter_(1, torch.from_numpy(idx).long(), torch.from_numpy(logit))
    ref = torch.nn.functional.kl_div(torch.log_softmax(z / T, 1), torch.log_softmax(dense / T, 1),
                                     log_target=True, reduction="sum") * T * T
    assert out["loss"] == pytest.approx(ref.item(), rel=1e-10)


def test_tail_bucket_reduces_to_renormalised_when_the_cache_holds_all_mass():
    h, w, idx, logit = _rand_problem(33, n=5, d=6, v=15, k=5)
    T = 1.3
    tlse = scipy.special.logsumexp(logit / T, axis=1)      # "the top-K are everything"
    a = _run(h, w, idx, logit, T, teacher_lse=tlse)
    b = _run(h, w, idx, logit, T)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-12)
    np.testing.assert_allclose(a["grad_hidden"], b["grad_hidden"], rtol=1e-9, atol=1e-13)


@pytest.mark.parametrize("T", [1.0, 2.5])
def test_tail_bucket_gradients_and_brute_force(T):
    h, w, idx, logit, tlse, _ = _teacher_with_tail(34, n=3, d=4, v=11, k=4, T=T)
    kw = dict(teacher_lse=tlse, row_weight=np.array([1.0, 0.5, 2.0]),
              labels=np.array([3, -1, 7]), alpha=0.7, grad_scale=1.3)
    out = _run(h, w, idx, logit, T, **kw)
    bf = kl_oracle.brute_force(h, w, idx, logit, T, **kw)
    assert out["loss"] == pytest.approx(bf["loss"], rel=1e-12)
    np.testing.assert_allclose(out["grad_w"], bf["grad_w"], rtol=1e-10, atol=1e-13)

    def f():
        return 1.3 * _run(h, w, idx, logit, T, want_grads=False,
                          **{k: v for k, v in kw.items() if k != "grad_scale"})["loss"]

    np.testing.assert_allclose(out["grad_hidden"], _fd_grad(f, h), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(out["grad_w"], _fd_grad(f, w), rtol=1e-6, atol=1e-8)


def _tail_mutants():
    base = kl_oracle.forward_backward

    def tail_term_sign(h, w, idx, logit, T, teacher_lse=None, **k):
        out = dict(base(h, w, idx, logit, T, teacher_lse=teacher_lse, **k))
        if teacher_lse is not None:   # the tail bucket's term with the opposite sign
            z = np.asarray(h, np.float64) @ np.asarray(w, np.float64).T
            q = scipy.special.softmax(z / T, axis=1)
            S = np.take_along_axis(q, np.asarray(idx, np.int64), 1).sum(1)
            pk = np.exp(np.asarray(logit, np.float64) / T - np.asarray(teacher_lse)[:, None])
            pt = np.maximum(0.0, 1.0 - pk.sum(1))
            tail = np.where(pt > 0, pt * (np.log(np.where(pt > 0, pt, 1.0)) - np.log(1 - S)), 0.0)
            out["loss"] = out["loss"] - 2.0 * T * T * float(tail.sum())
        return out

    def no_tail_gradient(h, w, idx, logit, T, teacher_lse=None, **k):
        out = dict(base(h, w, idx, logit, T, teacher_lse=teacher_lse, **k))
        if teacher_lse is not None and k.get("want_grads", True):
            # gradients of the teacher-normalised KL without the tail bucket
            tl = np.asarray(logit, np.float64)
            z = np.asarray(h, np.float64) @ np.asarray(w, np.float64).T
            lse = scipy.special.logsumexp(z / T, axis=1, keepdims=True)
            q = np.exp(z / T - lse)
            p = np.exp(tl / T - np.asarray(teacher_lse)[:, None])
            P = np.zeros_like(q)
            np.put_along_axis(P, np.asarray(idx, np.int64), p, axis=1)
            G = k.get("grad_scale", 1.0) * T * (q * p.sum(1, keepdims=True) - P)
            out["grad_hidden"] = G @ np.asarray(w, np.float64)
        return out

    return [tail_term_sign, no_tail_gradient]


def _tail_pin_suite(fb):
    h, w, idx, logit, tlse, full = _teacher_with_tail(35, T=2.0)
    out = fb(h, w, idx, logit, 2.0, teacher_lse=tlse)
    pt = scipy.special.softmax(full / 2.0, axis=1)
    qs = scipy.special.softmax((h @ w.T) / 2.0, axis=1)
    ii = idx.astype(np.int64)
    P = np.concatenate([np.take_along_axis(pt, ii, 1), 1 - np.take_along_axis(pt, ii, 1).sum(1,
                        keepdims=True)], axis=1)
    Q = np.concatenate([np.take_along_axis(qs, ii, 1), 1 - np.take_along_axis(qs, ii, 1).sum(1,
                        keepdims=True)], axis=1)
    ok = [math.isclose(out["loss"], 4.0 * scipy.special.rel_entr(P, Q).sum(), rel_tol=1e-10)]

    def f():
        return fb(h, w, idx, logit, 2.0, teacher_lse=tlse, want_grads=False)["loss"]

    ok.append(np.allclose(out["grad_hidden"], _fd_grad(f, h), rtol=1e-5, atol=1e-7))
    return ok


def test_tail_pins_accept_the_oracle():
    assert all(_tail_pin_suite(kl_oracle.forward_backward))


@pytest.mark.parametrize("mutant", _tail_mutants(), ids=lambda f: f.__name__)
def test_planted_tail_mistakes_are_caught(mutant):
    assert not all(_tail_pin_suite(mutant))

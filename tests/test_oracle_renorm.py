"""Pins of the student-renormalised oracle (``oracle.renorm_oracle``) against
things other than itself: torch's kl_div / log_softmax / autograd on the
gathered logits, the main oracle when the cache holds the whole vocabulary
(both normalisations then coincide), pure-Python brute force, central finite
differences, closed forms (uniform student, K = 1), independence from the
weight rows of ids outside the cache, and the temperature-scaling identity.
``test_planted_renorm_mistakes_are_caught`` checks on mutated copies that a
plausible slip fails at least one of them."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import renorm_oracle


def _problem(seed, n=5, d=6, v=13, k=4, dup=False, pad=False):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((n, d))
    w = rng.standard_normal((v, d)) / math.sqrt(d)
    if dup:
        idx = rng.integers(0, v, size=(n, k))
    else:
        idx = np.stack([rng.permutation(v)[:k] for _ in range(n)])
    logit = rng.gumbel(size=(n, k)) + 3.0
    if pad:
        logit[0, -1] = -np.inf
        logit[2, 1:] = -np.inf
    return h, w, idx.astype(np.int32), logit


def _torch_loss(h, w, idx, logit, T, row_weight=None):
    """T^2 KL(softmax(l/T) || softmax(z_ids/T)) per row through torch, with the
    gradients from autograd (float64)."""
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    zk = (ht[:, None, :] * wt[torch.as_tensor(idx, dtype=torch.long)]).sum(-1)
    lt = torch.tensor(logit, dtype=torch.float64)
    rows = torch.nn.functional.kl_div(torch.log_softmax(zk / T, 1), torch.log_softmax(lt / T, 1),
                                      log_target=True, reduction="none").sum(1) * T * T
    if row_weight is not None:
        rows = rows * torch.tensor(row_weight, dtype=torch.float64)
    rows.sum().backward()
    return rows.detach().numpy(), ht.grad.numpy(), wt.grad.numpy()


def _fd_grad(f, x, eps=1e-6):
    g = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("T", [1.0, 2.0, 0.7])
def test_equals_torch_kl_div_and_autograd_on_the_gathered_logits(T):
    h, w, idx, logit = _problem(1)
    out = renorm_oracle.renorm_forward_backward(h, w, idx, logit, T)
    rows, gh, gw = _torch_loss(h, w, idx, logit, T)
    np.testing.assert_allclose(out["row_loss"], rows, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(out["grad_hidden"], gh, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(out["grad_w"], gw, rtol=1e-10, atol=1e-14)


def test_whole_vocabulary_cache_equals_the_full_vocabulary_loss():
    """With K = V (ids a permutation of the vocabulary) renormalising the
    student over the cache is normalising it over the vocabulary."""
    rng = np.random.default_rng(2)
    n, d, v, T = 4, 5, 9, 1.5
    h, w = rng.standard_normal((n, d)), rng.standard_normal((v, d))
    idx = np.stack([rng.permutation(v) for _ in range(n)]).astype(np.int32)
    logit = rng.standard_normal((n, v)) * 2.0
    a = renorm_oracle.renorm_forward_backward(h, w, idx, logit, T, grad_scale=0.6)
    b = oracle.forward_backward(h, w, idx, logit, T, grad_scale=0.6)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-12)
    for key in ("row_loss", "topk_z", "grad_hidden", "grad_w"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("dup,pad", [(False, False), (True, False), (False, True), (True, True)])
def test_vectorised_matches_brute_force(dup, pad):
    h, w, idx, logit = _problem(3, n=5, d=4, v=9, k=4, dup=dup, pad=pad)
    wr = np.array([1.0, 0.0, 0.5, 2.0, 1.0])
    kw = dict(grad_scale=-0.7, row_weight=wr)
    out = renorm_oracle.renorm_forward_backward(h, w, idx, logit, 1.7, **kw)
    bf = renorm_oracle.renorm_brute_force(h, w, idx, logit, 1.7, **kw)
    assert out["loss"] == pytest.approx(bf["loss"], rel=1e-12)
    for key in ("row_loss", "grad_hidden", "grad_w"):
        np.testing.assert_allclose(out[key], bf[key], rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("T", [1.0, 2.5])
def test_gradients_match_finite_differences(T):
    h, w, idx, logit = _problem(4, n=3, d=4, v=8, k=3, dup=True, pad=True)
    wr = np.array([0.5, 1.0, 2.0])

    def f():
        return renorm_oracle.renorm_forward_backward(h, w, idx, logit, T, row_weight=wr,
                                                     want_grads=False)["loss"]

    out = renorm_oracle.renorm_forward_backward(h, w, idx, logit, T, row_weight=wr)
    np.testing.assert_allclose(out["grad_hidden"], _fd_grad(f, h), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(out["grad_w"], _fd_grad(f, w), rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("T", [1.0, 3.0])
def test_uniform_student_closed_form(T):
    """W = 0: every cached logit is 0, so the student is uniform over the
    row's finite entries and loss = T^2 sum_r sum_k p log(p n_r)."""
    h, w, idx, logit = _problem(5, pad=True)
    w[:] = 0.0
    out = renorm_oracle.renorm_forward_backward(h, w, idx, logit, T)
    ref = 0.0
    for r in range(len(logit)):
        a = logit[r][np.isfinite(logit[r])] / T
        p = np.exp(a - a.max())
        p /= p.sum()
        ref += T * T * float(np.sum(p * np.log(p * len(a))))
    assert out["loss"] == pytest.approx(ref, rel=1e-12)
    # equal teacher logits as well: both uniform, nothing to learn
    out = renorm_oracle.renorm_forward_backward(h, w, idx, np.zeros_like(logit), T)
    assert abs(out["loss"]) < 1e-14 and np.abs(out["grad_hidden"]).max() < 1e-14


def test_a_single_cached_entry_gives_zero_loss_and_gradient():
    h, w, idx, logit = _problem(6, k=1)
    out = renorm_oracle.renorm_forward_backward(h, w, idx, logit, 2.0)
    assert out["loss"] == 0.0
    assert np.abs(out["grad_hidden"]).max() == 0.0 and np.abs(out["grad_w"]).max() == 0.0


def test_weight_rows_outside_the_cache_change_nothing():
    """Unlike the full-vocabulary loss, the renormalised one reads W only at
    the cached ids: other rows of W do not enter, and their gradient is 0."""
    h, w, idx, logit = _problem(7, n=4, v=30, k=5)
    out = renorm_oracle.renorm_forward_backward(h, w, idx, logit, 1.3)
    unused = np.setdiff1d(np.arange(30), idx.ravel())
    assert len(unused) > 5
    w2 = w.copy()
    w2[unused] = np.random.default_rng(8).standard_normal((len(unused), w.shape[1])) * 5.0
    out2 = renorm_oracle.renorm_forward_backward(h, w2, idx, logit, 1.3)
    assert out2["loss"] == out["loss"]
    np.testing.assert_array_equal(out2["grad_hidden"], out["grad_hidden"])
    assert np.all(out["grad_w"][unused] == 0.0)


def test_temperature_scaling_identity():
    """L(H, W, l; T) = T^2 L(H, W/T, l/T; 1); grad_H scales by T^2, grad_W by T."""
    h, w, idx, logit = _problem(9, dup=True)
    T = 2.0
    a = renorm_oracle.renorm_forward_backward(h, w, idx, logit, T)
    b = renorm_oracle.renorm_forward_backward(h, w / T, idx, logit / T, 1.0)
    assert a["loss"] == pytest.approx(T * T * b["loss"], rel=1e-12)
    np.testing.assert_allclose(a["grad_hidden"], T * T * b["grad_hidden"], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(a["grad_w"], T * b["grad_w"], rtol=1e-10, atol=1e-14)


def test_nonnegative_and_zero_weight_rows_with_padding_are_harmless():
    h, w, idx, logit = _problem(10, n=6, pad=True)
    logit[4, :] = -np.inf                 # a padding row, weight 0 below
    wr = np.array([1.0, 1.0, 1.0, 1.0, 0.0, 1.0])
    out = renorm_oracle.renorm_forward_backward(h, w, idx, logit, 1.0, row_weight=wr)
    assert np.all(out["row_loss"] >= 0.0)
    assert out["row_loss"][4] == 0.0 and np.all(out["grad_hidden"][4] == 0.0)
    with pytest.raises(ValueError):
        renorm_oracle.renorm_forward_backward(h, w, idx, logit, 1.0)


# ------------------------------------------------------------ planted mistakes

def _mutants():
    base = renorm_oracle.renorm_forward_backward

    def student_over_vocabulary(h, w, idx, logit, T, **k):
        """normalises the student over the whole vocabulary (the main loss)"""
        return oracle.forward_backward(h, w, idx, np.where(np.isfinite(logit), logit, -np.inf), T,
                                       grad_scale=k.get("grad_scale", 1.0),
                                       row_weight=k.get("row_weight"),
                                       want_grads=k.get("want_grads", True))

    def no_t_squared(h, w, idx, logit, T, **k):
        out = dict(base(h, w, idx, logit, T, **k))
        out["loss"] = out["loss"] / (T * T)
        out["row_loss"] = out["row_loss"] / (T * T)
        return out

    def gradient_sign(h, w, idx, logit, T, **k):
        out = dict(base(h, w, idx, logit, T, **k))
        if "grad_hidden" in out:
            out["grad_hidden"] = -out["grad_hidden"]
            out["grad_w"] = -out["grad_w"]
        return out

    def padding_in_student_normaliser(h, w, idx, logit, T, **k):
        """lets -inf teacher entries stay in the student's softmax"""
        lg = np.asarray(logit, np.float64)
        zk = np.einsum("nd,nkd->nk", np.asarray(h, np.float64), np.asarray(w, np.float64)[idx])
        out = dict(base(h, w, idx, logit, T, **k))
        extra = []
        wr = k.get("row_weight")
        for r in range(len(lg)):
            pad = ~np.isfinite(lg[r])
            if wr is not None and wr[r] == 0 or not pad.any() or pad.all():
                extra.append(0.0)
                continue
            u = zk[r] / T
            full = np.log(np.exp(u - u.max()).sum()) + u.max()
            part = np.log(np.exp(u[~pad] - u.max()).sum()) + u.max()
            extra.append(T * T * (full - part) * (1.0 if wr is None else wr[r]))
        out["row_loss"] = out["row_loss"] + np.array(extra)
        out["loss"] = math.fsum(out["row_loss"].tolist())
        return out

    def weights_not_in_gradient(h, w, idx, logit, T, **k):
        kk = dict(k)
        wr = kk.pop("row_weight", None)
        out = dict(base(h, w, idx, logit, T, row_weight=wr, **kk))
        if wr is not None and "grad_hidden" in out:
            g = base(h, w, idx, logit, T, **kk)
            out["grad_hidden"], out["grad_w"] = g["grad_hidden"], g["grad_w"]
        return out

    return [student_over_vocabulary, no_t_squared, gradient_sign, padding_in_student_normaliser,
            weights_not_in_gradient]


def _pin_suite(fb):
    ok = []
    h, w, idx, logit = _problem(11, n=4, v=30, k=5)
    out = fb(h, w, idx, logit, 2.0)
    rows, gh, gw = _torch_loss(h, w, idx, logit, 2.0)
    ok.append(np.allclose(out["row_loss"], rows, rtol=1e-10, atol=1e-14))
    unused = np.setdiff1d(np.arange(30), idx.ravel())
    w2 = w.copy()
    w2[unused] *= 7.0
    ok.append(fb(h, w2, idx, logit, 2.0)["loss"] == out["loss"])
    h, w, idx, logit = _problem(12, n=4, d=4, v=8, k=4, dup=True, pad=True)
    wr = np.array([0.5, 1.0, 2.0, 1.5])
    bf = renorm_oracle.renorm_brute_force(h, w, idx, logit, 1.5, row_weight=wr)
    out = fb(h, w, idx, logit, 1.5, row_weight=wr)
    ok.append(math.isclose(out["loss"], bf["loss"], rel_tol=1e-11))

    def f():
        return fb(h, w, idx, logit, 1.5, row_weight=wr, want_grads=False)["loss"]

    ok.append(np.allclose(out["grad_hidden"], _fd_grad(f, h), rtol=1e-5, atol=1e-7))
    return ok


def test_renorm_pins_accept_the_oracle():
    assert all(_pin_suite(renorm_oracle.renorm_forward_backward))


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_renorm_mistakes_are_caught(mutant):
    assert not all(_pin_suite(mutant))

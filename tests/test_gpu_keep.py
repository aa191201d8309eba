"""Forward-chunked variant (kept logits) against the fp64 oracle and against
the fused path, at sizes the oracle finishes in seconds.

The forward of the variant runs the same kernels as the fused forward plus a
store of the logits, so its loss, lse, per-row loss and gathered logits must be
bitwise equal to fkl_forward's. The kept logits are checked element by element
against the oracle's z (bf16: within one rounding to bf16 plus fp32
accumulation error; fp32: the loss tolerance), with exact zeros in the padding
columns. The gradients, formed from the kept (rounded) logits instead of a
recompute, must meet the same tolerances against the oracle as the fused path.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
from sparse_top_kl_amd import fkl, synth
from tests.gpu_helpers import TOL, announce, compare, upload

pytestmark = pytest.mark.gpu


def _run_keep(inp, grad_scale=None, with_topk_z=True):
    T, chunk = inp["T"], inp["chunk"]
    h, w, idx, lg = upload(inp)
    out, z = fkl.fkl_forward_keep(h, w, idx, lg, T, chunk)
    ref_out = fkl.fkl_forward(h, w, idx, lg, T, chunk)
    torch.cuda.synchronize()
    for name in ("loss", "lse", "row_loss", "topk_z"):
        a, b = getattr(out, name), getattr(ref_out, name)
        assert torch.equal(a, b), f"kept-logits forward differs from the fused forward in {name}"
    kept = z.double().cpu().numpy()
    g = None if grad_scale is None else torch.tensor(float(grad_scale), device=h.device)
    gh, gw = fkl.fkl_backward_keep(h, w, idx, lg, out.lse, T, z,
                                   topk_z=out.topk_z if with_topk_z else None, grad_loss=g)
    torch.cuda.synchronize()
    res = {
        "loss": out.loss.item(),
        "lse": out.lse.double().cpu().numpy(),
        "row_loss": out.row_loss.double().cpu().numpy(),
        "topk_z": out.topk_z.double().cpu().numpy(),
        "grad_hidden": gh.double().cpu().numpy(),
        "grad_w": gw.double().cpu().numpy(),
    }
    return res, kept


def _check_kept_logits(kept, inp):
    V = inp["weight"].shape[0]
    assert kept.shape == (inp["hidden"].shape[0], fkl.keep_pitch(V))
    assert np.all(kept[:, V:] == 0.0), "padding columns of the kept logits must be zero"
    z = oracle.student_logits(inp["hidden"], inp["weight"])
    err = np.abs(kept[:, :V] - z)
    if inp["dtype"] == "bf16":
        # one round-to-nearest to bf16 (half an ulp, 2^-9 relative) plus fp32 accumulation
        bound = 2.0 ** -8 * np.abs(z) + 1e-4
    else:
        bound = TOL["fp32"]["loss"] * np.maximum(np.abs(z), 1.0)
    worst = float((err / bound).max())
    print(f"    kept logits: max err / bound = {worst:.3f}", flush=True)
    assert worst <= 1.0


def _oracle(inp, grad_scale=1.0):
    return oracle.forward_backward(inp["hidden"], inp["weight"], inp["topk_idx"],
                                   inp["topk_logit"], inp["T"], grad_scale=grad_scale)


def test_keep_tiny_workload(gpu_device):
    """512 tokens, d=512, V=8192, K=100, fp32, chunk 128, T=1."""
    announce("keep: tiny fp32 workload")
    inp = synth.make_inputs("tiny")
    res, kept = _run_keep(inp)
    _check_kept_logits(kept, inp)
    compare(res, _oracle(inp), "fp32")


CASES = [
    # name, n, d, V, K, T, dtype, chunk, ids
    ("keep_ragged_bf16", 700, 264, 3001, 100, 1.5, "bf16", 300, "uniform"),
    ("keep_ragged_fp32", 700, 264, 3001, 100, 1.5, "fp32", 300, "uniform"),
    ("keep_zipf_T2_bf16", 600, 512, 5000, 100, 2.0, "bf16", 256, "zipf"),
    ("keep_small_vocab_bf16", 300, 64, 300, 100, 1.0, "bf16", 1000, "uniform"),
    ("keep_one_row_fp32", 1, 128, 1000, 7, 0.5, "fp32", 1, "uniform"),
    ("keep_k1_bf16", 257, 128, 2000, 1, 1.0, "bf16", 100, "uniform"),
    ("keep_wide_d_bf16", 300, 1032, 1500, 50, 1.0, "bf16", 128, "uniform"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_keep_parity_small_shapes(gpu_device, case):
    name, n, d, V, K, T, dtype, chunk, ids = case
    announce(f"{name}: n={n} d={d} V={V} K={K} T={T} {dtype} chunk={chunk} {ids}")
    w = synth.small_workload(name, n=n, d=d, V=V, K=K, T=T, dtype=dtype, chunk=chunk, ids=ids,
                             seed=zlib.crc32(name.encode()) % 1000)
    inp = synth.make_inputs(w)
    res, kept = _run_keep(inp)
    _check_kept_logits(kept, inp)
    compare(res, _oracle(inp), dtype)


def test_keep_upstream_scale_and_recomputed_ids(gpu_device):
    announce("keep: grad_loss = -0.37, topk_z recomputed in the backward")
    w = synth.small_workload("keep_scale", n=300, d=128, V=1200, K=100, T=1.0, dtype="bf16",
                             chunk=128)
    inp = synth.make_inputs(w)
    res, _ = _run_keep(inp, grad_scale=-0.37, with_topk_z=False)
    compare(res, _oracle(inp, grad_scale=-0.37), "bf16")


def test_keep_repeated_ids_and_minus_inf(gpu_device):
    announce("keep: repeated ids and -inf teacher entries, fp32")
    w = synth.small_workload("keep_dup", n=270, d=64, V=700, K=30, T=1.0, dtype="fp32", chunk=100)
    inp = synth.make_inputs(w)
    inp["topk_idx"][::2, 5] = inp["topk_idx"][::2, 4]
    inp["topk_logit"][::3, 20:] = -np.inf
    res, _ = _run_keep(inp)
    assert np.isfinite(res["loss"]) and np.all(np.isfinite(res["grad_w"]))
    compare(res, _oracle(inp), "fp32")


def test_keep_accumulates_grad_weight(gpu_device):
    announce("keep: FKL_FLAG_ACCUMULATE_GRAD_W")
    w = synth.small_workload("keep_acc", n=300, d=128, V=1100, K=20, T=1.0, dtype="fp32",
                             chunk=64)
    inp = synth.make_inputs(w)
    h, W, idx, lg = upload(inp)
    out, z = fkl.fkl_forward_keep(h, W, idx, lg, w.T, w.chunk)
    base = torch.randn(W.shape, generator=torch.Generator().manual_seed(3)).to(h.device)
    gw = base.clone()
    fkl.fkl_backward_keep(h, W, idx, lg, out.lse, w.T, z, topk_z=out.topk_z, grad_weight=gw,
                          accumulate=True)
    torch.cuda.synchronize()
    ref = _oracle(inp)
    got = gw.double().cpu().numpy() - base.double().cpu().numpy()
    err = np.abs(got - ref["grad_w"]).max() / np.abs(ref["grad_w"]).max()
    assert err <= TOL["fp32"]["grad"], err


def test_keep_empty_batch(gpu_device):
    announce("keep: N = 0")
    W = torch.randn(300, 64, device=gpu_device)
    h = torch.empty(0, 64, device=gpu_device)
    idx = torch.empty(0, 5, dtype=torch.int32, device=gpu_device)
    lg = torch.empty(0, 5, device=gpu_device)
    out, z = fkl.fkl_forward_keep(h, W, idx, lg, 1.0, 16)
    gh, gw = fkl.fkl_backward_keep(h, W, idx, lg, out.lse, 1.0, z)
    torch.cuda.synchronize()
    assert out.loss.item() == 0.0 and gh.numel() == 0
    assert torch.count_nonzero(gw).item() == 0


def test_autograd_keep_matches_fused(gpu_device):
    """fused_chunked_kl with keep_logits=True / "auto" against keep_logits=False."""
    announce("autograd: kept logits vs recompute, bf16")
    w = synth.small_workload("keep_autograd", n=2 * 333, d=256, V=2500, K=64, T=1.0,
                             dtype="bf16", chunk=200)
    inp = synth.make_inputs(w)
    h, W, idx, lg = upload(inp)
    h3 = h.reshape(2, 333, -1)
    results = {}
    for keep in (False, True, "auto"):
        hh = h3.detach().clone().requires_grad_(True)
        WW = W.detach().clone().requires_grad_(True)
        loss = fkl.fused_chunked_kl(hh, WW, idx.reshape(2, 333, -1), lg.reshape(2, 333, -1),
                                    T=w.T, chunk=w.chunk, keep_logits=keep,
                                    memory_budget=1 << 40 if keep == "auto" else None)
        (0.5 * loss).backward()
        torch.cuda.synchronize()
        results[keep] = (loss.item(), hh.grad.double().cpu(), WW.grad.double().cpu())
    l0, gh0, gw0 = results[False]
    for keep in (True, "auto"):
        l1, gh1, gw1 = results[keep]
        assert l1 == l0
        assert (gh1 - gh0).abs().max() / gh0.abs().max() <= TOL["bf16"]["grad"]
        assert (gw1 - gw0).abs().max() / gw0.abs().max() <= TOL["bf16"]["grad"]
    with pytest.raises(ValueError):
        fkl.fused_chunked_kl(h, W, idx, lg, keep_logits="always")


def test_second_backward_through_kept_logits_is_refused(gpu_device):
    """The kept logits become G in the first backward; a second backward on
    the same graph (retain_graph) must raise instead of reading G as logits.
    The first backward's gradients equal the recompute path's."""
    announce("autograd: a second backward through consumed kept logits raises")
    w = synth.small_workload("keep_twice", n=300, d=128, V=1500, K=32, T=2.0,
                             dtype="fp32", chunk=128)
    inp = synth.make_inputs(w)
    h, W, idx, lg = upload(inp)
    grads = {}
    for keep in (False, True):
        hh = h.detach().clone().requires_grad_(True)
        WW = W.detach().clone().requires_grad_(True)
        loss = fkl.fused_chunked_kl(hh, WW, idx, lg, T=w.T, chunk=w.chunk, keep_logits=keep)
        loss.backward(retain_graph=True)
        torch.cuda.synchronize()
        grads[keep] = (hh.grad.double().cpu(), WW.grad.double().cpu())
        if keep:
            with pytest.raises(RuntimeError, match="consumed"):
                loss.backward()
        else:  # the recompute path may run backward again and gives the same gradient twice
            loss.backward()
            torch.cuda.synchronize()
            assert torch.equal(hh.grad.double().cpu(), 2 * grads[False][0])
    for a, b in zip(grads[True], grads[False]):
        assert (a - b).abs().max() / b.abs().max() <= TOL["fp32"]["grad"]

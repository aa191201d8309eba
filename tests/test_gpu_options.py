"""Loss options on the GPU against the fp64 oracle: per-row weights (with
zero-weight padding rows whose teacher logits are all -inf), hard labels (some
rows without one, some equal to a teacher id) mixed in with alpha at T = 1
(one softmax) and T != 1 (a separate temperature-1 softmax), for the fused
path and the kept-logits path, plus the autograd wrapper. Same tolerances as
the plain parity tests."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from sparse_top_kl_amd import fkl, synth
from tests.gpu_helpers import TOL, announce, compare, elementwise_ok, upload

pytestmark = pytest.mark.gpu


def _inputs(name, n, d, V, K, T, dtype, chunk, seed=None):
    w = synth.small_workload(name, n=n, d=d, V=V, K=K, T=T, dtype=dtype, chunk=chunk,
                             seed=zlib.crc32(name.encode()) % 1000 if seed is None else seed)
    return synth.make_inputs(w)


def _options(inp, weights, labels, rng):
    n, V = inp["hidden"].shape[0], inp["weight"].shape[0]
    wr = y = None
    if weights:
        wr = rng.uniform(0.25, 2.0, size=n).astype(np.float32)
        pad = rng.choice(n, size=max(1, n // 10), replace=False)
        wr[pad] = 0.0
        inp["topk_logit"][pad] = -np.inf                  # padding rows: no teacher entries
    if labels:
        y = rng.integers(0, V, size=n).astype(np.int32)
        y[rng.choice(n, size=max(1, n // 8), replace=False)] = -1                   # no label
        same = rng.choice(n, size=max(1, n // 8), replace=False)
        y[same] = inp["topk_idx"][same, 2]                # label equal to a teacher id
    return wr, y


def _tail_lse(inp, rng):
    """A teacher lse at T for the cached logits: the cache holds 1 / (1 + delta)
    of the teacher's mass, delta ~ U(0.05, 1.5) per row."""
    lg = inp["topk_logit"].astype(np.float64) / inp["T"]
    m = np.max(lg, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        cached = m[:, 0] + np.log(np.exp(lg - m).sum(axis=1))
    cached = np.where(np.isfinite(cached), cached, 0.0)
    return (cached + np.log1p(rng.uniform(0.05, 1.5, size=lg.shape[0]))).astype(np.float32)


def _run(inp, wr, y, alpha, keep, grad_scale=None, tlse=None):
    T, chunk = inp["T"], inp["chunk"]
    h, W, idx, lg = upload(inp)
    dev = h.device
    rwt = None if wr is None else torch.from_numpy(wr).to(dev)
    yt = None if y is None else torch.from_numpy(y).to(dev)
    tt = None if tlse is None else torch.from_numpy(tlse).to(dev)
    g = None if grad_scale is None else torch.tensor(float(grad_scale), device=dev)
    opts = dict(row_weight=rwt, labels=yt, alpha=alpha, teacher_lse=tt)
    if keep:
        out, z = fkl.fkl_forward_keep_ex(h, W, idx, lg, T, chunk, **opts)
        gh, gw = fkl.fkl_backward_keep_ex(h, W, idx, lg, out.lse, T, z, topk_z=out.topk_z,
                                          grad_loss=g, lse1=out.lse1, **opts)
    else:
        out = fkl.fkl_forward_ex(h, W, idx, lg, T, chunk, **opts)
        gh, gw = fkl.fkl_backward_ex(h, W, idx, lg, out.lse, T, chunk, topk_z=out.topk_z,
                                     grad_loss=g, lse1=out.lse1, **opts)
    torch.cuda.synchronize()
    res = {
        "loss": out.loss.item(),
        "lse": out.lse.double().cpu().numpy(),
        "row_loss": out.row_loss.double().cpu().numpy(),
        "topk_z": out.topk_z.double().cpu().numpy(),
        "grad_hidden": gh.double().cpu().numpy(),
        "grad_w": gw.double().cpu().numpy(),
    }
    if out.lse1 is not None:
        res["lse1"] = out.lse1.double().cpu().numpy()
    return res


CASES = [
    # name, n, d, V, K, T, dtype, chunk, weights, labels, alpha[, tail]
    ("weights_bf16", 600, 264, 3001, 100, 1.5, "bf16", 256, True, False, 1.0),
    ("weights_fp32", 300, 128, 2000, 60, 2.0, "fp32", 128, True, False, 1.0),
    ("labels_T2_bf16", 600, 264, 3001, 100, 2.0, "bf16", 256, False, True, 0.3),
    ("labels_T2_fp32", 300, 128, 2000, 60, 2.0, "fp32", 100, True, True, 0.7),
    ("labels_T1_bf16", 500, 256, 2500, 100, 1.0, "bf16", 200, True, True, 0.6),
    ("pure_ce_T15_bf16", 400, 128, 1800, 40, 1.5, "bf16", 128, False, True, 0.0),
    ("tail_T2_bf16", 600, 264, 3001, 100, 2.0, "bf16", 256, False, False, 1.0, True),
    ("tail_T1_fp32", 300, 128, 2000, 60, 1.0, "fp32", 128, False, False, 1.0, True),
    ("tail_all_options_bf16", 500, 256, 2500, 100, 1.5, "bf16", 200, True, True, 0.6, True),
]


@pytest.mark.parametrize("keep", [False, True], ids=["fused", "keep"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_options_against_oracle(gpu_device, case, keep):
    name, n, d, V, K, T, dtype, chunk, weights, labels, alpha = case[:11]
    tail = len(case) > 11 and case[11]
    announce(f"{name} ({'kept logits' if keep else 'fused'}): n={n} d={d} V={V} K={K} T={T} "
             f"{dtype} weights={weights} labels={labels} alpha={alpha} tail={tail}")
    inp = _inputs(name, n, d, V, K, T, dtype, chunk)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    wr, y = _options(inp, weights, labels, rng)
    tlse = _tail_lse(inp, rng) if tail else None
    res = _run(inp, wr, y, alpha, keep, grad_scale=-0.8, tlse=tlse)
    ref = oracle.forward_backward(inp["hidden"], inp["weight"], inp["topk_idx"],
                                  inp["topk_logit"], T, grad_scale=-0.8, row_weight=wr,
                                  labels=y, alpha=alpha, teacher_lse=tlse)
    assert np.all(np.isfinite(res["grad_w"])) and np.all(np.isfinite(res["row_loss"]))
    compare(res, ref, dtype)
    if y is not None:
        err = elementwise_ok(res["lse1"], ref["lse1"], TOL[dtype]["loss"])
        assert err <= TOL[dtype]["loss"], err
    if wr is not None:
        assert np.all(res["row_loss"][wr == 0] == 0.0)
        assert np.all(res["grad_hidden"][wr == 0] == 0.0)


def test_autograd_with_options(gpu_device):
    announce("autograd: row weights + labels, bf16, T = 2")
    inp = _inputs("opt_autograd", 2 * 150, 128, 2200, 50, 2.0, "bf16", 128)
    wr, y = _options(inp, True, True, np.random.default_rng(5))
    h, W, idx, lg = upload(inp)
    hh = h.detach().clone().reshape(2, 150, -1).requires_grad_(True)
    WW = W.detach().clone().requires_grad_(True)
    loss = fkl.fused_chunked_kl(hh, WW, idx.reshape(2, 150, -1), lg.reshape(2, 150, -1), T=2.0,
                                chunk=128, row_weight=torch.from_numpy(wr).cuda().reshape(2, 150),
                                labels=torch.from_numpy(y).cuda().reshape(2, 150), alpha=0.4)
    loss.backward()
    torch.cuda.synchronize()
    ref = oracle.forward_backward(inp["hidden"], inp["weight"], inp["topk_idx"],
                                  inp["topk_logit"], 2.0, row_weight=wr, labels=y, alpha=0.4)
    assert abs(loss.item() - ref["loss"]) <= TOL["bf16"]["loss"] * abs(ref["loss"])
    gh = hh.grad.reshape(300, -1).double().cpu().numpy()
    gw = WW.grad.double().cpu().numpy()
    assert np.abs(gh - ref["grad_hidden"]).max() / np.abs(ref["grad_hidden"]).max() <= 2e-2
    assert np.abs(gw - ref["grad_w"]).max() / np.abs(ref["grad_w"]).max() <= 2e-2


def test_validate_flag_rejects_a_label_out_of_range(gpu_device):
    announce("validate: label >= V")
    inp = _inputs("opt_validate", 50, 64, 500, 10, 1.0, "fp32", 32)
    h, W, idx, lg = upload(inp)
    y = torch.zeros(50, dtype=torch.int32, device=h.device)
    y[7] = 500
    with pytest.raises(fkl.FklError) as e:
        fkl.fkl_forward_ex(h, W, idx, lg, 1.0, 32, labels=y, alpha=0.5, validate=True)
    assert e.value.status == fkl.FKL_E_INDEX
    y[7] = -1                                     # no label: allowed
    fkl.fkl_forward_ex(h, W, idx, lg, 1.0, 32, labels=y, alpha=0.5, validate=True)
    torch.cuda.synchronize()


def test_teacher_cache_to_student_loss_with_tail(gpu_device):
    """The whole pipeline: the teacher top-K cache and its lse at T from
    fkl_teacher_topk_ex, fed to the student loss with the tail bucket, against
    the oracle computed from the same teacher inputs."""
    announce("pipeline: teacher cache (top-K + lse) -> student loss with tail, bf16, T = 2")
    T, K = 2.0, 64
    tw = synth.small_teacher_workload("pipe_teacher", n=400, d=192, V=2600, K=K, dtype="bf16",
                                      chunk=128)
    tin = synth.make_teacher_inputs(tw)
    sw = synth.small_workload("pipe_student", n=400, d=128, V=2600, K=K, T=T, dtype="bf16",
                              chunk=128)
    sin = synth.make_inputs(sw)
    dev = torch.device("cuda")
    th = torch.from_numpy(tin["hidden"]).to(dev).to(torch.bfloat16)
    tW = torch.from_numpy(tin["weight"]).to(dev).to(torch.bfloat16)
    idx, val, tlse = fkl.fkl_teacher_topk_ex(th, tW, K, 128, T=T)
    h = torch.from_numpy(sin["hidden"]).to(dev).to(torch.bfloat16)
    W = torch.from_numpy(sin["weight"]).to(dev).to(torch.bfloat16)
    out = fkl.fkl_forward_ex(h, W, idx, val, T, 128, teacher_lse=tlse)
    gh, gw = fkl.fkl_backward_ex(h, W, idx, val, out.lse, T, 128, topk_z=out.topk_z,
                                 teacher_lse=tlse)
    torch.cuda.synchronize()
    tl = oracle.teacher_logits(tin["hidden"], tin["weight"])
    ref_tlse = np.log(np.exp(tl / T - (tl / T).max(1, keepdims=True)).sum(1)) + (tl / T).max(1)
    assert elementwise_ok(tlse.double().cpu().numpy(), ref_tlse, 1e-5) <= 1e-5
    ref = oracle.forward_backward(sin["hidden"], sin["weight"], idx.cpu().numpy(),
                                  val.cpu().numpy(), T, teacher_lse=ref_tlse)
    res = {"loss": out.loss.item(), "lse": out.lse.double().cpu().numpy(),
           "row_loss": out.row_loss.double().cpu().numpy(),
           "topk_z": out.topk_z.double().cpu().numpy(),
           "grad_hidden": gh.double().cpu().numpy(), "grad_w": gw.double().cpu().numpy()}
    compare(res, ref, "bf16")


@pytest.mark.parametrize("T", [1.0, 2.0])
def test_lse1_without_labels_is_the_temperature_one_lse(gpu_device, T):
    """lse1 requested without labels: the forward writes ln sum exp(z) at
    temperature 1 (a second set of partials when T != 1), not the lse at T."""
    announce(f"lse1 without labels, T={T}")
    w = synth.small_workload("lse1_nolabels", n=300, d=64, V=1000, K=16, T=T, dtype="fp32",
                             chunk=128)
    inp = synth.make_inputs(w)
    h, W, idx, lg = upload(inp)
    lse1 = torch.empty(w.N, dtype=torch.float32, device=gpu_device)
    out = fkl.fkl_forward_ex(h, W, idx, lg, T, w.chunk, lse1=lse1)
    torch.cuda.synchronize()
    ref = oracle.forward_backward(inp["hidden"], inp["weight"], inp["topk_idx"],
                                  inp["topk_logit"], T, want_grads=False)
    tol = TOL["fp32"]["loss"]
    assert elementwise_ok(lse1.double().cpu().numpy(), ref["lse1"], tol) <= tol
    assert elementwise_ok(out.lse.double().cpu().numpy(), ref["lse"], tol) <= tol

"""The student-renormalised top-K loss on the GPU (fkl_renorm_forward /
fkl_renorm_backward through the C ABI) against the fp64 oracle
``oracle.renorm_forward_backward``, with the tolerances of the main loss.

Small shapes compare every output element: bf16 and fp32, uniform and
Zipf-skewed ids (hot ids whose pairs span several sort chunks), duplicate ids
in a row, -inf padding entries, zero-weight padding rows, K from 1 to 1024,
odd hidden sizes, a negative upstream scale, enough rows that the
frequent ids' dense product is split over rows and blocked, and ids that are
all below its threshold with runs of hundreds of pairs. Then: grad_W and
grad_hidden are bitwise repeatable, the accumulate flag adds, passing the forward's
gathered logits changes nothing, an empty batch zeroes grad_W, the autograd
wrapper matches, and at the long32k size sampled rows match the oracle while
the whole grad_W matches an independent fp32 PyTorch computation."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from sparse_top_kl_amd import fkl, synth
from tests.gpu_helpers import TOL, announce, elementwise_ok, max_rel_to_max, rel_err, upload

pytestmark = pytest.mark.gpu


def _inputs(name, n, d, V, K, T, dtype, ids="uniform", dup=False, pad=False):
    seed = zlib.crc32(name.encode()) % 1000
    w = synth.small_workload(name, n=n, d=d, V=V, K=K, T=T, dtype=dtype, chunk=128, ids=ids,
                             seed=seed)
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(seed)
    if dup:   # a few rows repeat an id (entries act separately)
        rows = rng.choice(n, size=max(1, n // 10), replace=False)
        inp["topk_idx"][rows, -1] = inp["topk_idx"][rows, 0]
    if pad and K > 1:   # trailing -inf entries: fewer than K cached
        rows = rng.choice(n, size=max(1, n // 5), replace=False)
        for r in rows:
            inp["topk_logit"][r, rng.integers(1, K):] = -np.inf
    return inp


def _run(inp, T, row_weight=None, grad_scale=None, pass_z=True):
    h, W, idx, lg = upload(inp)
    dev = h.device
    rw = None if row_weight is None else torch.from_numpy(row_weight).to(dev)
    g = None if grad_scale is None else torch.tensor(float(grad_scale), device=dev)
    out = fkl.fkl_renorm_forward(h, W, idx, lg, T, row_weight=rw)
    gh, gw = fkl.fkl_renorm_backward(h, W, idx, lg, T, topk_z=out.topk_z if pass_z else None,
                                     grad_loss=g, row_weight=rw)
    torch.cuda.synchronize()
    return {"loss": out.loss.item(), "row_loss": out.row_loss.double().cpu().numpy(),
            "topk_z": out.topk_z.double().cpu().numpy(),
            "grad_hidden": gh.double().cpu().numpy(), "grad_w": gw.double().cpu().numpy()}


def _compare(res, ref, dtype):
    tol = TOL[dtype]
    errs = {"loss": rel_err(res["loss"], ref["loss"]),
            "row_loss": elementwise_ok(res["row_loss"], ref["row_loss"], tol["loss"]),
            "topk_z": elementwise_ok(res["topk_z"], ref["topk_z"], tol["loss"]),
            "grad_hidden": max_rel_to_max(res["grad_hidden"], ref["grad_hidden"]),
            "grad_w": max_rel_to_max(res["grad_w"], ref["grad_w"])}
    print("    errors: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items()
           if not v <= (tol["grad"] if k.startswith("grad") else tol["loss"])}
    assert not bad, f"outside tolerance: {bad}"


CASES = [
    # name, n, d, V, K, T, dtype, ids, dup, pad, weights, grad_scale
    ("bf16_uniform", 600, 264, 3001, 100, 2.0, "bf16", "uniform", False, False, False, None),
    ("fp32_uniform", 300, 128, 2000, 60, 1.0, "fp32", "uniform", False, False, False, -0.6),
    ("bf16_zipf_hot_ids", 900, 256, 4000, 100, 2.0, "bf16", "zipf", False, False, False, None),
    ("fp32_zipf_dup_pad_weights", 700, 136, 2500, 100, 1.5, "fp32", "zipf", True, True, True,
     0.8),
    ("bf16_dup_pad_weights", 500, 2880, 3000, 100, 1.0, "bf16", "uniform", True, True, True,
     None),
    ("bf16_K1", 200, 64, 500, 1, 1.0, "bf16", "uniform", False, False, False, None),
    ("fp32_K300", 150, 72, 1200, 300, 3.0, "fp32", "zipf", True, True, False, None),
    ("bf16_K1024_d8192", 40, 8192, 2048, 1024, 1.0, "bf16", "uniform", False, True, False, None),
    # many rows: the frequent ids' dense product runs in 8 row splits, and for fp32 its
    # coefficient matrix (at most 256 MiB) takes three row blocks accumulated in turn
    ("bf16_40k_rows_hot_splits", 40000, 64, 3000, 16, 2.0, "bf16", "zipf", True, False, False,
     None),
    ("fp32_70k_rows_hot_blocks", 70000, 64, 3000, 16, 1.0, "fp32", "zipf", False, True, True,
     0.5),
    # a 7-id vocabulary: every id is frequent, the sorted walk gets no pair at all
    ("bf16_tiny_vocab_all_hot", 400, 64, 7, 5, 1.0, "bf16", "uniform", True, True, False, None),
    # every id has ~700 (~800) pairs: more ids than the dense product takes reach each
    # power-of-two threshold below 1024, so none is frequent and the sorted walk sums runs
    # that span many of a chunk's shares and cross chunks; d not a multiple of the walk's
    # 64-column slices
    ("bf16_long_cold_runs", 21000, 72, 3000, 100, 2.0, "bf16", "uniform", False, False, False,
     None),
    ("fp32_long_cold_runs", 20000, 40, 2500, 100, 1.0, "fp32", "uniform", True, False, False,
     None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_renorm_against_oracle(gpu_device, case):
    name, n, d, V, K, T, dtype, ids, dup, pad, weights, gs = case
    announce(f"renorm {name}: n={n} d={d} V={V} K={K} T={T} {dtype} ids={ids} dup={dup} "
             f"pad={pad} weights={weights} grad_scale={gs}")
    inp = _inputs(name, n, d, V, K, T, dtype, ids, dup, pad)
    wr = None
    if weights:
        rng = np.random.default_rng(3)
        wr = rng.uniform(0.25, 2.0, size=n).astype(np.float32)
        zero = rng.choice(n, size=max(1, n // 10), replace=False)
        wr[zero] = 0.0
        inp["topk_logit"][zero[0]] = -np.inf        # a padding row: weight 0, no entries
    res = _run(inp, T, row_weight=wr, grad_scale=gs)
    ref = oracle.renorm_forward_backward(inp["hidden"], inp["weight"], inp["topk_idx"],
                                         inp["topk_logit"], T, grad_scale=1.0 if gs is None else gs,
                                         row_weight=wr)
    assert np.all(np.isfinite(res["grad_w"])) and np.all(np.isfinite(res["row_loss"]))
    _compare(res, ref, dtype)
    # ids no row caches get an exact zero row
    unused = np.setdiff1d(np.arange(V), inp["topk_idx"].ravel())
    assert np.all(res["grad_w"][unused] == 0.0)
    if wr is not None:
        assert np.all(res["row_loss"][wr == 0] == 0.0)
        assert np.all(res["grad_hidden"][wr == 0] == 0.0)


def test_renorm_is_bitwise_repeatable_and_accumulates(gpu_device):
    announce("renorm: repeatability, accumulate flag, gathered logits passed or recomputed")
    inp = _inputs("repeat", 800, 192, 3000, 100, 2.0, "bf16", "zipf", True, True)
    h, W, idx, lg = upload(inp)
    out = fkl.fkl_renorm_forward(h, W, idx, lg, 2.0)
    gh1, gw1 = fkl.fkl_renorm_backward(h, W, idx, lg, 2.0, topk_z=out.topk_z)
    gh2, gw2 = fkl.fkl_renorm_backward(h, W, idx, lg, 2.0)          # gathers again
    out2 = fkl.fkl_renorm_forward(h, W, idx, lg, 2.0)
    torch.cuda.synchronize()
    assert torch.equal(out.loss, out2.loss) and torch.equal(out.row_loss, out2.row_loss)
    assert torch.equal(gh1, gh2) and torch.equal(gw1, gw2)
    base = torch.randn_like(gw1)
    acc = base.clone()
    fkl.fkl_renorm_backward(h, W, idx, lg, 2.0, topk_z=out.topk_z, grad_weight=acc,
                            accumulate=True)
    torch.cuda.synchronize()
    assert torch.allclose(acc, base + gw1, rtol=1e-6, atol=1e-6)


def test_renorm_empty_batch_and_validation(gpu_device):
    announce("renorm: N = 0, id validation")
    dev = torch.device("cuda")
    h = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    W = torch.randn(500, 64, device=dev).to(torch.bfloat16)
    idx = torch.empty(0, 10, dtype=torch.int32, device=dev)
    lg = torch.empty(0, 10, dtype=torch.float32, device=dev)
    out = fkl.fkl_renorm_forward(h, W, idx, lg, 1.0)
    gw = torch.full((500, 64), float("nan"), device=dev)
    fkl.fkl_renorm_backward(h, W, idx, lg, 1.0, grad_weight=gw)
    torch.cuda.synchronize()
    assert out.loss.item() == 0.0 and torch.all(gw == 0)
    inp = _inputs("validate", 50, 64, 500, 10, 1.0, "fp32")
    h, W, idx, lg = upload(inp)
    idx[7, 3] = 500
    with pytest.raises(fkl.FklError) as e:
        fkl.fkl_renorm_forward(h, W, idx, lg, 1.0, validate=True)
    assert e.value.status == fkl.FKL_E_INDEX


def test_renorm_autograd(gpu_device):
    announce("renorm: autograd wrapper, [B, S, d] input, row weights")
    inp = _inputs("autograd", 2 * 160, 128, 2200, 50, 2.0, "bf16", "zipf")
    h, W, idx, lg = upload(inp)
    wr = np.random.default_rng(9).uniform(0.0, 1.0, size=320).astype(np.float32)
    hh = h.detach().clone().reshape(2, 160, -1).requires_grad_(True)
    WW = W.detach().clone().requires_grad_(True)
    loss = fkl.renorm_topk_kl(hh, WW, idx.reshape(2, 160, -1), lg.reshape(2, 160, -1), T=2.0,
                              row_weight=torch.from_numpy(wr).cuda().reshape(2, 160))
    (-0.5 * loss).backward()
    torch.cuda.synchronize()
    ref = oracle.renorm_forward_backward(inp["hidden"], inp["weight"], inp["topk_idx"],
                                         inp["topk_logit"], 2.0, grad_scale=-0.5, row_weight=wr)
    assert rel_err(loss.item(), ref["loss"]) <= TOL["bf16"]["loss"]
    assert max_rel_to_max(hh.grad.reshape(320, -1).double().cpu().numpy(),
                          ref["grad_hidden"]) <= TOL["bf16"]["grad"]
    assert max_rel_to_max(WW.grad.double().cpu().numpy(), ref["grad_w"]) <= TOL["bf16"]["grad"]


def _torch_renorm(h, W, idx, lg, T, rows_per=1024):
    """fp32 PyTorch version of the renormalised loss's gradients: torch's
    log_softmax over the cached entries, index_add_ for grad_W."""
    N, d = h.shape
    gh = torch.empty(N, d, dtype=torch.float32, device=h.device)
    gw = torch.zeros(W.shape[0], d, dtype=torch.float32, device=h.device)
    rl = torch.empty(N, dtype=torch.float64, device=h.device)
    for r0 in range(0, N, rows_per):
        hb = h[r0:r0 + rows_per].float()
        ib = idx[r0:r0 + rows_per].long()
        wb = W[ib].float()                                  # [R, K, d]
        zk = torch.einsum("rd,rkd->rk", hb, wb)
        lp = torch.log_softmax(lg[r0:r0 + rows_per] / T, 1)
        lq = torch.log_softmax(zk / T, 1)
        p = lp.exp()
        rl[r0:r0 + rows_per] = (T * T * (p * (lp - lq)).sum(1)).double()
        G = T * (lq.exp() * p.sum(1, keepdim=True) - p)
        gh[r0:r0 + rows_per] = torch.einsum("rk,rkd->rd", G, wb)
        gw.index_add_(0, ib.reshape(-1), (G[:, :, None] * hb[:, None, :]).reshape(-1, d))
        del wb
    return rl, gh, gw


@pytest.mark.timeout(600)
def test_renorm_full_size_long32k(gpu_device):
    w = synth.WORKLOADS["long32k"]
    announce(f"renorm full size long32k: N={w.N} d={w.d} V={w.V} K={w.K} T={w.T} (generating)")
    inp = synth.make_inputs(w)
    h, W, idx, lg = upload(inp)
    out = fkl.fkl_renorm_forward(h, W, idx, lg, w.T)
    gh, gw = fkl.fkl_renorm_backward(h, W, idx, lg, w.T, topk_z=out.topk_z)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, w.N - 1} | set(np.random.default_rng(5).choice(w.N, 30).tolist())))
    announce(f"renorm full size: oracle on {len(rows)} rows")
    ref = oracle.renorm_forward_backward(inp["hidden"][rows], inp["weight"], inp["topk_idx"][rows],
                                         inp["topk_logit"][rows], w.T)
    sel = torch.as_tensor(rows, device=gpu_device)
    tol = TOL["bf16"]
    errs = {"row_loss": elementwise_ok(out.row_loss[sel].double().cpu().numpy(), ref["row_loss"],
                                       tol["loss"]),
            "topk_z": elementwise_ok(out.topk_z[sel].double().cpu().numpy(), ref["topk_z"],
                                     tol["loss"]),
            "grad_hidden": max_rel_to_max(gh[sel].double().cpu().numpy(), ref["grad_hidden"])}
    announce("renorm full size: fp32 PyTorch gradients of all rows")
    rl_t, gh_t, gw_t = _torch_renorm(h, W, idx, lg, w.T)
    errs["loss_vs_torch"] = rel_err(out.loss.item(), float(rl_t.sum().item()))
    errs["grad_hidden_vs_torch"] = float(((gh.float() - gh_t).abs().max() /
                                          gh_t.abs().max()).item())
    errs["grad_w_vs_torch"] = float(((gw - gw_t).abs().max() / gw_t.abs().max()).item())
    print("    errors: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    limits = {"row_loss": tol["loss"], "topk_z": tol["loss"], "grad_hidden": tol["grad"],
              "loss_vs_torch": tol["loss"], "grad_hidden_vs_torch": tol["grad"],
              "grad_w_vs_torch": tol["grad"]}
    bad = {k: (errs[k], limits[k]) for k in limits if not errs[k] <= limits[k]}
    assert not bad, f"outside tolerance: {bad}"

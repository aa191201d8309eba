"""Parity at the full workload sizes, in the launch configuration the
benchmark times (same chunk, library-planned blocking, bf16 inputs).

The fp64 oracle cannot afford the whole N x V problem, so these tests check
  * sampled rows against the oracle, element by element: lse, per-row loss,
    z at the teacher ids, and the full grad_hidden row (each needs only its
    own row of logits);
  * properties that hold at any size: every per-row loss is a temperature-
    scaled KL divergence (>= 0), the loss is the fixed-order sum of the
    per-row losses, every row of the logit gradient G sums to zero so
    sum_v grad_W[v, :] vanishes, and <grad_W, W> = <grad_hidden, H> (both
    equal sum over rows and vocabulary of G * z);
  * grad_W rows of sampled vocabulary ids against an independent PyTorch
    fp32 computation that builds its own log-sum-exp over the whole
    vocabulary (no value of the HIP path enters it).
The forward-chunked variant (kept logits) runs on two of the workloads: its
forward outputs must equal the fused forward's bitwise, and its gradients
pass the same checks.
Tolerances are those of the small-shape parity tests (bf16: 1e-3 relative on
loss-like values, 2e-2 of the largest reference magnitude on gradients); the
two summation properties use bounds derived in the test from bf16 rounding of
G and fp32 accumulation.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_top_kl_amd import fkl, synth
from tests.gpu_helpers import TOL, announce, elementwise_ok, max_rel_to_max

pytestmark = pytest.mark.gpu

FULL_WORKLOADS = ["llama3b_8k", "long32k", "gptoss20b_32k", "stress_b1_64k", "stress_b4_32k"]
N_SAMPLE_ROWS = 8
N_SAMPLE_VOCAB = 48


def _sample_rows(w, rng):
    """First and last rows, both sides of the first chunk boundary, and random rows."""
    fixed = {0, w.N - 1, min(w.chunk, w.N) - 1, min(w.chunk, w.N - 1)}
    rest = rng.choice(w.N, size=N_SAMPLE_ROWS - len(fixed), replace=False)
    return np.array(sorted(fixed | set(int(r) for r in rest)))


def _torch_grad_w_rows(h32, w32, idx, lg, T, vocab, chunk=2048):
    """grad_W[v, :] for the given vocabulary ids, in fp32 on the GPU: own
    log-sum-exp over all V, teacher softmax over the K entries, then
    G[:, v] = T * (q[:, v] * sum_k p - sum_{k: idx = v} p) and G[:, v]^T H."""
    N = h32.shape[0]
    lse = torch.empty(N, dtype=torch.float32, device=h32.device)
    for r0 in range(0, N, chunk):
        z = torch.matmul(h32[r0:r0 + chunk], w32.t())                 # fp32, 2-D
        lse[r0:r0 + chunk] = torch.logsumexp(z / T, dim=1)
        del z
    p = torch.softmax(lg / T, dim=1)                                   # [N, K]
    vv = torch.as_tensor(vocab, device=h32.device, dtype=torch.long)
    zv = torch.matmul(h32, w32[vv].t().contiguous())                  # [N, S]
    q = torch.exp(zv / T - lse[:, None])
    scatter = torch.stack([(p * (idx == int(v)).float()).sum(dim=1) for v in vocab], dim=1)
    G = T * (q * p.sum(dim=1, keepdim=True) - scatter)                # [N, S]
    return (G.t().contiguous() @ h32).double().cpu().numpy()          # [S, d]


# (workload, keep, options): keep=True runs the forward-chunked variant (kept
# logits); options=True adds hard labels (alpha 0.5) and the teacher-tail bucket
CASES = ([(n, False, False) for n in FULL_WORKLOADS] +
         [("long32k", True, False), ("stress_b4_32k", True, False), ("long32k", False, True)])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,keep,options", CASES,
                         ids=[n + ("-keep" if k else "") + ("-options" if o else "")
                              for n, k, o in CASES])
def test_full_size_parity(name, keep, options, gpu_device):
    w = synth.WORKLOADS[name]
    tol = TOL[w.dtype]
    announce(f"full size {name}{' (kept logits)' if keep else ''}"
             f"{' (labels + tail)' if options else ''}: N={w.N} d={w.d} V={w.V} "
             f"K={w.K} T={w.T} chunk={w.chunk} {w.dtype} ids={w.ids} (generating inputs)")
    inp = synth.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    h = torch.from_numpy(inp["hidden"]).to(gpu_device).to(dt).contiguous()
    W = torch.from_numpy(inp["weight"]).to(gpu_device).to(dt).contiguous()
    idx = torch.from_numpy(inp["topk_idx"]).to(gpu_device)
    lg = torch.from_numpy(inp["topk_logit"]).to(gpu_device)

    opts = {}
    if options:
        rng_o = np.random.default_rng(99)
        y = rng_o.integers(0, w.V, size=w.N).astype(np.int32)
        lg64 = inp["topk_logit"].astype(np.float64) / w.T
        mx = lg64.max(axis=1)
        tlse = (mx + np.log(np.exp(lg64 - mx[:, None]).sum(axis=1)) + np.log(2.0)).astype(
            np.float32)
        opts = dict(labels=y, alpha=0.5, teacher_lse=tlse)
    announce(f"full size {name}: HIP forward + backward")
    if options:
        topts = dict(labels=torch.from_numpy(y).to(gpu_device), alpha=0.5,
                     teacher_lse=torch.from_numpy(tlse).to(gpu_device))
        out = fkl.fkl_forward_ex(h, W, idx, lg, w.T, w.chunk, **topts)
        gh, gw = fkl.fkl_backward_ex(h, W, idx, lg, out.lse, w.T, w.chunk, topk_z=out.topk_z,
                                     lse1=out.lse1, **topts)
    elif keep:
        out, z = fkl.fkl_forward_keep(h, W, idx, lg, w.T, w.chunk)
        ref_out = fkl.fkl_forward(h, W, idx, lg, w.T, w.chunk)
        for field in ("loss", "lse", "row_loss", "topk_z"):
            assert torch.equal(getattr(out, field), getattr(ref_out, field)), field
        del ref_out
        gh, gw = fkl.fkl_backward_keep(h, W, idx, lg, out.lse, w.T, z, topk_z=out.topk_z)
        torch.cuda.synchronize()
        del z
    else:
        out = fkl.fkl_forward(h, W, idx, lg, w.T, w.chunk)
        gh, gw = fkl.fkl_backward(h, W, idx, lg, out.lse, w.T, w.chunk, topk_z=out.topk_z)
    torch.cuda.synchronize()
    loss = out.loss.item()
    row_loss = out.row_loss.double().cpu().numpy()
    assert math.isfinite(loss)
    assert np.isfinite(row_loss).all()

    # properties of the forward at full size
    assert abs(loss - math.fsum(row_loss.tolist())) <= 1e-6 * max(1.0, abs(loss))
    assert row_loss.min() >= -tol["loss"] * max(1.0, float(np.abs(row_loss).max()))

    # sampled rows against the oracle
    rng = np.random.default_rng(20261203)
    rows = _sample_rows(w, rng)
    announce(f"full size {name}: oracle on rows {rows.tolist()}")
    sub = {k: v[rows] for k, v in opts.items() if k != "alpha"}
    if options:
        sub["alpha"] = opts["alpha"]
    ref = oracle.forward_backward(inp["hidden"][rows], inp["weight"], inp["topk_idx"][rows],
                                  inp["topk_logit"][rows], w.T, **sub)
    sel = torch.as_tensor(rows, device=gpu_device)
    errs = {
        "lse": elementwise_ok(out.lse[sel].double().cpu().numpy(), ref["lse"], tol["loss"]),
        "row_loss": elementwise_ok(row_loss[rows], ref["row_loss"], tol["loss"]),
        "topk_z": elementwise_ok(out.topk_z[sel].double().cpu().numpy(), ref["topk_z"],
                                 tol["loss"]),
        "grad_hidden": max_rel_to_max(gh[sel].double().cpu().numpy(), ref["grad_hidden"]),
    }
    del ref

    # grad_W: column sums vanish. Each G element is rounded to bf16 (relative
    # 2^-9) and sum_v |G[n, v]| <= 2T (sum_v q_v + sum_k p_k), so
    # |sum_v grad_W[v, j]| <= (2^-9 + N 2^-24) 2T sum_n |H[n, j]|, plus the
    # same order again for fp32 accumulation; the bound uses twice that.
    colsum = gw.double().sum(dim=0)
    habs = h.float().abs().double().sum(dim=0)
    bound = 2.0 * (2.0 ** -9 + w.N * 2.0 ** -24) * 2.0 * w.T * habs
    worst = float((colsum.abs() / bound).max().item())
    errs["grad_w_colsum/bound"] = worst

    # <grad_W, W> = <grad_hidden, H>
    a = float((gw.double() * W.double()).sum().item())
    b = float((gh.double() * h.double()).sum().item())
    scale = float((gw.double().abs() * W.double().abs()).sum().item())
    errs["<gW,W>-<gH,H>"] = abs(a - b) / max(scale, 1e-30)

    limits = {"lse": tol["loss"], "row_loss": tol["loss"], "topk_z": tol["loss"],
              "grad_hidden": tol["grad"], "grad_w_colsum/bound": 1.0,
              "<gW,W>-<gH,H>": tol["grad"], "grad_w_rows": tol["grad"]}
    if options:  # the torch fp32 grad_W rows below implement the plain loss only
        print("    errors: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
        bad = {k: (errs[k], limits[k]) for k in errs if not errs[k] <= limits[k]}
        assert not bad, f"outside tolerance: {bad}"
        return
    # grad_W rows of sampled vocabulary ids (teacher ids included) against torch fp32
    teacher = inp["topk_idx"][rows[0]][:N_SAMPLE_VOCAB // 2]
    vocab = np.unique(np.concatenate([teacher, rng.choice(w.V, N_SAMPLE_VOCAB // 2, replace=False),
                                      [0, w.V - 1]]))
    announce(f"full size {name}: torch fp32 grad_W on {len(vocab)} vocabulary rows")
    ref_gw = _torch_grad_w_rows(h.float(), W.float(), idx, lg, w.T, vocab)
    errs["grad_w_rows"] = max_rel_to_max(gw[torch.as_tensor(vocab, device=gpu_device)]
                                         .double().cpu().numpy(), ref_gw)
    print("    errors: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: (errs[k], limits[k]) for k in limits if not errs[k] <= limits[k]}
    assert not bad, f"outside tolerance: {bad}"

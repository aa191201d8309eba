"""Shared helpers of the GPU tests: upload seeded inputs, run the HIP path
through the C ABI, compare against the fp64 oracle with the stated tolerances.

Tolerances (fixed by the target of this library, not derived from results):
  loss:  relative error <= 1e-3 (bf16 inputs) / 1e-5 (fp32 inputs)
  grads: max |err| / max |reference| <= 2e-2 (bf16) / 1e-4 (fp32)
lse, per-row loss and gathered logits use the loss tolerance (relative, per
element, with an absolute floor of the same size for values near 0).
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from sparse_top_kl_amd import fkl

TOL = {
    "bf16": {"loss": 1e-3, "grad": 2e-2},
    "fp32": {"loss": 1e-5, "grad": 1e-4},
}


def announce(msg: str):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def upload(inp: dict, device="cuda"):
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    h = torch.from_numpy(np.ascontiguousarray(inp["hidden"])).to(device).to(dt).contiguous()
    w = torch.from_numpy(np.ascontiguousarray(inp["weight"])).to(device).to(dt).contiguous()
    idx = torch.from_numpy(np.ascontiguousarray(inp["topk_idx"]).astype(np.int32)).to(device)
    lg = torch.from_numpy(np.ascontiguousarray(inp["topk_logit"]).astype(np.float32)).to(device)
    return h, w, idx, lg


def run_gpu(inp: dict, T=None, chunk=None, grad_scale=None, with_backward=True):
    T = inp["T"] if T is None else T
    chunk = inp["chunk"] if chunk is None else chunk
    h, w, idx, lg = upload(inp)
    out = fkl.fkl_forward(h, w, idx, lg, T, chunk)
    res = {
        "loss": out.loss.item(),
        "lse": out.lse.double().cpu().numpy(),
        "row_loss": out.row_loss.double().cpu().numpy(),
        "topk_z": out.topk_z.double().cpu().numpy(),
    }
    if with_backward:
        g = None if grad_scale is None else torch.tensor(float(grad_scale), device=h.device)
        gh, gw = fkl.fkl_backward(h, w, idx, lg, out.lse, T, chunk, topk_z=out.topk_z,
                                  grad_loss=g)
        torch.cuda.synchronize()
        res["grad_hidden"] = gh.double().cpu().numpy()
        res["grad_w"] = gw.double().cpu().numpy()
    torch.cuda.synchronize()
    return res


def rel_err(a, b):
    return abs(a - b) / max(abs(b), 1e-30)


def max_rel_to_max(a: np.ndarray, ref: np.ndarray) -> float:
    scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(a).max())
    return float(np.abs(a - ref).max() / scale)


def elementwise_ok(a: np.ndarray, ref: np.ndarray, tol: float) -> float:
    """Largest |a - ref| / max(|ref|, 1) (relative with an absolute floor)."""
    return float((np.abs(a - ref) / np.maximum(np.abs(ref), 1.0)).max()) if a.size else 0.0


def compare(gpu: dict, ref: dict, dtype: str, grads=True) -> dict:
    tol = TOL[dtype]
    errs = {
        "loss": rel_err(gpu["loss"], ref["loss"]),
        "lse": elementwise_ok(gpu["lse"], ref["lse"], tol["loss"]),
        "row_loss": elementwise_ok(gpu["row_loss"], ref["row_loss"], tol["loss"]),
        "topk_z": elementwise_ok(gpu["topk_z"], ref["topk_z"], tol["loss"]),
    }
    if grads:
        errs["grad_hidden"] = max_rel_to_max(gpu["grad_hidden"], ref["grad_hidden"])
        errs["grad_w"] = max_rel_to_max(gpu["grad_w"], ref["grad_w"])
    limits = {k: (tol["grad"] if k.startswith("grad") else tol["loss"]) for k in errs}
    bad = {k: (errs[k], limits[k]) for k in errs if not errs[k] <= limits[k]}
    print(f"    errors: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert not bad, f"outside tolerance: {bad}"
    return errs

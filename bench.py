#!/usr/bin/env python3
"""Benchmark of the fused chunked top-K KL loss (forward + backward) on one MI355X.

One step = fkl_forward + fkl_backward over all rows of the workload (every
chunk), inputs resident in HBM, workspaces allocated before timing. Prints one
JSON line: throughput in tokens/s, the MFMA roofline of the dominant kernel
(its average launch time measured with HIP events inside the timed region),
peak HBM of one step, a sampled parity check against the fp64 oracle and the
oracle's own host throughput on a bounded sample of the same rows.

With --memory-sweep it measures the peak HBM of one step at 4096 .. 65536
tokens and fits it linearly (memory grows linearly with sequence length, no
N x V buffer). With --teacher-topk it times the teacher top-K cache producer
(fkl_teacher_topk over a teacher workload) and prints that line instead.
With --keep-logits the step is the forward-chunked variant instead
(fkl_forward_keep + fkl_backward_keep: the logits are kept in an N x V buffer
and not recomputed, 6 N d V flops per step). Where tests/golden holds the
oracle's values for the workload, every row's lse and row loss, the total
loss and the stored grad_W rows are compared with them (parity_fixture).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--keep-logits]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "fused KL fwd+bwd tokens/s + % bf16 MFMA peak; peak HBM GiB at 32K tokens"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2516.6, "fp32": 157.3}
PEAK_HBM_GBS = 8000.0
GEMM_KERNELS = ("k_logits_lse", "k_gprod", "k_grad_hidden", "k_grad_w")
# figures printed on the pages (context only, other hardware, other scope)
PAGE_CONTEXT = {
    "isolated_32k_loss_peak_GiB": {"dense": 85.2, "fused_chunked": 5.45},
    "h200_8k_training_peak_GB": {"online": 102.8, "fully_chunked": 58.3},
    "gptoss20b_32768_step_s": {"before": 57.0, "after": 12.23},
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the kernel and library sources without comments or blank lines,
    so that counters stay attached to the code they were measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_top_kl_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
        h.update(name.encode() + "\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(workload, {}).get(kernel)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(inp, gpu_rows: dict, budget_s: float):
    """Time the fp64 oracle (as it stands) on a bounded prefix of the rows and
    compare its outputs for those rows with the GPU's."""
    import oracle
    from threadpoolctl import threadpool_info

    w = inp["workload"]

    def run(n):
        t0 = time.perf_counter()
        out = oracle.forward_backward(inp["hidden"][:n], inp["weight"], inp["topk_idx"][:n],
                                      inp["topk_logit"][:n], w.T)
        return out, time.perf_counter() - t0

    # The oracle works in blocks of 128 rows, each costing three fp64 products
    # over the whole vocabulary, plus a fixed cost per call (the fp64 copy of
    # W); calibrate on one and two blocks, then size the sample to the budget.
    _, t1 = run(128)
    _, t2 = run(256)
    per_row = max((t2 - t1) / 128, 1e-6)
    fixed = max(t1 - 128 * per_row, 0.0)
    n = int((budget_s - fixed) / per_row) // 128 * 128
    n = max(128, min(w.N, n))
    out, t = run(n)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    tol = 1e-3 if w.dtype == "bf16" else 1e-5
    gtol = 2e-2 if w.dtype == "bf16" else 1e-4
    lse_err = float(np.max(np.abs(gpu_rows["lse"][:n] - out["lse"]) / np.abs(out["lse"])))
    rl_err = float(np.max(np.abs(gpu_rows["row_loss"][:n] - out["row_loss"]) /
                          np.maximum(np.abs(out["row_loss"]), 1.0)))
    gh_err = float(np.max(np.abs(gpu_rows["grad_hidden"][:n] - out["grad_hidden"])) /
                   np.max(np.abs(out["grad_hidden"])))
    parity = {
        "rows": n,
        "lse_rel_err": lse_err,
        "row_loss_rel_err": rl_err,
        "grad_hidden_err_over_max": gh_err,
        "ok": bool(lse_err <= tol and rl_err <= tol and gh_err <= gtol),
    }
    base = {
        "value": n / t,
        "unit": "tokens/s",
        "cores": int(threads),
        "gflops_fp64": 6.0 * n * w.d * w.V / t / 1e9,   # the oracle needs no recompute
        "kind": "oracle",
        "sample": f"first {n} of {w.N} rows of {w.name}, forward+backward in fp64 "
                  f"(NumPy BLAS), {t:.1f} s; grad_W restricted to those rows",
    }
    return base, parity


def fixture_parity(case: str, w, gpu_rows: dict, gw_rows):
    """Every row's lse and row loss, the total loss and the stored grad_W rows
    against the oracle's values for this workload (tests/golden, written by
    tests/golden/make_fullsize_fixtures.py, which runs only the oracle);
    None when there is no fixture for the case."""
    path = os.path.join(ROOT, "tests", "golden", f"fullsize_{case}.npz")
    if not os.path.exists(path):
        return None
    with np.load(path, allow_pickle=False) as f:
        fx = {k: f[k] for k in f.files}
    if (list(fx["params"]) != [w.B, w.S, w.d, w.V, w.K, w.chunk, w.seed]
            or float(fx["T"]) != w.T):
        return None
    tol = 1e-3 if w.dtype == "bf16" else 1e-5
    gtol = 2e-2 if w.dtype == "bf16" else 1e-4

    def rel_floor(a, b):
        return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1.0)))

    out = {
        "case": case,
        "rows": int(w.N),
        "lse_err": rel_floor(gpu_rows["lse"], fx["lse"].astype(np.float64)),
        "row_loss_err": rel_floor(gpu_rows["row_loss"], fx["row_loss"].astype(np.float64)),
        "loss_rel_err": abs(gpu_rows["loss"] - float(fx["loss"])) / abs(float(fx["loss"])),
    }
    for g in ("hot", "cold", "tail", "random"):
        ref = fx[f"grad_w_{g}"].astype(np.float64)
        out[f"grad_w_{g}_err_over_max"] = float(np.max(np.abs(gw_rows(fx[f"vocab_{g}"]) - ref)) /
                                                np.max(np.abs(ref)))
    out["ok"] = bool(out["lse_err"] <= tol and out["row_loss_err"] <= tol and
                     out["loss_rel_err"] <= tol and
                     all(out[f"grad_w_{g}_err_over_max"] <= gtol
                         for g in ("hot", "cold", "tail", "random")))
    return out


def calibration_copy(args, torch, dev):
    """A plain device copy of known size (for calibrating byte counters)."""
    if args.copy_calibration_mib <= 0:
        return
    nb = args.copy_calibration_mib << 20
    src = torch.ones(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    log(f"[bench] calibration copy of {args.copy_calibration_mib} MiB done")


def cpu_baseline_topk(inp, gpu_idx, gpu_val, budget_s: float):
    """Time the fp64 teacher top-K oracle on a bounded prefix of the rows and
    compare those rows with the GPU's."""
    import oracle
    from threadpoolctl import threadpool_info

    w = inp["workload"]

    def run(n):
        t0 = time.perf_counter()
        logits = oracle.teacher_logits(inp["hidden"][:n], inp["weight"])
        ids, vals = oracle.topk_rows(logits, w.K)
        return logits, ids, vals, time.perf_counter() - t0

    _, _, _, t1 = run(32)
    _, _, _, t2 = run(64)
    per_row = max((t2 - t1) / 32, 1e-6)
    fixed = max(t1 - 32 * per_row, 0.0)
    n = int((budget_s - fixed) / per_row) // 32 * 32
    n = max(32, min(w.N, n))
    logits, ids, vals, t = run(n)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    tol = 1e-5  # fp32 accumulation against fp64 (relative, absolute floor 1)
    val_err = float(np.max(np.abs(gpu_val[:n] - vals) / np.maximum(np.abs(vals), 1.0)))
    # ids may order near-equal logits differently from fp64; what is unique is
    # the k-th largest value, so the GPU's k-th id must carry it (in fp64)
    at = np.take_along_axis(logits, gpu_idx[:n].astype(np.int64), axis=1)
    rank_err = float(np.max(np.abs(at - vals) / np.maximum(np.abs(vals), 1.0)))
    distinct = all(len(set(r.tolist())) == w.K for r in gpu_idx[:n])
    rows_differ = int((gpu_idx[:n] != ids).any(axis=1).sum())
    parity = {"rows": n, "value_rel_err": val_err, "kth_id_value_rel_err": rank_err,
              "rows_ordering_near_ties_differently": rows_differ,
              "ok": bool(val_err <= tol and rank_err <= 2 * tol and distinct)}
    base = {"value": n / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {w.N} rows of {w.name}: fp64 logits (NumPy BLAS) and "
                      f"exact per-row selection, {t:.1f} s"}
    return base, parity


def run_teacher_topk(args, torch, fkl, synth, dev):
    """Benchmark of the teacher top-K cache producer (fkl_teacher_topk)."""
    name = args.workload if args.workload in synth.TEACHER_WORKLOADS else "teacher_llama8b_32k"
    w = synth.TEACHER_WORKLOADS[name]
    log(f"[bench] generating {w.name}: N={w.N} d={w.d} V={w.V} K={w.K} chunk={w.chunk} {w.dtype}")
    inp = synth.make_teacher_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    h = torch.from_numpy(inp["hidden"]).to(dev).to(dt).contiguous()
    W = torch.from_numpy(inp["weight"]).to(dev).to(dt).contiguous()
    torch.cuda.synchronize()
    input_bytes = sum(t.numel() * t.element_size() for t in (h, W))
    nb = fkl.fkl_topk_workspace_size(w.N, w.d, w.V, w.K, w.chunk, dt)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    def step():
        return fkl.fkl_teacher_topk(h, W, w.K, w.chunk, workspace=ws)

    calibration_copy(args, torch, dev)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    del ws
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    idx, val = step()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev)
    gpu_idx, gpu_val = idx.cpu().numpy(), val.double().cpu().numpy()
    del idx, val

    log(f"[bench] timing {args.steps} steps")
    fkl.fkl_timing_reset()
    fkl.fkl_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fkl.fkl_timing_enable(False)
    ktimes = fkl.kernel_times()
    ms_step = elapsed / args.steps * 1e3
    log(f"[bench] {ms_step:.2f} ms/step")
    kernels = {k: {"launches_per_step": n / args.steps, "avg_ms": ms / n,
                   "ms_per_step": ms / args.steps} for k, (n, ms) in ktimes.items()}
    dom = max(ktimes, key=lambda k: ktimes[k][1])
    n_launch, dom_ms = ktimes[dom]
    avg_ms = dom_ms / n_launch
    peak_tf = PEAK_TFLOPS[w.dtype]
    flops_step = 2.0 * w.N * w.d * w.V
    if dom == "k_teacher_logits":
        flops_launch = flops_step / (n_launch / args.steps)
        achieved = flops_launch / (avg_ms * 1e-3) / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": peak_tf,
                    "unit": "TFLOP/s", "frac": achieved / peak_tf,
                    "traffic": load_traffic(dom, w.name), "flops_per_launch": flops_launch,
                    "avg_launch_ms": avg_ms}
    else:
        roofline = {"kernel": dom, "bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": None, "traffic": load_traffic(dom, w.name),
                    "avg_launch_ms": avg_ms}
    if args.no_cpu_baseline:
        base, parity = None, None
    else:
        log("[bench] oracle on the host (cpu_baseline and sampled parity)")
        base, parity = cpu_baseline_topk(inp, gpu_idx, gpu_val, args.cpu_seconds)
    result = {
        "metric": "teacher top-K cache tokens/s + % bf16 MFMA peak",
        "value": w.N * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "N": w.N, "d": w.d, "V": w.V,
                   "K": w.K, "chunk": w.chunk},
        "mfma_frac_step": flops_step / (ms_step * 1e-3) / (peak_tf * 1e12),
        "flops_per_step": flops_step,
        "roofline": roofline,
        "cpu_baseline": base,
        "parity_sampled": parity,
        "peak_hbm_gib": peak / 2**30,
        "peak_hbm_path_gib": (peak - input_bytes) / 2**30,
        "workspace_gib": nb / 2**30,
        "kernels": kernels,
        "source_hash": source_hash(),
    }
    print(json.dumps(result), flush=True)


def cpu_baseline_renorm(inp, gpu_rows, budget_s: float):
    """Time the fp64 oracle of the student-renormalised loss on a bounded
    prefix of the rows (forward + backward of those rows) and compare them."""
    import oracle
    from threadpoolctl import threadpool_info

    w = inp["workload"]

    def run(n):
        t0 = time.perf_counter()
        out = oracle.renorm_forward_backward(inp["hidden"][:n], inp["weight"], inp["topk_idx"][:n],
                                             inp["topk_logit"][:n], w.T)
        return out, time.perf_counter() - t0

    _, t1 = run(64)
    _, t2 = run(128)
    per_row = max((t2 - t1) / 64, 1e-6)
    fixed = max(t1 - 64 * per_row, 0.0)
    n = int((budget_s - fixed) / per_row) // 64 * 64
    n = max(64, min(w.N, n))
    ref, t = run(n)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    errs = {"row_loss_rel_err": float(np.max(np.abs(gpu_rows["row_loss"][:n] - ref["row_loss"]) /
                                             np.maximum(np.abs(ref["row_loss"]), 1.0))),
            "grad_hidden_err_over_max": float(np.abs(gpu_rows["grad_hidden"][:n] -
                                                     ref["grad_hidden"]).max() /
                                              np.abs(ref["grad_hidden"]).max())}
    tol = 1e-3 if w.dtype == "bf16" else 1e-5
    gtol = 2e-2 if w.dtype == "bf16" else 1e-4
    parity = {"rows": n, **errs,
              "ok": bool(errs["row_loss_rel_err"] <= tol and
                         errs["grad_hidden_err_over_max"] <= gtol)}
    base = {"value": n / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {w.N} rows of {w.name}: the renormalised loss forward + "
                      f"backward in fp64 (NumPy), {t:.1f} s; grad_W restricted to those rows"}
    return base, parity


def run_renorm(args, torch, fkl, synth, dev):
    """Benchmark of the student-renormalised loss (fkl_renorm_forward + backward)."""
    w = synth.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name}: N={w.N} d={w.d} V={w.V} K={w.K} T={w.T} {w.dtype}")
    inp = synth.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    h = torch.from_numpy(inp["hidden"]).to(dev).to(dt).contiguous()
    W = torch.from_numpy(inp["weight"]).to(dev).to(dt).contiguous()
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    lg = torch.from_numpy(inp["topk_logit"]).to(dev)
    torch.cuda.synchronize()
    input_bytes = sum(t.numel() * t.element_size() for t in (h, W, idx, lg))
    fw, bw = fkl.fkl_renorm_workspace_size(w.N, w.d, w.V, w.K, dt)
    ws_f = torch.empty(fw, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(bw, dtype=torch.uint8, device=dev)
    gw = torch.empty(w.V, w.d, dtype=torch.float32, device=dev)

    def step():
        out = fkl.fkl_renorm_forward(h, W, idx, lg, w.T, workspace=ws_f)
        gh, _ = fkl.fkl_renorm_backward(h, W, idx, lg, w.T, topk_z=out.topk_z, grad_weight=gw,
                                        workspace=ws_b)
        return out, gh

    calibration_copy(args, torch, dev)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    out, gh = step()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev)
    gpu_rows = {"row_loss": out.row_loss.double().cpu().numpy(),
                "grad_hidden": gh.double().cpu().numpy()}
    del out, gh

    log(f"[bench] timing {args.steps} steps")
    fkl.fkl_timing_reset()
    fkl.fkl_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fkl.fkl_timing_enable(False)
    ktimes = fkl.kernel_times()
    ms_step = elapsed / args.steps * 1e3
    log(f"[bench] {ms_step:.2f} ms/step")
    kernels = {k: {"launches_per_step": n / args.steps, "avg_ms": ms / n,
                   "ms_per_step": ms / args.steps} for k, (n, ms) in ktimes.items()}
    dom = max(ktimes, key=lambda k: ktimes[k][1])
    n_launch, dom_ms = ktimes[dom]
    avg_ms = dom_ms / n_launch
    eb = 2 if w.dtype == "bf16" else 4
    NK = w.N * w.K
    # compulsory bytes per launch: every input byte once, every output byte once (the
    # kernels gather one d-wide row per cached entry; how many of those the caches serve
    # is in the measured traffic)
    compulsory = {
        "k_gather_dot": w.V * w.d * eb + w.N * w.d * eb + NK * 8,
        "k_renorm_grad_h": w.V * w.d * eb + NK * 8 + w.N * w.d * eb,
        "k_rs_chunks": w.N * w.d * eb + NK * 12 + w.V * w.d * 4,
    }
    if dom in compulsory:
        cb = compulsory[dom]
        achieved = cb / (avg_ms * 1e-3) / 1e9
        roofline = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                    "traffic": load_traffic(dom, w.name + "/renorm"), "bytes_per_launch": cb,
                    "avg_launch_ms": avg_ms}
    else:
        roofline = {"kernel": dom, "bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": None, "traffic": None, "avg_launch_ms": avg_ms}
    if args.no_cpu_baseline:
        base, parity = None, None
    else:
        log("[bench] oracle on the host (cpu_baseline and sampled parity)")
        base, parity = cpu_baseline_renorm(inp, gpu_rows, args.cpu_seconds)
    result = {
        "metric": "student-renormalised top-K KL fwd+bwd tokens/s",
        "value": w.N * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "N": w.N, "d": w.d, "V": w.V,
                   "K": w.K, "T": w.T, "ids": w.ids, "loss": "student renormalised over K"},
        "roofline": roofline,
        "cpu_baseline": base,
        "parity_sampled": parity,
        "peak_hbm_gib": peak / 2**30,
        "peak_hbm_path_gib": (peak - input_bytes) / 2**30,
        "workspace_gib": (fw + bw) / 2**30,
        "kernels": kernels,
        "source_hash": source_hash(),
    }
    print(json.dumps(result), flush=True)


def memory_sweep(args, torch, fkl, dev):
    """Peak HBM of one training step (inputs, outputs, workspaces, grad_W, autograd-saved
    tensors) through fused_chunked_kl at S in {4096 .. 65536} tokens, gpt-oss-20B
    student shape (d 2880, V 201088, K 100, chunk 2048, bf16); a linear fit
    peak = a + b S, and the largest single allocation of the step against one
    N x V bf16 matrix."""
    d, V, K, chunk, T = 2880, 201088, 100, 2048, 1.0
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    W = (torch.randn(V, d, device=dev, generator=g) / d ** 0.5).to(torch.bfloat16)
    W.requires_grad_(True)
    points = []
    for S in (4096, 8192, 16384, 32768, 65536):
        h = torch.randn(1, S, d, device=dev, generator=g).to(torch.bfloat16).requires_grad_(True)
        idx = torch.randint(0, V, (1, S, K), device=dev, generator=g, dtype=torch.int32)
        lg = torch.randn(1, S, K, device=dev, generator=g)
        W.grad = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        torch.cuda.memory._record_memory_history(max_entries=100000)
        loss = fkl.fused_chunked_kl(h, W, idx, lg, T=T, chunk=chunk)
        loss.backward()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev)
        snap = torch.cuda.memory._snapshot()
        torch.cuda.memory._record_memory_history(enabled=None)
        largest = 0
        for trace in snap.get("device_traces", []):
            for ev in trace:
                if ev.get("action") == "alloc":
                    largest = max(largest, int(ev.get("size", 0)))
        points.append({"S": S, "peak_bytes": peak, "largest_alloc_bytes": largest,
                       "nxv_bf16_bytes": S * V * 2})
        log(f"[bench] S={S}: peak {peak / 2**30:.3f} GiB, largest allocation "
            f"{largest / 2**30:.3f} GiB (one N x V bf16 matrix: {S * V * 2 / 2**30:.2f} GiB)")
        del h, idx, lg, loss
    xs = np.array([p["S"] for p in points], dtype=np.float64)
    ys = np.array([p["peak_bytes"] for p in points], dtype=np.float64)
    b, a = np.polyfit(xs, ys, 1)
    r2 = 1.0 - float(np.sum((ys - (a + b * xs)) ** 2) / np.sum((ys - ys.mean()) ** 2))
    result = {
        "metric": "peak HBM of one fwd+bwd step vs tokens (linear fit)",
        "config": {"workload": "gptoss20b shape", "d": d, "V": V, "K": K, "chunk": chunk,
                   "dtype": "bf16", "path": "fused_chunked_kl (autograd)"},
        "points": points,
        "fit": {"intercept_bytes": a, "slope_bytes_per_token": b, "r2": r2},
        # the largest buffer is the fp32 grad_W (V x d x 4 bytes) at every S
        "largest_alloc_is_grad_w": bool(all(p["largest_alloc_bytes"] <= V * d * 4 * 1.01
                                            for p in points)),
        "grad_w_fp32_bytes": V * d * 4,
        "data": "synthetic",
    }
    print(json.dumps(result), flush=True)


def vendor_gemm_step(args, torch, w, dev):
    """hipBLASLt (torch.mm) on the plain contractions of one step of the workload, 8 N d V
    flops in bf16 with no exp, log-sum-exp, gather or G formation: (a) per chunk of rows
    over the whole vocabulary (logits, recomputed logits, grad_hidden, grad_W), as a PyTorch
    version of the chunked recompute runs them; (b) the forward per chunk and the backward
    in row blocks x vocabulary slices of the given shape (--vendor-block; 16384 x 16032 is
    what the library plans for long32k). A reference time for the same flops through the
    vendor GEMMs under the same board power limit, not a product path."""
    N, d, V, chunk = w.N, w.d, w.V, w.chunk
    R, S = (int(x) for x in args.vendor_block.split(","))
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    H = torch.randn(N, d, device=dev, generator=g).to(bf)
    W = (torch.randn(V, d, device=dev, generator=g) / d ** 0.5).to(bf)
    Z = torch.empty(chunk, V, device=dev, dtype=bf)
    gh = torch.empty(max(R, chunk), d, device=dev, dtype=bf)
    gw = torch.empty(V, d, device=dev, dtype=bf)
    G = torch.empty(R, S, device=dev, dtype=bf)

    def chunked():
        for r0 in range(0, N, chunk):
            torch.mm(H[r0:r0 + chunk], W.t(), out=Z)
        for r0 in range(0, N, chunk):
            h = H[r0:r0 + chunk]
            torch.mm(h, W.t(), out=Z)
            torch.mm(Z, W, out=gh[:chunk])
            torch.mm(Z.t(), h, out=gw)

    def blocked():
        for r0 in range(0, N, chunk):
            torch.mm(H[r0:r0 + chunk], W.t(), out=Z)
        for r0 in range(0, N, R):
            h = H[r0:r0 + R]
            for v0 in range(0, V, S):
                ws = W[v0:v0 + S]
                gg = G[:h.shape[0], :ws.shape[0]]
                if ws.shape[0] == S and h.shape[0] == R:
                    torch.mm(h, ws.t(), out=gg)
                    torch.mm(gg, ws, out=gh[:R])
                    torch.mm(gg.t(), h, out=gw[v0:v0 + S])
                else:
                    gg = torch.mm(h, ws.t())
                    torch.mm(gg, ws)
                    torch.mm(gg.t(), h)

    out = {}
    for name, fn in (("chunked", chunked), ("blocked", blocked)):
        for _ in range(args.warmup + 1):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / args.steps * 1e3
        tf = 8.0 * N * d * V / ms / 1e9
        out[name] = {"ms_per_step": ms, "tflops": tf, "frac_of_peak": tf / PEAK_TFLOPS["bf16"]}
        log(f"[bench] hipBLASLt {name}: {ms:.2f} ms/step, {tf:.1f} TFLOP/s over 8NdV")
    print(json.dumps({"metric": "vendor GEMM time for the step's contractions",
                      "config": {"workload": w.name, "N": N, "d": d, "V": V, "chunk": chunk,
                                 "block": [R, S], "dtype": "bf16"},
                      "steps": args.steps, "warmup": args.warmup, **out, "data": "synthetic"}),
          flush=True)


def loop_probe(args, torch, fkl, synth, dev):
    """The contraction k-loop away from the board's power limit: the loss on one
    512-row chunk with d 8192 and V 12 288 (bf16) makes the logit kernel
    (k_logits_lse) a launch of 2 x 48 = 96 output tiles of 256 x 256. Each XCD's
    share is rounded up to a round of 32 tiles, so three XCDs run 32 tiles each,
    sharing operand panels in their L2 as at full load, while 96 of the 256 CUs
    draw power; each tile contracts over d = 8192 (128 k-blocks of 64). Reports
    the kernel's rate per busy CU against one CU's dense bf16 MFMA peak at 2.4 GHz
    (4096 flop per clock)."""
    w = synth.small_workload("loop_probe", n=512, d=8192, V=12288, K=100, T=2.0,
                             dtype="bf16", chunk=512, ids="zipf", seed=11)
    inp = synth.make_inputs(w)
    h = torch.from_numpy(inp["hidden"]).to(dev).to(torch.bfloat16).contiguous()
    W = torch.from_numpy(inp["weight"]).to(dev).to(torch.bfloat16).contiguous()
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    lg = torch.from_numpy(inp["topk_logit"]).to(dev)
    fw, bw = fkl.fkl_workspace_size(w.N, w.d, w.V, w.K, w.chunk, torch.bfloat16)
    ws_f = torch.empty(fw, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(bw, dtype=torch.uint8, device=dev)
    gw = torch.empty(w.V, w.d, dtype=torch.float32, device=dev)

    def step():
        out = fkl.fkl_forward(h, W, idx, lg, w.T, w.chunk, workspace=ws_f)
        fkl.fkl_backward(h, W, idx, lg, out.lse, w.T, w.chunk, topk_z=out.topk_z,
                         grad_weight=gw, workspace=ws_b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    fkl.fkl_timing_reset()
    fkl.fkl_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    fkl.fkl_timing_enable(False)
    kt = fkl.kernel_times()
    tiles = -(-w.N // 256) * -(-w.V // 256)
    flops = 2.0 * w.N * w.d * w.V  # per launch: one launch of each per step
    cu_peak = 4096 * 2.4e9 / 1e12
    res = {}
    for k in ("k_logits_lse",):
        n, ms = kt[k]
        avg_ms = ms / n
        per_cu = flops / tiles / (avg_ms * 1e-3) / 1e12
        res[k] = {"launches_per_step": n / args.steps, "avg_launch_ms": avg_ms,
                  "tflops_per_busy_cu": per_cu, "frac_of_cu_peak": per_cu / cu_peak}
    print(json.dumps({
        "metric": "contraction k-loop rate per busy CU, 96 CUs busy",
        "value": res["k_logits_lse"]["tflops_per_busy_cu"], "unit": "TFLOP/s",
        "cu_peak_2p4ghz": cu_peak, "busy_cus": tiles, "k_blocks": w.d // 64,
        "flops_per_launch": flops, "kernels": res, "steps": args.steps,
        "config": {"N": w.N, "d": w.d, "V": w.V, "K": w.K, "chunk": w.chunk, "dtype": w.dtype},
        "source_hash": source_hash()}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="long32k")
    ap.add_argument("--chunk", type=int, default=0,
                    help="rows per pass instead of the workload's (a different memory budget; "
                         "the line then names it and no stored oracle values apply)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--keep-logits", action="store_true",
                    help="time the forward-chunked variant (kept logits, no recompute)")
    ap.add_argument("--options", action="store_true",
                    help="time the loss with its options on: hard labels for every row mixed "
                         "in with alpha 0.5 and a teacher-tail bucket (teacher lse = lse of the "
                         "cached logits + ln 2)")
    ap.add_argument("--memory-sweep", action="store_true",
                    help="measure peak HBM of one step at S = 4096 .. 65536 (gpt-oss-20B student "
                         "shape) and fit it linearly instead of timing")
    ap.add_argument("--teacher-topk", action="store_true",
                    help="time the teacher top-K cache producer instead of the loss "
                         "(workload teacher_llama8b_32k unless --workload names a teacher one)")
    ap.add_argument("--renorm", action="store_true",
                    help="time the student-renormalised loss (both softmaxes over the K "
                         "cached entries; no vocabulary GEMM) instead of the main loss")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time hipBLASLt (torch.mm) on the plain contractions of one step "
                         "(8NdV flops, no exp/LSE/gather) instead of the library")
    ap.add_argument("--vendor-block", default="16384,16032",
                    help="row block and vocabulary slice of the blocked backward for "
                         "--vendor-gemm (the library's plan for long32k)")
    ap.add_argument("--loop-probe", action="store_true",
                    help="the contraction k-loop with 96 CUs busy (below the power limit): "
                         "the logit kernel's rate per CU against one CU's MFMA peak")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, copy this many MiB once on the device (a plain "
                         "copy of known size for calibrating rocprofv3 byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this loss is benchmarked on a single MI355X "
              "(row sharding across GPUs would add one grad_W all-reduce; not built). "
              f"Got --gpus {args.gpus}, WORLD_SIZE {world}.", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_top_kl_amd import fkl, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.teacher_topk:
        run_teacher_topk(args, torch, fkl, synth, dev)
        return
    if args.memory_sweep:
        memory_sweep(args, torch, fkl, dev)
        return
    if args.loop_probe:
        loop_probe(args, torch, fkl, synth, dev)
        return
    w = synth.WORKLOADS[args.workload]
    if args.chunk > 0:
        import dataclasses
        w = dataclasses.replace(w, chunk=args.chunk)
    if args.vendor_gemm:
        vendor_gemm_step(args, torch, w, dev)
        return
    if args.renorm:
        run_renorm(args, torch, fkl, synth, dev)
        return
    log(f"[bench] generating {w.name}: N={w.N} d={w.d} V={w.V} K={w.K} T={w.T} "
        f"chunk={w.chunk} {w.dtype}")
    inp = synth.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    h = torch.from_numpy(inp["hidden"]).to(dev).to(dt).contiguous()
    W = torch.from_numpy(inp["weight"]).to(dev).to(dt).contiguous()
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    lg = torch.from_numpy(inp["topk_logit"]).to(dev)
    torch.cuda.synchronize()
    input_bytes = sum(t.numel() * t.element_size() for t in (h, W, idx, lg))

    keep = args.keep_logits
    fw, bw = fkl.fkl_workspace_size(w.N, w.d, w.V, w.K, w.chunk, dt)
    zbytes = 0
    if keep:
        zbytes, bw = fkl.fkl_keep_sizes(w.N, w.d, w.V, w.K, dt)
    ws_f = torch.empty(fw, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(bw, dtype=torch.uint8, device=dev)
    gw = torch.empty(w.V, w.d, dtype=torch.float32, device=dev)
    zbuf = torch.empty(w.N, fkl.keep_pitch(w.V), dtype=dt, device=dev) if keep else None

    opts = {}
    if args.options:  # the generator's option inputs (those of the oracle fixture)
        o = synth.make_loss_options(w)
        opts = dict(labels=torch.from_numpy(o["labels"]).to(dev), alpha=o["alpha"],
                    teacher_lse=torch.from_numpy(o["teacher_lse"]).to(dev))

    def step():
        if opts:
            res = fkl.fkl_forward_ex(h, W, idx, lg, w.T, w.chunk, keep_logits=zbuf if keep else None,
                                     workspace=ws_f, **opts)
            out, z = res if keep else (res, None)
            gh, _ = fkl.fkl_backward_ex(h, W, idx, lg, out.lse, w.T, w.chunk, topk_z=out.topk_z,
                                        lse1=out.lse1, logits=z, grad_weight=gw, workspace=ws_b,
                                        **opts)
            return out, gh
        if keep:
            out, z = fkl.fkl_forward_keep(h, W, idx, lg, w.T, w.chunk, logits=zbuf, workspace=ws_f)
            gh, _ = fkl.fkl_backward_keep(h, W, idx, lg, out.lse, w.T, z, topk_z=out.topk_z,
                                          grad_weight=gw, workspace=ws_b)
            return out, gh
        out = fkl.fkl_forward(h, W, idx, lg, w.T, w.chunk, workspace=ws_f)
        gh, _ = fkl.fkl_backward(h, W, idx, lg, out.lse, w.T, w.chunk, topk_z=out.topk_z,
                                 grad_weight=gw, workspace=ws_b)
        return out, gh

    calibration_copy(args, torch, dev)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # peak HBM of one step (inputs, outputs, workspaces, grad_W, kept logits)
    del ws_f, ws_b, zbuf
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    ws_f = torch.empty(fw, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(bw, dtype=torch.uint8, device=dev)
    zbuf = torch.empty(w.N, fkl.keep_pitch(w.V), dtype=dt, device=dev) if keep else None
    out, gh = step()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev)
    largest_ws = max(fw, bw)
    gpu_rows = {
        "lse": out.lse.double().cpu().numpy(),
        "row_loss": out.row_loss.double().cpu().numpy(),
        "grad_hidden": gh.double().cpu().numpy(),
    }
    loss_val = out.loss.item()
    gpu_rows["loss"] = loss_val
    parity_fx = fixture_parity(
        w.name + ("-options" if args.options else ""), w, gpu_rows,
        lambda v: gw[torch.as_tensor(v, device=dev)].double().cpu().numpy())
    del out, gh

    log(f"[bench] timing {args.steps} steps")
    fkl.fkl_timing_reset()
    fkl.fkl_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fkl.fkl_timing_enable(False)
    ktimes = fkl.kernel_times()
    log(f"[bench] {elapsed / args.steps * 1e3:.2f} ms/step")

    # four contractions of 2 N d V each (logits, their recompute, grad_hidden,
    # grad_W); the kept-logits variant skips the recompute
    flops_step = (6.0 if keep else 8.0) * w.N * w.d * w.V
    ms_step = elapsed / args.steps * 1e3
    kernels = {k: {"launches_per_step": n / args.steps, "avg_ms": ms / n,
                   "ms_per_step": ms / args.steps} for k, (n, ms) in ktimes.items()}
    kernel_ms_step = sum(v["ms_per_step"] for v in kernels.values())
    dom = max(ktimes, key=lambda k: ktimes[k][1])
    n_launch, dom_ms = ktimes[dom]
    avg_ms = dom_ms / n_launch
    peak_tf = PEAK_TFLOPS[w.dtype]
    traffic_key = w.name + ("/keep" if keep else "")  # stored counters per workload and variant
    if dom in GEMM_KERNELS:
        # each contraction covers all N x V logits once per step
        flops_launch = 2.0 * w.N * w.d * w.V / (n_launch / args.steps)
        achieved = flops_launch / (avg_ms * 1e-3) / 1e12
        traffic = load_traffic(dom, traffic_key)
        roofline = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": peak_tf,
                    "unit": "TFLOP/s", "frac": achieved / peak_tf, "traffic": traffic,
                    "flops_per_launch": flops_launch, "avg_launch_ms": avg_ms}
    else:
        roofline = {"kernel": dom, "bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": None, "traffic": load_traffic(dom, traffic_key),
                    "avg_launch_ms": avg_ms}

    if args.no_cpu_baseline or args.options:
        base, parity = None, None
    else:
        log("[bench] oracle on the host (cpu_baseline and sampled parity)")
        base, parity = cpu_baseline(inp, gpu_rows, args.cpu_seconds)

    tokens_s = w.N * args.steps / elapsed
    result = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "N": w.N, "d": w.d, "V": w.V,
                   "K": w.K, "T": w.T, "chunk": w.chunk, "teacher_ids": w.ids,
                   "variant": "forward-chunked, kept logits" if keep else "fused chunked",
                   "options": "labels (alpha 0.5) + teacher tail" if args.options else None},
        "mfma_frac_step": flops_step / (ms_step * 1e-3) / (peak_tf * 1e12),
        # the same over the summed kernel durations of a step (HIP events), i.e. without gaps
        "kernel_ms_per_step": kernel_ms_step,
        "mfma_frac_kernel_time": flops_step / (kernel_ms_step * 1e-3) / (peak_tf * 1e12),
        "flops_per_step": flops_step,
        "roofline": roofline,
        "cpu_baseline": base,
        "parity_sampled": parity,
        "parity_fixture": parity_fx,
        "peak_hbm_gib": peak / 2**30,
        "peak_hbm_path_gib": (peak - input_bytes) / 2**30,
        "largest_workspace_gib": largest_ws / 2**30,
        "kept_logits_gib": zbytes / 2**30,
        "dense_nxv_fp32_gib": w.N * w.V * 4 / 2**30,
        "loss": loss_val,
        "kernels": kernels,
        "source_hash": source_hash(),
        "context_pages": PAGE_CONTEXT,
    }
    if not math.isfinite(loss_val):
        log("[bench] non-finite loss")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

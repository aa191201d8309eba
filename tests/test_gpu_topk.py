"""Teacher top-K cache on the GPU against the fp64 oracle.

Exact-integer inputs (every logit a small integer, exact in fp32 and fp64,
with many ties) must give the oracle's ids and values bit for bit, including
the tie order. Gaussian inputs give logits that differ from fp64 by fp32
rounding, so there the unique parts are compared (values within the fp32
tolerance, ordering) and the ids are checked to be a valid top-K: distinct,
in range, carrying the logits they claim, and no unselected logit above the
K-th selected one beyond rounding. At full size every row is checked that way
against an independent PyTorch fp32 recomputation of its logits, and sampled
rows against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_top_kl_amd import fkl, synth
from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu


def _upload(inp, device="cuda"):
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    h = torch.from_numpy(np.ascontiguousarray(inp["hidden"])).to(device).to(dt).contiguous()
    w = torch.from_numpy(np.ascontiguousarray(inp["weight"])).to(device).to(dt).contiguous()
    return h, w


def _run(inp, K=None, chunk=None):
    h, w = _upload(inp)
    idx, val = fkl.fkl_teacher_topk(h, w, inp["K"] if K is None else K,
                                    inp["chunk"] if chunk is None else chunk)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.double().cpu().numpy()


EXACT = [
    # name, n, d, V, K, dtype, chunk
    ("int_ragged_bf16", 700, 264, 3001, 100, "bf16", 300),
    ("int_ragged_fp32", 700, 264, 3001, 100, "fp32", 300),
    ("int_small_vocab_bf16", 300, 64, 300, 100, "bf16", 128),   # fewer slices than K
    ("int_k1_bf16", 257, 128, 2000, 1, "bf16", 100),
    ("int_k_equals_v_fp32", 130, 32, 200, 200, "fp32", 64),
    ("int_wide_d_bf16", 300, 1032, 1500, 50, "bf16", 512),
    ("int_k1024_bf16", 64, 64, 5000, 1024, "bf16", 64),
]


@pytest.mark.parametrize("case", EXACT, ids=[c[0] for c in EXACT])
def test_topk_exact_integer_logits(gpu_device, case):
    name, n, d, V, K, dtype, chunk = case
    announce(f"{name}: n={n} d={d} V={V} K={K} {dtype} chunk={chunk}")
    w = synth.small_teacher_workload(name, n=n, d=d, V=V, K=K, dtype=dtype, chunk=chunk,
                                     values="integer", seed=len(name))
    inp = synth.make_teacher_inputs(w)
    idx, val = _run(inp)
    ref_idx, ref_val = oracle.teacher_topk(inp["hidden"], inp["weight"], K)
    np.testing.assert_array_equal(val, ref_val)
    np.testing.assert_array_equal(idx, ref_idx)


def test_topk_all_ties_take_the_exact_path(gpu_device):
    """W = 0: every logit is 0, every row's list overflows and the exact radix
    path must return ids 0..K-1."""
    announce("all-equal logits (W = 0), bf16")
    w = synth.small_teacher_workload("zeros", n=70, d=32, V=3001, K=100, dtype="bf16", chunk=64)
    inp = synth.make_teacher_inputs(w)
    inp["weight"] = np.zeros_like(inp["weight"])
    idx, val = _run(inp)
    np.testing.assert_array_equal(idx, np.tile(np.arange(100, dtype=np.int32), (70, 1)))
    assert np.all(val == 0.0)


def test_topk_is_chunk_invariant(gpu_device):
    announce("chunk invariance, exact integers")
    w = synth.small_teacher_workload("chunks", n=333, d=96, V=2500, K=64, dtype="bf16",
                                     values="integer")
    inp = synth.make_teacher_inputs(w)
    base = _run(inp, chunk=333)
    for chunk in (1, 64, 100, 5000):
        idx, val = _run(inp, chunk=chunk)
        np.testing.assert_array_equal(idx, base[0])
        np.testing.assert_array_equal(val, base[1])


def _check_valid_topk(idx, val, logits, tol):
    """ids form a valid top-K of `logits` (rows) given values computed with
    rounding up to tol: distinct, in range, carrying their logits, sorted, and
    no unselected logit above the K-th selected one beyond rounding."""
    R, K = idx.shape
    V = logits.shape[1]
    assert np.all((idx >= 0) & (idx < V))
    for r in range(R):
        assert len(set(idx[r].tolist())) == K, f"row {r}: repeated ids"
    assert np.all(np.diff(val, axis=1) <= 0), "values not in descending order"
    at = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    assert np.max(np.abs(at - val) / np.maximum(np.abs(at), 1.0)) <= tol
    mask = np.ones_like(logits, dtype=bool)
    np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
    outside = np.where(mask, logits, -np.inf).max(axis=1)
    kth = at.min(axis=1)
    assert np.all(outside <= kth + 2 * tol * np.maximum(np.abs(kth), 1.0)), \
        "an unselected logit exceeds the K-th selected one"


@pytest.mark.parametrize("name,dtype", [("teacher_tiny", "fp32"), ("normal_bf16", "bf16")])
def test_topk_gaussian_against_oracle(gpu_device, name, dtype):
    announce(f"Gaussian teacher inputs: {name}")
    if name == "teacher_tiny":
        w = synth.TEACHER_WORKLOADS[name]
    else:
        w = synth.small_teacher_workload(name, n=600, d=520, V=7000, K=100, dtype=dtype,
                                         chunk=256)
    inp = synth.make_teacher_inputs(w)
    idx, val = _run(inp)
    logits = oracle.teacher_logits(inp["hidden"], inp["weight"])
    ref_idx, ref_val = oracle.topk_rows(logits, w.K)
    tol = 1e-5   # fp32 accumulation against fp64, relative with an absolute floor of 1
    assert np.max(np.abs(val - ref_val) / np.maximum(np.abs(ref_val), 1.0)) <= tol
    _check_valid_topk(idx, val, logits, tol)
    # the k-th largest value is unique: the GPU's k-th id must carry it in fp64
    at = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    assert np.max(np.abs(at - ref_val) / np.maximum(np.abs(ref_val), 1.0)) <= 2 * tol
    differ = int((idx != ref_idx).any(axis=1).sum())
    print(f"    rows ordering near-equal logits differently from fp64: {differ} of {w.N}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["teacher_llama8b_32k", "teacher_gptoss120b_b4_32k"])
def test_topk_full_size(gpu_device, name):
    w = synth.TEACHER_WORKLOADS[name]
    announce(f"full size {name}: N={w.N} d={w.d} V={w.V} K={w.K} chunk={w.chunk} (inputs)")
    inp = synth.make_teacher_inputs(w)
    h, W = _upload(inp)
    announce(f"full size {name}: HIP teacher top-K")
    idx, val = fkl.fkl_teacher_topk(h, W, w.K, w.chunk)
    torch.cuda.synchronize()
    tol = 1e-5
    # every row: validity against PyTorch fp32 logits, 2048 rows at a time
    announce(f"full size {name}: checking all rows against PyTorch fp32 logits")
    Wf = W.float()
    worst_val, worst_gap = 0.0, -np.inf
    for r0 in range(0, w.N, 2048):
        z = torch.matmul(h[r0:r0 + 2048].float(), Wf.t())             # [rows, V] fp32
        ii = idx[r0:r0 + 2048].long()
        vv = val[r0:r0 + 2048]
        at = torch.gather(z, 1, ii)
        worst_val = max(worst_val, float(((at - vv).abs() / at.abs().clamp(min=1.0)).max()))
        assert bool((vv[:, 1:] <= vv[:, :-1]).all()), "values not descending"
        srt, _ = torch.sort(ii, dim=1)
        assert bool((srt[:, 1:] != srt[:, :-1]).all()), "repeated ids"
        z.scatter_(1, ii, -float("inf"))
        outside = z.max(dim=1).values
        kth = vv[:, -1]
        gap = float(((outside - kth) / kth.abs().clamp(min=1.0)).max())
        worst_gap = max(worst_gap, gap)
        del z
    print(f"    all rows: max |value - fp32 logit| rel {worst_val:.2e}, "
          f"max (best unselected - K-th) rel {worst_gap:.2e}", flush=True)
    assert worst_val <= tol
    assert worst_gap <= 2 * tol
    # sampled rows: the oracle's fp64 answer
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, w.N - 1, w.chunk - 1, w.chunk],
                                     rng.choice(w.N, 6, replace=False)]))
    announce(f"full size {name}: oracle on rows {rows.tolist()}")
    logits = oracle.teacher_logits(inp["hidden"][rows], inp["weight"])
    ref_idx, ref_val = oracle.topk_rows(logits, w.K)
    g_idx = idx.cpu().numpy()[rows]
    g_val = val.double().cpu().numpy()[rows]
    assert np.max(np.abs(g_val - ref_val) / np.maximum(np.abs(ref_val), 1.0)) <= tol
    _check_valid_topk(g_idx, g_val, logits, tol)
    at = np.take_along_axis(logits, g_idx.astype(np.int64), axis=1)
    assert np.max(np.abs(at - ref_val) / np.maximum(np.abs(ref_val), 1.0)) <= 2 * tol


@pytest.mark.parametrize("values,dtype,T", [("integer", "bf16", 2.0), ("normal", "fp32", 0.7)])
def test_teacher_lse_output(gpu_device, values, dtype, T):
    announce(f"teacher lse at T={T}: {values} {dtype}")
    w = synth.small_teacher_workload("lse_" + values, n=333, d=136, V=3100, K=50, dtype=dtype,
                                     chunk=128, values=values)
    inp = synth.make_teacher_inputs(w)
    h, W = _upload(inp)
    idx, val, lse = fkl.fkl_teacher_topk_ex(h, W, w.K, w.chunk, T=T)
    idx0, val0 = fkl.fkl_teacher_topk(h, W, w.K, w.chunk)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0) and torch.equal(val, val0)   # the lse changes nothing else
    u = oracle.teacher_logits(inp["hidden"], inp["weight"]) / T
    m = u.max(axis=1)
    ref = m + np.log(np.exp(u - m[:, None]).sum(axis=1))
    got = lse.double().cpu().numpy()
    assert np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1.0)) <= 1e-5

"""HIP path vs the fp64 oracle, element by element, at sizes the oracle
finishes in seconds. Shapes span several 256x256 tiles with ragged tails in
every dimension (rows, vocabulary, hidden size, chunks)."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from sparse_top_kl_amd import fkl, synth
from tests.gpu_helpers import TOL, announce, compare, run_gpu, upload

pytestmark = pytest.mark.gpu


def _oracle(inp, T=None, grad_scale=1.0):
    return oracle.forward_backward(inp["hidden"], inp["weight"], inp["topk_idx"],
                                   inp["topk_logit"], inp["T"] if T is None else T,
                                   grad_scale=grad_scale)


def test_tiny_workload_full_parity(gpu_device):
    """512 tokens, d=512, V=8192, K=100, fp32, chunk 128, T=1."""
    announce("tiny fp32 workload")
    inp = synth.make_inputs("tiny")
    compare(run_gpu(inp), _oracle(inp), "fp32")


CASES = [
    # name, n, d, V, K, T, dtype, chunk, ids
    ("ragged_bf16", 700, 264, 3001, 100, 1.5, "bf16", 300, "uniform"),
    ("ragged_fp32", 700, 264, 3001, 100, 1.5, "fp32", 300, "uniform"),
    ("zipf_T2_bf16", 600, 512, 5000, 100, 2.0, "bf16", 256, "zipf"),
    ("small_vocab_bf16", 300, 64, 300, 100, 1.0, "bf16", 1000, "uniform"),
    ("one_row_fp32", 1, 128, 1000, 7, 0.5, "fp32", 1, "uniform"),
    ("k1_bf16", 257, 128, 2000, 1, 1.0, "bf16", 100, "uniform"),
    ("wide_d_bf16", 300, 1032, 1500, 50, 1.0, "bf16", 128, "uniform"),
    # the largest K the library takes (4096), and a large hidden size
    ("max_k_bf16", 96, 256, 6000, 4096, 1.0, "bf16", 40, "uniform"),
    ("d8192_fp32", 130, 8192, 1100, 64, 2.0, "fp32", 64, "zipf"),
    # a vocabulary smaller than one 256-row tile
    ("tiny_vocab_bf16", 200, 128, 7, 5, 1.5, "bf16", 64, "uniform"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_parity_small_shapes(gpu_device, case):
    name, n, d, V, K, T, dtype, chunk, ids = case
    announce(f"{name}: n={n} d={d} V={V} K={K} T={T} {dtype} chunk={chunk} {ids}")
    w = synth.small_workload(name, n=n, d=d, V=V, K=K, T=T, dtype=dtype, chunk=chunk, ids=ids,
                             seed=zlib.crc32(name.encode()) % 1000)
    inp = synth.make_inputs(w)
    compare(run_gpu(inp), _oracle(inp), dtype)


def test_full_vocab_teacher(gpu_device):
    """K = V: the loss is the full T^2 KL between the two softened distributions."""
    announce("K = V = 256, fp32")
    w = synth.small_workload("kv", n=130, d=32, V=256, K=256, T=1.3, dtype="fp32", chunk=64)
    inp = synth.make_inputs(w)
    compare(run_gpu(inp), _oracle(inp), "fp32")


def test_upstream_gradient_scale(gpu_device):
    announce("grad_loss = -0.37")
    w = synth.small_workload("scale", n=300, d=128, V=1200, K=100, T=1.0, dtype="bf16",
                             chunk=128)
    inp = synth.make_inputs(w)
    compare(run_gpu(inp, grad_scale=-0.37), _oracle(inp, grad_scale=-0.37), "bf16")


def test_minus_inf_teacher_logits(gpu_device):
    announce("-inf teacher entries")
    w = synth.small_workload("ninf", n=280, d=64, V=900, K=40, T=1.0, dtype="fp32", chunk=128)
    inp = synth.make_inputs(w)
    inp["topk_logit"][::3, 20:] = -np.inf
    res = run_gpu(inp)
    assert np.isfinite(res["loss"]) and np.all(np.isfinite(res["grad_w"]))
    compare(res, _oracle(inp), "fp32")


def test_repeated_ids_act_additively(gpu_device):
    announce("repeated ids within rows")
    w = synth.small_workload("dup", n=260, d=64, V=700, K=30, T=1.0, dtype="fp32", chunk=100)
    inp = synth.make_inputs(w)
    inp["topk_idx"][:, 5] = inp["topk_idx"][:, 0]
    inp["topk_idx"][::2, 9] = inp["topk_idx"][::2, 0]
    compare(run_gpu(inp), _oracle(inp), "fp32")


@pytest.mark.parametrize("chunk", [1, 37, 256, 5000])
def test_chunk_invariance(gpu_device, chunk):
    """The chunk only schedules memory: results agree with the oracle for any chunk."""
    announce(f"chunk={chunk}")
    w = synth.small_workload("chunks", n=520, d=128, V=2100, K=100, T=1.0, dtype="bf16",
                             chunk=chunk)
    inp = synth.make_inputs(w)
    compare(run_gpu(inp, chunk=chunk), _oracle(inp), "bf16")


def test_one_hot_probe_gather_is_bit_exact(gpu_device):
    """Hidden rows are unit vectors e_j, so z at an id is exactly W[id, j]:
    the gathered logits must equal the weight entries bit for bit."""
    announce("one-hot probe")
    w = synth.small_workload("onehot", n=512, d=256, V=4096, K=100, T=1.0, dtype="bf16",
                             chunk=200)
    inp = synth.make_inputs(w)
    j = np.arange(512) % 256
    H = np.zeros((512, 256), np.float32)
    H[np.arange(512), j] = 1.0
    inp["hidden"] = H
    h, W, idx, lg = upload(inp)
    out = fkl.fkl_forward(h, W, idx, lg, 1.0, 200)
    got = out.topk_z.cpu().numpy()
    expect = inp["weight"][inp["topk_idx"], j[:, None]].astype(np.float32)
    assert np.array_equal(got.view(np.uint32), expect.view(np.uint32))
    # and the per-row loss uses exactly those ids
    ref = oracle.forward_backward(H, inp["weight"], inp["topk_idx"], inp["topk_logit"], 1.0,
                                  want_grads=False)
    assert np.max(np.abs(out.row_loss.cpu().numpy() - ref["row_loss"]) /
                  np.abs(ref["row_loss"])) < 1e-3


def test_empty_batch(gpu_device):
    announce("N = 0")
    dev = gpu_device
    h = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    W = torch.randn(500, 64, device=dev).to(torch.bfloat16)
    idx = torch.empty(0, 10, dtype=torch.int32, device=dev)
    lg = torch.empty(0, 10, dtype=torch.float32, device=dev)
    out = fkl.fkl_forward(h, W, idx, lg, 1.0, 16)
    assert out.loss.item() == 0.0
    gw = torch.full((500, 64), 7.0, device=dev)
    gh, gw = fkl.fkl_backward(h, W, idx, lg, out.lse, 1.0, 16, grad_weight=gw)
    assert gh.numel() == 0 and torch.count_nonzero(gw).item() == 0


def test_accumulate_grad_w(gpu_device):
    announce("FKL_FLAG_ACCUMULATE_GRAD_W")
    w = synth.small_workload("acc", n=300, d=64, V=800, K=20, T=1.0, dtype="fp32", chunk=128)
    inp = synth.make_inputs(w)
    h, W, idx, lg = upload(inp)
    out = fkl.fkl_forward(h, W, idx, lg, 1.0, 128)
    _, g1 = fkl.fkl_backward(h, W, idx, lg, out.lse, 1.0, 128)
    g2 = g1.clone()
    fkl.fkl_backward(h, W, idx, lg, out.lse, 1.0, 128, grad_weight=g2, accumulate=True)
    torch.testing.assert_close(g2, 2 * g1, rtol=1e-6, atol=1e-7)


def test_recomputed_gather_matches_saved(gpu_device):
    """Backward without the saved gathered logits recomputes them (one dot
    product per teacher id, a different summation order from the logit
    tiles' that produce the saved ones): the gradients agree to rounding, and
    both pass the oracle check."""
    announce("backward with topk_z = NULL")
    w = synth.small_workload("nozk", n=400, d=128, V=1500, K=100, T=1.0, dtype="bf16", chunk=128)
    inp = synth.make_inputs(w)
    h, W, idx, lg = upload(inp)
    out = fkl.fkl_forward(h, W, idx, lg, 1.0, 128)
    a = fkl.fkl_backward(h, W, idx, lg, out.lse, 1.0, 128, topk_z=out.topk_z)
    b = fkl.fkl_backward(h, W, idx, lg, out.lse, 1.0, 128, topk_z=None)
    torch.cuda.synchronize()
    for x, y in zip(a, b):  # G entries at the ids differ by at most one bf16 rounding
        assert (x.double() - y.double()).abs().max() <= 1e-3 * y.double().abs().max()
    ref = _oracle(inp)
    for got, key in ((b[0], "grad_hidden"), (b[1], "grad_w")):
        err = np.abs(got.double().cpu().numpy() - ref[key]).max() / np.abs(ref[key]).max()
        assert err <= TOL["bf16"]["grad"], (key, err)


def test_validate_flag_rejects_bad_ids(gpu_device):
    announce("FKL_FLAG_VALIDATE_IDX")
    w = synth.small_workload("val", n=64, d=64, V=500, K=10, T=1.0, dtype="bf16", chunk=32)
    inp = synth.make_inputs(w)
    inp["topk_idx"][5, 3] = 500
    h, W, idx, lg = upload(inp)
    with pytest.raises(fkl.FklError) as e:
        fkl.fkl_forward(h, W, idx, lg, 1.0, 32, validate=True)
    assert e.value.status == fkl.FKL_E_INDEX
    idx[5, 3] = -1
    lse = torch.zeros(64, device=h.device)
    with pytest.raises(fkl.FklError) as e:
        fkl.fkl_backward(h, W, idx, lg, lse, 1.0, 32, validate=True)
    assert e.value.status == fkl.FKL_E_INDEX


def test_deterministic(gpu_device):
    """No float atomics: two runs are bitwise identical (doubles as a race check)."""
    announce("determinism")
    w = synth.small_workload("det", n=600, d=256, V=3000, K=100, T=1.0, dtype="bf16", chunk=256,
                             ids="zipf")
    inp = synth.make_inputs(w)
    a, b = run_gpu(inp), run_gpu(inp)
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k


def test_autograd_wrapper(gpu_device):
    announce("autograd wrapper")
    w = synth.small_workload("ag", n=2 * 150, d=64, V=900, K=30, T=2.0, dtype="fp32", chunk=64)
    inp = synth.make_inputs(w)
    h, W, idx, lg = upload(inp)
    h3 = h.reshape(2, 150, 64).clone().requires_grad_(True)
    W2 = W.clone().requires_grad_(True)
    loss = fkl.fused_chunked_kl(h3, W2, idx.reshape(2, 150, 30).long(), lg.reshape(2, 150, 30),
                                T=2.0, chunk=64)
    (0.5 * loss).backward()
    ref = oracle.forward_backward(inp["hidden"], inp["weight"], inp["topk_idx"], inp["topk_logit"],
                                  2.0, grad_scale=0.5)
    assert abs(loss.item() - ref["loss"]) / ref["loss"] < 1e-5
    np.testing.assert_allclose(h3.grad.reshape(300, 64).double().cpu().numpy(), ref["grad_hidden"],
                               atol=1e-4 * np.abs(ref["grad_hidden"]).max())
    np.testing.assert_allclose(W2.grad.double().cpu().numpy(), ref["grad_w"],
                               atol=1e-4 * np.abs(ref["grad_w"]).max())


@pytest.mark.parametrize("labels", [False, True])
def test_vocabulary_too_wide_to_bucket(gpu_device, labels):
    """Above 16384 buckets of 512 ids (V > 8 388 608) the logits at the teacher
    ids come from separate dot products and the exact G entries from a
    separate fixup kernel instead of the logit tiles; results still match the
    oracle (with and without hard labels)."""
    w = synth.small_workload("widevocab", n=40, d=16, V=8_400_000 + 1000, K=8, T=2.0,
                             dtype="bf16", chunk=16, seed=41)
    announce(f"vocabulary of {w.V} ids (no pair index), labels={labels}")
    inp = synth.make_inputs(w)
    h, W, idx, lg = upload(inp)
    y = np.random.default_rng(3).integers(0, w.V, size=w.N).astype(np.int32)
    if labels:
        yt = torch.from_numpy(y).to(gpu_device)
        out = fkl.fkl_forward_ex(h, W, idx, lg, w.T, w.chunk, labels=yt, alpha=0.25)
        gh, gw = fkl.fkl_backward_ex(h, W, idx, lg, out.lse, w.T, w.chunk, topk_z=out.topk_z,
                                     labels=yt, alpha=0.25, lse1=out.lse1)
    else:
        out = fkl.fkl_forward(h, W, idx, lg, w.T, w.chunk)
        gh, gw = fkl.fkl_backward(h, W, idx, lg, out.lse, w.T, w.chunk, topk_z=out.topk_z)
    torch.cuda.synchronize()
    opts = dict(labels=y, alpha=0.25) if labels else {}
    ref = oracle.forward_backward(inp["hidden"], inp["weight"], inp["topk_idx"],
                                  inp["topk_logit"], w.T, block_rows=4, **opts)
    gpu = {"loss": out.loss.item(), "lse": out.lse.double().cpu().numpy(),
           "row_loss": out.row_loss.double().cpu().numpy(),
           "topk_z": out.topk_z.double().cpu().numpy(),
           "grad_hidden": gh.double().cpu().numpy()}
    # grad_W: the rows of the ids that occur (teacher ids, labels) and a sample of the rest
    rows = np.unique(np.concatenate([inp["topk_idx"].ravel(), y if labels else [],
                                     np.arange(0, w.V, 997)]).astype(np.int64))
    gpu["grad_w"] = gw[torch.as_tensor(rows, device=gpu_device)].double().cpu().numpy()
    ref = dict(ref, grad_w=ref["grad_w"][rows])
    compare(gpu, ref, "bf16")

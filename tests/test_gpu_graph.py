"""The loss under HIP graph capture: one forward + backward step (fused and
kept-logits paths, with and without options) captured into a graph with
preallocated workspaces and outputs, replayed several times with eager work
and synchronisations in between, and every replay checked bitwise against the
eager result (the kernels are deterministic). The library enqueues no memset
nodes and never synchronises, so a captured step is the same launches. The
student-renormalised loss is captured too, with its workspace scrambled
between replays."""

import numpy as np
import pytest
import torch

from sparse_top_kl_amd import fkl, synth
from tests.gpu_helpers import announce, upload

pytestmark = pytest.mark.gpu


def _setup(dtype):
    w = synth.small_workload("graph", n=700, d=264, V=3001, K=100, T=2.0, dtype=dtype, chunk=256,
                             seed=31)
    inp = synth.make_inputs(w)
    return w, upload(inp)


@pytest.mark.parametrize("keep", [False, True], ids=["fused", "keep"])
@pytest.mark.parametrize("options", [False, True], ids=["plain", "options"])
def test_graph_replays_match_eager(gpu_device, keep, options):
    announce(f"graph capture: keep={keep} options={options}")
    w, (h, W, idx, lg) = _setup("bf16")
    N, d, V, K = h.shape[0], h.shape[1], W.shape[0], idx.shape[1]
    fw, bw = fkl.fkl_workspace_size(N, d, V, K, w.chunk, torch.bfloat16)
    if keep:
        _, bw = fkl.fkl_keep_sizes(N, d, V, K, torch.bfloat16)
    ws_f = torch.empty(fw, dtype=torch.uint8, device=gpu_device)
    ws_b = torch.empty(bw, dtype=torch.uint8, device=gpu_device)
    gw = torch.empty(V, d, dtype=torch.float32, device=gpu_device)
    z = torch.empty(N, fkl.keep_pitch(V), dtype=h.dtype, device=gpu_device) if keep else None
    opts = {}
    if options:
        g = torch.Generator(device=gpu_device)
        g.manual_seed(3)
        opts = dict(labels=torch.randint(0, V, (N,), device=gpu_device, generator=g,
                                         dtype=torch.int32),
                    row_weight=torch.rand(N, device=gpu_device, generator=g), alpha=0.4)

    def step():
        res = fkl.fkl_forward_ex(h, W, idx, lg, w.T, w.chunk, keep_logits=z, workspace=ws_f,
                                 **opts)
        out, zz = res if keep else (res, None)
        gh, _ = fkl.fkl_backward_ex(h, W, idx, lg, out.lse, w.T, w.chunk, topk_z=out.topk_z,
                                    lse1=out.lse1, logits=zz, grad_weight=gw, workspace=ws_b,
                                    **opts)
        return out.loss, out.lse, gh

    loss0, lse0, gh0 = (t.clone() for t in step())
    gw0 = gw.clone()
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loss_g, lse_g, gh_g = step()
    torch.cuda.synchronize()
    for rep in range(4):
        gw.fill_(float("nan"))                   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss_g, loss0), f"replay {rep}: loss"
        assert torch.equal(lse_g, lse0), f"replay {rep}: lse"
        assert torch.equal(gh_g, gh0), f"replay {rep}: grad_hidden"
        assert torch.equal(gw, gw0), f"replay {rep}: grad_W"
        _ = torch.randn(1000, device=gpu_device).sum().item()
    assert np.isfinite(loss0.item())


def test_renorm_graph_replays_match_eager(gpu_device):
    """The student-renormalised loss captured the same way: its counting sort
    clears its counters with fill kernels, so every replay starts from the
    same state and matches the eager step bitwise."""
    announce("graph capture: student-renormalised loss")
    w = synth.small_workload("graph_renorm", n=900, d=256, V=4000, K=100, T=2.0, dtype="bf16",
                             chunk=256, ids="zipf", seed=37)
    h, W, idx, lg = upload(synth.make_inputs(w))
    N, d, V, K = h.shape[0], h.shape[1], W.shape[0], idx.shape[1]
    fw, bw = fkl.fkl_renorm_workspace_size(N, d, V, K, torch.bfloat16)
    ws_f = torch.empty(fw, dtype=torch.uint8, device=gpu_device)
    ws_b = torch.empty(bw, dtype=torch.uint8, device=gpu_device)
    gw = torch.empty(V, d, dtype=torch.float32, device=gpu_device)

    def step():
        out = fkl.fkl_renorm_forward(h, W, idx, lg, w.T, workspace=ws_f)
        gh, _ = fkl.fkl_renorm_backward(h, W, idx, lg, w.T, topk_z=out.topk_z, grad_weight=gw,
                                        workspace=ws_b)
        return out.loss, out.row_loss, gh

    loss0, rl0, gh0 = (t.clone() for t in step())
    gw0 = gw.clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loss_g, rl_g, gh_g = step()
    torch.cuda.synchronize()
    for rep in range(4):
        gw.fill_(float("nan"))
        ws_b.fill_(0xAB)                         # scramble the sort's state between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss_g, loss0), f"replay {rep}: loss"
        assert torch.equal(rl_g, rl0), f"replay {rep}: row_loss"
        assert torch.equal(gh_g, gh0), f"replay {rep}: grad_hidden"
        assert torch.equal(gw, gw0), f"replay {rep}: grad_W"
        _ = torch.randn(1000, device=gpu_device).sum().item()

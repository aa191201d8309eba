"""fkl_forward_noalloc (the forward on the library's static per-device
scratch, for callers that cannot allocate) against fkl_forward (the same
kernels on a caller-provided workspace), through the C ABI: two calls in a
row, the second with a smaller input, each compared bitwise with the
workspace entry point on the same inputs (the same kernels run in the same
order, so the results are identical), and a call whose workspace would not fit
the scratch is refused before anything runs."""

from __future__ import annotations

import pytest
import torch

from sparse_top_kl_amd import fkl, synth
from tests.gpu_helpers import announce, upload

pytestmark = pytest.mark.gpu


def _noalloc(h, W, idx, lg, T, chunk, want_rows=True):
    N, K = idx.shape
    dev = h.device
    out = fkl.ForwardResult(torch.empty((), dtype=torch.float32, device=dev),
                            torch.empty(N, dtype=torch.float32, device=dev),
                            torch.empty(N, dtype=torch.float32, device=dev) if want_rows else None,
                            torch.empty(N, K, dtype=torch.float32, device=dev) if want_rows
                            else None)
    return fkl.fkl_forward_noalloc(h, W, idx, lg, T, chunk, out=out)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_forward_matches_workspace_forward(gpu_device, dtype):
    big = synth.small_workload("noalloc_big", n=3000, d=256, V=5003, K=100, T=2.0, dtype=dtype,
                               chunk=1024, ids="zipf", seed=31)
    small = synth.small_workload("noalloc_small", n=700, d=128, V=2001, K=40, T=1.0,
                                 dtype=dtype, chunk=256, ids="uniform", seed=32)
    for w in (big, small):  # the second call is smaller: stale scratch must not matter
        announce(f"noalloc forward {w.name} {dtype}: N={w.N} d={w.d} V={w.V} K={w.K}")
        inp = synth.make_inputs(w)
        h, W, idx, lg = upload(inp)
        got = _noalloc(h, W, idx, lg, w.T, w.chunk)
        # row_loss and topk_z left to the scratch: the loss must not change
        got_lean = _noalloc(h, W, idx, lg, w.T, w.chunk, want_rows=False)
        ref = fkl.fkl_forward(h, W, idx, lg, w.T, w.chunk)
        torch.cuda.synchronize()
        for field in ("loss", "lse", "row_loss", "topk_z"):
            assert torch.equal(getattr(got, field), getattr(ref, field)), field
        assert torch.equal(got_lean.loss, ref.loss) and torch.equal(got_lean.lse, ref.lse)


def test_noalloc_forward_refuses_a_workspace_beyond_the_scratch(gpu_device):
    announce("noalloc forward: shapes beyond the 64 MiB scratch are refused")
    N, d, V, K = 200000, 64, 128256, 100
    f, _ = fkl.fkl_workspace_size(N, d, V, K, 2048, fkl.FKL_BF16)
    assert f > 64 << 20
    # placeholder (never dereferenced) pointers: the call fails before any launch
    A = 0x10000
    st = fkl.lib().fkl_forward_noalloc(A, A, A, A, 1.0, 2048, N, d, V, K, fkl.FKL_BF16, 0, A, A,
                                      None, None, None)
    assert st == fkl.FKL_E_WORKSPACE
    assert "static scratch" in fkl.fkl_last_error()

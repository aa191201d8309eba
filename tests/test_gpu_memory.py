"""Memory of the fused chunked loss grows linearly with the number of tokens
and no allocation of a step reaches one N x V matrix ("Multiverse Computing
... (iitak.ru)", third paragraph: memory grows linearly with the text length,
without a jump; fifth paragraph: the dense loss no longer runs from 64K
tokens). One training step through the autograd wrapper at S = 4096 .. 32768
tokens, gpt-oss-20B student shape."""

import numpy as np
import pytest
import torch

from sparse_top_kl_amd import fkl
from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
def test_peak_memory_is_linear_in_tokens_and_never_n_by_v(gpu_device):
    d, V, K, chunk = 2880, 201088, 100, 2048
    g = torch.Generator(device=gpu_device)
    g.manual_seed(11)
    W = (torch.randn(V, d, device=gpu_device, generator=g) / d ** 0.5).to(torch.bfloat16)
    W.requires_grad_(True)
    xs, ys = [], []
    for S in (4096, 8192, 16384, 32768):
        announce(f"memory: S={S}")
        h = torch.randn(1, S, d, device=gpu_device, generator=g).to(torch.bfloat16)
        h.requires_grad_(True)
        idx = torch.randint(0, V, (1, S, K), device=gpu_device, generator=g, dtype=torch.int32)
        lg = torch.randn(1, S, K, device=gpu_device, generator=g)
        W.grad = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(gpu_device)
        torch.cuda.memory._record_memory_history(max_entries=100000)
        loss = fkl.fused_chunked_kl(h, W, idx, lg, T=1.0, chunk=chunk)
        loss.backward()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(gpu_device)
        snap = torch.cuda.memory._snapshot()
        torch.cuda.memory._record_memory_history(enabled=None)
        sizes = [int(ev.get("size", 0)) for tr in snap.get("device_traces", []) for ev in tr
                 if ev.get("action") == "alloc"]
        assert sizes, "no allocation events recorded"
        largest = max(sizes)
        print(f"    S={S}: peak {peak / 2**30:.3f} GiB, largest allocation "
              f"{largest / 2**30:.3f} GiB, one N x V bf16 matrix {S * V * 2 / 2**30:.2f} GiB",
              flush=True)
        # the largest buffer is the fp32 grad_W, V x d x 4 bytes, whatever N; nothing
        # N-dependent comes near one N x V matrix
        assert largest <= V * d * 4 * 1.01
        if S >= 8192:          # from here one N x V bf16 matrix exceeds grad_W
            assert largest < S * V * 2
        assert np.isfinite(loss.item())
        xs.append(S)
        ys.append(peak)
        del h, idx, lg, loss
    b, a = np.polyfit(np.array(xs, float), np.array(ys, float), 1)
    pred = a + b * np.array(xs, float)
    r2 = 1 - np.sum((np.array(ys) - pred) ** 2) / np.sum((np.array(ys) - np.mean(ys)) ** 2)
    print(f"    fit: {a / 2**30:.3f} GiB + {b / 1024:.2f} KiB/token, R^2 = {r2:.6f}", flush=True)
    assert r2 > 0.999
    # per token at least hidden + grad_hidden (bf16) and the teacher entries;
    # far below one vocabulary row of logits (V * 2 bytes = 393 KiB)
    assert 4 * d + 8 * K <= b <= 64 * 1024

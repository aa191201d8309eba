"""The C ABI without a GPU: symbols, constants, workspace planning, validation.

Validation happens before anything is enqueued, so calls that must fail can
be made here with placeholder (never dereferenced) device addresses.
"""

import ctypes
import os
import re

import pytest

from sparse_top_kl_amd import fkl

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "fkl.h")


def _declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fkl_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = fkl.lib()
    names = _declared_functions()
    assert {"fkl_forward", "fkl_backward", "fkl_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in fkl.h but not exported"


def test_binding_covers_every_declared_function():
    for n in _declared_functions():
        assert callable(getattr(fkl, n)), n


def test_abi_version_and_status_strings():
    assert fkl.fkl_abi_version() == 1
    assert fkl.fkl_status_string(fkl.FKL_OK) == "ok"
    assert fkl.fkl_status_string(fkl.FKL_E_WORKSPACE) == "workspace too small"
    assert fkl.fkl_status_string(12345) == "unknown status"


def pair_index_bytes(N, V, K):
    """The teacher-id pair index both passes build: per tile of 256 rows, one
    offset per 32-id vocabulary bucket (+1) and room for 256 (K + 1) packed
    pairs (the +1: a hard label per row)."""
    tiles = (N + 255) // 256
    return tiles * ((V + 31) // 32 + 1) * 4 + tiles * 256 * (K + 1) * 4


def test_workspace_is_bounded_by_chunk_times_vocab_and_never_rows_times_vocab():
    d, V, K, chunk = 3072, 128256, 100, 2048
    Vpad = (V + 7) // 8 * 8
    for N in (8192, 32768, 65536, 131072):
        f, b = fkl.fkl_workspace_size(N, d, V, K, chunk, fkl.FKL_BF16)
        # forward: per-chunk partials (one float2 per row and 128-wide slice, at T and at
        # temperature 1 for the cross-entropy option) + per-row scratch + the pair index
        assert f <= 2 * chunk * ((V + 255) // 256) * 2 * 8 + N * (8 + 4 * K) + \
            pair_index_bytes(N, V, K) + (1 << 16)
        # backward: one logit-gradient block within the chunk x V budget (its rows padded
        # by fewer than 64 elements to whole 128-byte lines), plus per-row scratch of a
        # row block (fp32 grad_hidden accumulator, teacher coefficients, the constants of
        # the exact entries; up to four fp32 accumulators when grad_hidden's contraction is
        # split) and the pair index
        assert b <= chunk * Vpad * 2 + min(N, 1 << 16) * (16 * d + 16 * K + 16 + 128) + \
            pair_index_bytes(N, V, K) + (1 << 16)
        if N >= 8 * chunk:
            assert b < N * V * 2 / 4  # far below one dense bf16 N x V matrix
    # a larger chunk buys a larger block
    _, b1 = fkl.fkl_workspace_size(32768, d, V, K, 1024, fkl.FKL_BF16)
    _, b2 = fkl.fkl_workspace_size(32768, d, V, K, 4096, fkl.FKL_BF16)
    assert b2 > 1.5 * b1


def test_backward_row_blocks_keep_hidden_rows_within_32_bit_offsets():
    """grad_W reads a row block's hidden rows through 32-bit buffer offsets, so
    rows * d * element size stays below 2 GiB even when the chunk x V budget
    would allow more rows (small vocabulary, large hidden size). The backward
    workspace holds, per row of a block, the G row (padded to 64 elements),
    the fp32 grad_hidden accumulator, two K-entry coefficient rows and seven
    scalars, so the planned block size can be read back from its size."""
    for dtype, eb in ((fkl.FKL_BF16, 2), (fkl.FKL_F32, 4)):
        N, d, V, K = 200000, 8192, 1024, 16
        _, b = fkl.fkl_workspace_size(N, d, V, K, N, dtype)
        # G row, grad_hidden accumulator, K-entry coefficient rows (two of K, two of
        # K + 1) and seven scalars; the pair index depends on N only
        per_row = ((V + 63) // 64 * 64) * eb + 4 * d + 8 * K + 8 * (K + 1) + 7 * 4
        rows = (b - pair_index_bytes(N, V, K)) // per_row
        assert rows * d * eb < 2 ** 31, (dtype, rows)
        assert rows >= 256
        # a smaller batch still fits in one block
        n_small = (2 ** 31 - 2 ** 20) // (d * eb) // 2
        _, b_small = fkl.fkl_workspace_size(n_small, d, V, K, n_small, dtype)
        assert (b_small - pair_index_bytes(n_small, V, K)) // per_row == n_small


def test_workspace_size_rejects_bad_shapes():
    with pytest.raises(fkl.FklError) as e:
        fkl.fkl_workspace_size(10, 12, 100, 5, 4, fkl.FKL_BF16)
    assert e.value.status == fkl.FKL_E_UNSUPPORTED
    with pytest.raises(fkl.FklError) as e:
        fkl.fkl_workspace_size(10, 16, 100, 101, 4, fkl.FKL_BF16)
    assert e.value.status == fkl.FKL_E_ARG
    with pytest.raises(fkl.FklError) as e:
        fkl.fkl_workspace_size(10, 16, 100, 5, 0, fkl.FKL_BF16)
    assert e.value.status == fkl.FKL_E_ARG
    with pytest.raises(fkl.FklError) as e:
        fkl.fkl_workspace_size(10, 16, 100, 5, 4, 7)
    assert e.value.status == fkl.FKL_E_UNSUPPORTED


# placeholder addresses: 16-byte aligned, never dereferenced on the error paths
A = 0x10000


def _fwd(**over):
    args = dict(hidden=A, weight=A, idx=A, logit=A, T=1.0, chunk=4, N=10, d=16, V=100, K=5,
                dtype=fkl.FKL_BF16, flags=0, loss=A, lse=A, row_loss=None, topk_z=None,
                ws=A, ws_bytes=1 << 40, stream=None)
    args.update(over)
    return fkl.lib().fkl_forward(*args.values())


def _bwd(**over):
    args = dict(hidden=A, weight=A, idx=A, logit=A, lse=A, topk_z=None, grad_loss=None, T=1.0,
                chunk=4, N=10, d=16, V=100, K=5, dtype=fkl.FKL_BF16, flags=0, gh=A, gw=A, ws=A,
                ws_bytes=1 << 40, stream=None)
    args.update(over)
    return fkl.lib().fkl_backward(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(hidden=None), fkl.FKL_E_ARG),
    (dict(loss=None), fkl.FKL_E_ARG),
    (dict(lse=None), fkl.FKL_E_ARG),
    (dict(hidden=A + 2), fkl.FKL_E_ARG),
    (dict(lse=A + 2), fkl.FKL_E_ARG),
    (dict(T=0.0), fkl.FKL_E_ARG),
    (dict(T=-1.0), fkl.FKL_E_ARG),
    (dict(T=float("nan")), fkl.FKL_E_ARG),
    (dict(T=float("inf")), fkl.FKL_E_ARG),
    (dict(chunk=0), fkl.FKL_E_ARG),
    (dict(N=-1), fkl.FKL_E_ARG),
    (dict(K=0), fkl.FKL_E_ARG),
    (dict(K=101), fkl.FKL_E_ARG),
    (dict(d=12), fkl.FKL_E_UNSUPPORTED),
    (dict(dtype=5), fkl.FKL_E_UNSUPPORTED),
    (dict(flags=1), fkl.FKL_E_ARG),
    (dict(ws_bytes=16), fkl.FKL_E_WORKSPACE),
])
def test_forward_validation(over, code):
    assert _fwd(**over) == code
    assert fkl.fkl_last_error() != ""


@pytest.mark.parametrize("over,code", [
    (dict(gh=None), fkl.FKL_E_ARG),
    (dict(gw=None), fkl.FKL_E_ARG),
    (dict(lse=None), fkl.FKL_E_ARG),
    (dict(gw=A + 4), fkl.FKL_E_ARG),
    (dict(grad_loss=A + 1), fkl.FKL_E_ARG),
    (dict(T=0.0), fkl.FKL_E_ARG),
    (dict(flags=4), fkl.FKL_E_ARG),
    (dict(K=5000, V=10000), fkl.FKL_E_UNSUPPORTED),
    (dict(ws_bytes=1024), fkl.FKL_E_WORKSPACE),
])
def test_backward_validation(over, code):
    assert _bwd(**over) == code


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(fkl, "_lib", None)
    monkeypatch.setattr(fkl, "LIB_PATH", "/nonexistent/libfkl.so")
    with pytest.raises(RuntimeError, match="missing"):
        fkl.lib()


# ----------------------------------------------------------- kept-logits variant

def test_keep_sizes_are_rows_times_padded_vocab():
    for N, d, V, K, dt, eb in ((32768, 3072, 128256, 100, fkl.FKL_BF16, 2),
                               (131072, 2880, 201088, 100, fkl.FKL_BF16, 2),
                               (512, 512, 8192, 100, fkl.FKL_F32, 4),
                               (7, 16, 1001, 5, fkl.FKL_BF16, 2)):
        z, b = fkl.fkl_keep_sizes(N, d, V, K, dt)
        assert z == N * fkl.keep_pitch(V) * eb
        assert fkl.keep_pitch(V) % 64 == 0 and 0 <= fkl.keep_pitch(V) - V < 64
        # per-row coefficients (p, z at the ids, seven scalars) and the fp32 grad_hidden rows
        assert N * (8 * K + 28 + 4 * d) <= b <= N * (8 * K + 28 + 4 * d) + 11 * 256


def test_keep_sizes_reject_a_vocabulary_too_large_to_keep():
    # 256 kept rows must fit in 2 GiB: V * 2 bytes * 256 > 2^31 from V ~ 4.19M on
    with pytest.raises(fkl.FklError) as e:
        fkl.fkl_keep_sizes(16, 8, 5_000_000, 5, fkl.FKL_BF16)
    assert e.value.status == fkl.FKL_E_UNSUPPORTED
    fkl.fkl_keep_sizes(16, 8, 4_000_000, 5, fkl.FKL_BF16)


def _fwd_keep(**over):
    args = dict(hidden=A, weight=A, idx=A, logit=A, T=1.0, chunk=4, N=10, d=16, V=100, K=5,
                dtype=fkl.FKL_BF16, flags=0, loss=A, lse=A, row_loss=None, topk_z=None,
                logits=A, logits_bytes=1 << 40, ws=A, ws_bytes=1 << 40, stream=None)
    args.update(over)
    return fkl.lib().fkl_forward_keep(*args.values())


def _bwd_keep(**over):
    args = dict(hidden=A, weight=A, idx=A, logit=A, lse=A, topk_z=None, grad_loss=None, T=1.0,
                N=10, d=16, V=100, K=5, dtype=fkl.FKL_BF16, flags=0, logits=A,
                logits_bytes=1 << 40, gh=A, gw=A, ws=A, ws_bytes=1 << 40, stream=None)
    args.update(over)
    return fkl.lib().fkl_backward_keep(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(logits=None), fkl.FKL_E_ARG),
    (dict(logits=A + 8), fkl.FKL_E_ARG),
    (dict(logits_bytes=10 * 128 * 2 - 2), fkl.FKL_E_WORKSPACE),
    (dict(hidden=None), fkl.FKL_E_ARG),
    (dict(T=0.0), fkl.FKL_E_ARG),
    (dict(flags=1), fkl.FKL_E_ARG),
    (dict(ws_bytes=16), fkl.FKL_E_WORKSPACE),
    (dict(V=5_000_000, d=8), fkl.FKL_E_UNSUPPORTED),
])
def test_forward_keep_validation(over, code):
    assert _fwd_keep(**over) == code
    assert fkl.fkl_last_error() != ""


@pytest.mark.parametrize("over,code", [
    (dict(logits=None), fkl.FKL_E_ARG),
    (dict(logits=A + 4), fkl.FKL_E_ARG),
    (dict(logits_bytes=10 * 128 * 2 - 2), fkl.FKL_E_WORKSPACE),
    (dict(gh=None), fkl.FKL_E_ARG),
    (dict(lse=None), fkl.FKL_E_ARG),
    (dict(grad_loss=A + 1), fkl.FKL_E_ARG),
    (dict(flags=4), fkl.FKL_E_ARG),
    (dict(ws_bytes=1024), fkl.FKL_E_WORKSPACE),
])
def test_backward_keep_validation(over, code):
    assert _bwd_keep(**over) == code
    assert fkl.fkl_last_error() != ""


def test_keep_buffers_one_byte_short_are_rejected():
    """One byte less than fkl_keep_sizes reports, for either buffer, is an error."""
    z, b = fkl.fkl_keep_sizes(10, 16, 100, 5, fkl.FKL_BF16)
    assert _bwd_keep(logits_bytes=z - 1) == fkl.FKL_E_WORKSPACE
    assert _bwd_keep(ws_bytes=b - 1) == fkl.FKL_E_WORKSPACE


# ------------------------------------------------------------- teacher top-K

def test_topk_workspace_holds_one_chunk_of_fp32_logits():
    for N, d, V, K, chunk in ((32768, 4096, 128256, 100, 2048), (100, 64, 1000, 10, 4096)):
        b = fkl.fkl_topk_workspace_size(N, d, V, K, chunk, fkl.FKL_BF16)
        rows = min(N, chunk)
        ld = (rows + 63) // 64 * 64
        lt = V * ld * 4
        part = ((V + 255) // 256) * 2 * ld * 8     # teacher lse partials (optional output)
        assert lt <= b <= lt + part + rows * (4 * ((V + 127) // 128 + 4) + 8 + 2048 * 8) + 7 * 256


def _topk(**over):
    args = dict(hidden=A, weight=A, N=10, d=16, V=100, K=5, chunk=4, dtype=fkl.FKL_BF16,
                flags=0, idx=A, val=A, ws=A, ws_bytes=1 << 40, stream=None)
    args.update(over)
    return fkl.lib().fkl_teacher_topk(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(hidden=None), fkl.FKL_E_ARG),
    (dict(idx=None), fkl.FKL_E_ARG),
    (dict(val=A + 2), fkl.FKL_E_ARG),
    (dict(weight=A + 8), fkl.FKL_E_ARG),
    (dict(K=0), fkl.FKL_E_ARG),
    (dict(K=101), fkl.FKL_E_ARG),
    (dict(K=1025, V=5000), fkl.FKL_E_UNSUPPORTED),
    (dict(d=12), fkl.FKL_E_UNSUPPORTED),
    (dict(chunk=0), fkl.FKL_E_ARG),
    (dict(flags=1), fkl.FKL_E_ARG),
    (dict(ws_bytes=64), fkl.FKL_E_WORKSPACE),
])
def test_teacher_topk_validation(over, code):
    assert _topk(**over) == code
    assert fkl.fkl_last_error() != ""


def _fwd_ex(opts, **over):
    args = dict(hidden=A, weight=A, idx=A, logit=A, T=2.0, chunk=4, N=10, d=16, V=100, K=5,
                dtype=fkl.FKL_BF16, flags=0, opts=opts, loss=A, lse=A, row_loss=None, topk_z=None,
                ws=A, ws_bytes=1 << 40, stream=None)
    args.update(over)
    return fkl.lib().fkl_forward_ex(*args.values())


def _bwd_ex(opts, **over):
    args = dict(hidden=A, weight=A, idx=A, logit=A, lse=A, topk_z=None, grad_loss=None, T=2.0,
                chunk=4, N=10, d=16, V=100, K=5, dtype=fkl.FKL_BF16, flags=0, opts=opts, gh=A,
                gw=A, ws=A, ws_bytes=1 << 40, stream=None)
    args.update(over)
    return fkl.lib().fkl_backward_ex(*args.values())


def test_loss_options_validation():
    import ctypes
    ok = fkl.LossOptions(A, A, 0.5, A)
    bad_alpha = fkl.LossOptions(None, A, float("nan"), A)
    bad_align = fkl.LossOptions(A + 2, None, 0.5, None)
    no_lse1 = fkl.LossOptions(None, A, 0.5, None)
    assert _fwd_ex(ctypes.byref(bad_alpha)) == fkl.FKL_E_ARG
    assert _fwd_ex(ctypes.byref(bad_align)) == fkl.FKL_E_ARG
    assert _bwd_ex(ctypes.byref(bad_alpha)) == fkl.FKL_E_ARG
    # with labels and T != 1 the backward needs the forward's lse1 ...
    assert _bwd_ex(ctypes.byref(no_lse1)) == fkl.FKL_E_ARG
    assert "lse1" in fkl.fkl_last_error()
    # ... but not at T = 1 (same softmax); these stop at the workspace check
    assert _bwd_ex(ctypes.byref(no_lse1), T=1.0, ws_bytes=16) == fkl.FKL_E_WORKSPACE
    assert _bwd_ex(ctypes.byref(ok), ws_bytes=16) == fkl.FKL_E_WORKSPACE


# ------------------------------------------------ student-renormalised loss

def test_renorm_workspace_is_linear_in_pairs_and_never_rows_times_vocab():
    for N, d, V, K in ((32768, 3072, 128256, 100), (131072, 2880, 201088, 100), (300, 64, 999, 7)):
        f, b = fkl.fkl_renorm_workspace_size(N, d, V, K, fkl.FKL_BF16)
        NK = N * K
        # forward: gathered logits + per-row losses
        assert NK * 4 <= f <= NK * 4 + N * 4 + 4 * 256
        # backward: coefficients, gathered logits, sorted pairs (row, id, coefficient), the
        # hidden rows in 64-column slices, per-id starts, at most 256 MiB
        # of per-block id counters (or one block), and two d-wide partials per chunk of 1920
        # sorted pairs; for the ids
        # summed by a dense product (as many as one round of 256 x 256 tiles of its hot x d
        # output takes), per-id slots, their coefficients for at most 256 MiB of rows and their
        # product (one copy per row split of the product)
        counters = max(256 << 20, V * 4)
        chunks = NK // 1920 + 1
        hot_max = min(2048, max(256, (256 // -(-d // 256)) * 256))
        rows = min(N, (256 << 20) // (hot_max * 2))
        groups = -(-hot_max // 2048) * -(-(-(-d // 256)) // 4)
        splits = min(1 if groups >= 8 else 8 // groups, max(1, rows // 1024))
        hot = rows * hot_max * 2 + splits * hot_max * d * 4 + hot_max * 4 + V * 4
        slices = N * -(-d // 64) * 64 * 2
        assert 5 * NK * 4 + slices + (2 * V + 1) * 4 + hot - rows * hot_max * 2 <= b
        assert b <= (5 * NK * 4 + slices + (2 * V + 1) * 4 + counters + chunks * 2 * d * 4 + hot
                     + 24 * 256)
        assert b < N * V * 2 / 4 or N < 4096


def _rfwd(**over):
    args = dict(hidden=A, weight=A, idx=A, logit=A, T=1.0, N=10, d=16, V=100, K=5,
                dtype=fkl.FKL_BF16, flags=0, row_weight=None, loss=A, row_loss=None, topk_z=None,
                ws=A, ws_bytes=1 << 40, stream=None)
    args.update(over)
    return fkl.lib().fkl_renorm_forward(*args.values())


def _rbwd(**over):
    args = dict(hidden=A, weight=A, idx=A, logit=A, topk_z=None, grad_loss=None, T=1.0, N=10,
                d=16, V=100, K=5, dtype=fkl.FKL_BF16, flags=0, row_weight=None, gh=A, gw=A, ws=A,
                ws_bytes=1 << 40, stream=None)
    args.update(over)
    return fkl.lib().fkl_renorm_backward(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(hidden=None), fkl.FKL_E_ARG),
    (dict(loss=None), fkl.FKL_E_ARG),
    (dict(hidden=A + 2), fkl.FKL_E_ARG),
    (dict(row_weight=A + 2), fkl.FKL_E_ARG),
    (dict(topk_z=A + 2), fkl.FKL_E_ARG),
    (dict(T=0.0), fkl.FKL_E_ARG),
    (dict(T=float("nan")), fkl.FKL_E_ARG),
    (dict(K=0), fkl.FKL_E_ARG),
    (dict(K=101), fkl.FKL_E_ARG),
    (dict(K=1025, V=5000), fkl.FKL_E_UNSUPPORTED),
    (dict(d=8200), fkl.FKL_E_UNSUPPORTED),
    (dict(d=12), fkl.FKL_E_UNSUPPORTED),
    (dict(N=1 << 22, K=1000, V=5000), fkl.FKL_E_UNSUPPORTED),
    (dict(flags=1), fkl.FKL_E_ARG),
    (dict(ws_bytes=16), fkl.FKL_E_WORKSPACE),
])
def test_renorm_forward_validation(over, code):
    assert _rfwd(**over) == code
    assert fkl.fkl_last_error() != ""


@pytest.mark.parametrize("over,code", [
    (dict(gh=None), fkl.FKL_E_ARG),
    (dict(gw=None), fkl.FKL_E_ARG),
    (dict(gw=A + 4), fkl.FKL_E_ARG),
    (dict(grad_loss=A + 1), fkl.FKL_E_ARG),
    (dict(logit=None), fkl.FKL_E_ARG),
    (dict(T=-2.0), fkl.FKL_E_ARG),
    (dict(flags=4), fkl.FKL_E_ARG),
    (dict(K=2000, V=5000), fkl.FKL_E_UNSUPPORTED),
    (dict(ws_bytes=1024), fkl.FKL_E_WORKSPACE),
])
def test_renorm_backward_validation(over, code):
    assert _rbwd(**over) == code
    assert fkl.fkl_last_error() != ""


def test_noalloc_forward_refuses_before_touching_a_device():
    """fkl_forward_noalloc checks its arguments and that the forward workspace
    fits its static 64 MiB scratch before any device call (so it fails the
    same way without a GPU)."""
    call = fkl.lib().fkl_forward_noalloc
    ok = dict(hidden=A, weight=A, idx=A, logit=A, T=1.0, chunk=2048, N=200000, d=64, V=128256,
              K=100, dtype=fkl.FKL_BF16, flags=0, loss=A, lse=A, row_loss=None, topk_z=None,
              stream=None)
    assert call(*ok.values()) == fkl.FKL_E_WORKSPACE
    assert "static scratch" in fkl.fkl_last_error()
    assert call(*dict(ok, loss=None).values()) == fkl.FKL_E_ARG
    assert call(*dict(ok, T=0.0).values()) == fkl.FKL_E_ARG
    assert call(*dict(ok, d=12).values()) == fkl.FKL_E_UNSUPPORTED

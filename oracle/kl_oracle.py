"""fp64 reference of the top-K KL distillation loss and its gradients.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
imports this module and this module never imports the HIP library.

What is computed, and where it comes from
-----------------------------------------
The pages describe the method in words only (their formulas did not survive
extraction). The quantities below are the plain definition that the fused
chunked method reorganises exactly:

* "Multiverse Computing ... (iitak.ru), third paragraph" and
  "Wissensdestillation mit deutlich weniger GPU-Speicher", section
  "KL-Verlust wird in Blöcken berechnet": the loss consumes the student's
  final hidden states together with its output projection, works through the
  sequence block by block, sums each block's contribution and drops the block,
  and recomputes the blocks in the backward pass. Chunking is therefore a
  memory schedule, not a change of the function: this oracle has no chunks.
* Same pages, first and second paragraphs: the teacher is a cache of the
  top-100 (token id, logit) pairs per position.
* "Дистилляция и сжатие моделей" (ml-book.com), section "Как это работает:
  мягкие метки и температура": logits are divided by the temperature T before
  the softmax, the KL divergence is taken between the two softened
  distributions, and the KL term is multiplied by T squared.

Extensions (options of the loss): the same page, same section, says the
student's total loss mixes the KL term with the ordinary cross-entropy on the
true labels. With hard labels y_r (a label < 0 marks a row without one) and a
mixing weight alpha, and per-row weights w_r (padding masks, mean
reductions), the loss becomes

    loss = sum_r w_r * (a_kl * T^2 * KL_r + a_ce * CE_r),
    CE_r = lse1_r - z_r,y_r,   lse1_r = log sum_v exp(z_rv)   (temperature 1)

with a_kl = alpha, a_ce = 1 - alpha when labels are given and a_kl = 1,
a_ce = 0 otherwise (readings: the formula itself was stripped from the page;
the cross-entropy is taken at temperature 1, as in the classic recipe the
page describes, and the mixture is convex). Rows with w_r = 0 contribute
nothing, whatever their teacher logits.

Teacher tail (an alternative to renormalising the teacher over its K
entries, which the pages leave open): given the teacher's full-vocabulary
log-sum-exp at T per row (``teacher_lse``, cached beside its top-K), the
teacher probabilities of the cached ids are p_k = exp(l_k / T - teacher_lse)
(not renormalised), the rest of the teacher's mass is one tail bucket
p_tail = 1 - sum_k p_k, the student's is 1 - S with S = sum_k q_(idx_k), and
the KL is taken between these K + 1 buckets:

    KL_r = sum_k p_k (log p_k - log q_(idx_k)) + p_tail (log p_tail - log(1 - S)).

Readings taken where the pages are silent (each listed in the design notes):
forward KL(p_t || p_s); the teacher softmax is renormalised over its K cached
entries; the student is normalised over the full vocabulary; tokens are summed
(not averaged); duplicate ids inside a row act additively; a teacher logit of
-inf contributes probability 0 and a zero term.

Per row r, with upstream scale s:

    z_r      = h_r . W_store^T                  (W stored [V, d], as nn.Linear)
    lse_r    = log sum_v exp(z_rv / T)
    a_rk     = l_rk / T,  log p_rk = a_rk - logsumexp_k(a_r.),  p_rk = exp(..)
    row_loss = T^2 * sum_k p_rk * (log p_rk - (z_r,idx_rk / T - lse_r))
    q_rv     = exp(z_rv / T - lse_r)
    P_rv     = sum_k p_rk [idx_rk == v]
    G_rv     = s * T * (q_rv * sum_k p_rk - P_rv)      (= d loss / d z_rv)
    grad_h_r = G_r . W_store        grad_W_store = G^T . H
"""

from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def student_logits(hidden, w_store) -> np.ndarray:
    """z = hidden . W, with W given in its stored [V, d] layout.

    The loss takes the hidden states and the output projection, not logits
    ("Wissensdestillation ...", section "KL-Verlust wird in Blöcken berechnet":
    the output projection is fused into the loss).
    """
    return _f64(hidden) @ _f64(w_store).T


def logsumexp_rows(u) -> np.ndarray:
    """Natural-log log-sum-exp of each row, shifted by the row maximum."""
    u = _f64(u)
    m = np.max(u, axis=1, keepdims=True)
    return (m + np.log(np.sum(np.exp(u - m), axis=1, keepdims=True)))[:, 0]


def teacher_log_probs(topk_logit, T: float):
    """Teacher softmax at temperature T, renormalised over the K cached entries.

    Temperature division before the softmax: "Дистилляция и сжатие моделей",
    section "Как это работает: мягкие метки и температура". Renormalising over
    the K cached entries is this implementation's reading (the pages do not
    say what happens to the tail beyond the top-K). Entries equal to -inf get
    probability 0 (log-probability -inf); a row needs one finite entry.

    Returns (log_p, p), both [N, K] fp64.
    """
    a = _f64(topk_logit) / float(T)
    m = np.max(a, axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("every teacher row needs at least one finite logit")
    with np.errstate(invalid="ignore"):
        shifted = a - m  # -inf stays -inf
    log_norm = np.log(np.sum(np.exp(shifted), axis=1, keepdims=True))
    log_p = shifted - log_norm
    p = np.exp(log_p)
    return log_p, p


def forward_backward(hidden, w_store, topk_idx, topk_logit, T: float,
                     grad_scale: float = 1.0, want_grads: bool = True,
                     block_rows: int = 128, row_weight=None, labels=None,
                     alpha: float = 1.0, teacher_lse=None) -> dict:
    """Loss, per-row pieces and gradients of the top-K KL loss, in fp64.

    hidden [N, d], w_store [V, d] (any float dtype; upcast exactly),
    topk_idx [N, K] integer ids in [0, V), topk_logit [N, K].
    ``block_rows`` only bounds host memory; the result does not depend on it
    beyond rounding (rows are independent).

    Returns a dict with ``loss`` (float, math.fsum of rows), ``row_loss`` [N],
    ``lse`` [N] (natural log of sum exp(z/T)), ``topk_z`` [N, K] (raw z at
    the ids), ``lse1`` [N] (log sum exp(z), temperature 1), and when
    ``want_grads``: ``grad_hidden`` [N, d] and ``grad_w`` [V, d] (stored
    layout). ``row_weight`` [N], ``labels`` [N] and ``alpha`` as in the module
    docstring.
    """
    h = _f64(hidden)
    w = _f64(w_store)
    idx = np.asarray(topk_idx)
    n, d = h.shape
    v = w.shape[0]
    if w.shape[1] != d or idx.shape != np.shape(topk_logit) or idx.shape[0] != n:
        raise ValueError("shape mismatch")
    if idx.size and (idx.min() < 0 or idx.max() >= v):
        raise ValueError("token id out of range")
    T = float(T)
    wr = np.ones(n) if row_weight is None else _f64(row_weight).reshape(n)
    if labels is None:
        a_kl, a_ce, y = 1.0, 0.0, np.full(n, -1)
    else:
        a_kl, a_ce, y = float(alpha), 1.0 - float(alpha), np.asarray(labels).reshape(n)
        if np.any(y >= v):
            raise ValueError("label out of range")
    # rows with weight 0 contribute nothing: give them finite placeholder
    # teacher logits so that a padding row of -inf entries stays harmless
    tl = np.array(topk_logit, dtype=np.float64)
    tl[wr == 0] = 0.0
    if teacher_lse is None:
        log_p, p = teacher_log_probs(tl, T)
        p_tail = np.zeros(n)
    else:
        # the cached ids' share of the teacher's full distribution, and the rest
        tlse = _f64(teacher_lse).reshape(n)
        tlse = np.where(wr == 0, 0.0, tlse)
        with np.errstate(invalid="ignore"):
            log_p = tl / T - tlse[:, None]
        p = np.exp(log_p)
        p_tail = np.maximum(0.0, 1.0 - p.sum(axis=1))

    row_loss = np.zeros(n)
    lse = np.zeros(n)
    lse1 = np.zeros(n)
    topk_z = np.zeros(idx.shape)
    grad_h = np.zeros((n, d)) if want_grads else None
    grad_w = np.zeros((v, d)) if want_grads else None

    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        z = h[r0:r1] @ w.T                     # [R, V]
        u = z / T
        lse_b = logsumexp_rows(u)
        zk = np.take_along_axis(z, idx[r0:r1], axis=1)
        log_ps = zk / T - lse_b[:, None]       # student log-prob at the ids
        pb, lpb = p[r0:r1], log_p[r0:r1]
        # p * (log p - log p_s), with the 0 * log 0 = 0 convention
        term = np.where(pb > 0, pb * (np.where(pb > 0, lpb, 0.0) - log_ps), 0.0)
        ptb = p_tail[r0:r1]
        S = np.exp(log_ps).sum(axis=1)                     # student mass on the cached ids
        one_s = np.maximum(1.0 - S, 1e-300)
        with np.errstate(divide="ignore"):
            tail = np.where(ptb > 0, ptb * (np.log(np.where(ptb > 0, ptb, 1.0)) - np.log(one_s)),
                            0.0)
        kl = T * T * (term.sum(axis=1) + tail)
        lse1_b = logsumexp_rows(z)
        yb = y[r0:r1]
        has = yb >= 0
        zy = np.where(has, np.take_along_axis(z, np.where(has, yb, 0)[:, None], axis=1)[:, 0], 0.0)
        ce = np.where(has, lse1_b - zy, 0.0)
        wb = wr[r0:r1]
        row_loss[r0:r1] = np.where(wb != 0, wb * (a_kl * kl + a_ce * ce), 0.0)
        lse[r0:r1] = lse_b
        lse1[r0:r1] = lse1_b
        topk_z[r0:r1] = zk
        if want_grads:
            q = np.exp(u - lse_b[:, None])
            P = np.zeros_like(q)
            rows = np.repeat(np.arange(r1 - r0), idx.shape[1])
            np.add.at(P, (rows, idx[r0:r1].ravel()), pb.ravel())
            G = a_kl * T * (q * pb.sum(axis=1, keepdims=True) - P)
            if teacher_lse is not None:
                # d/dz of p_tail (log p_tail - log(1 - S)): T p_tail (Q - q S) / (1 - S),
                # Q_v = q_v times the number of cached ids equal to v
                M = np.zeros_like(q)
                np.add.at(M, (rows, idx[r0:r1].ravel()), 1.0)
                G = G + a_kl * T * (ptb / one_s)[:, None] * (M * q - q * S[:, None])
            if a_ce != 0.0:
                q1 = np.exp(z - lse1_b[:, None])
                E = np.zeros_like(q1)
                E[np.arange(r1 - r0)[has], yb[has]] = 1.0
                G = G + a_ce * (q1 * has[:, None] - E)
            G = grad_scale * wb[:, None] * G
            grad_h[r0:r1] = G @ w
            grad_w += G.T @ h[r0:r1]

    out = {
        "loss": math.fsum(row_loss.tolist()),
        "row_loss": row_loss,
        "lse": lse,
        "lse1": lse1,
        "topk_z": topk_z,
    }
    if want_grads:
        out["grad_hidden"] = grad_h
        out["grad_w"] = grad_w
    return out


def brute_force(hidden, w_store, topk_idx, topk_logit, T: float,
                grad_scale: float = 1.0, row_weight=None, labels=None,
                alpha: float = 1.0, teacher_lse=None) -> dict:
    """The same quantities written as scalar Python loops (tiny inputs only).

    No NumPy arithmetic: every sum is ``math.fsum`` over Python floats, so a
    vectorisation slip in ``forward_backward`` (a transposed operand, a wrong
    axis) cannot hide behind the same slip here.
    """
    H = [[float(x) for x in row] for row in np.asarray(hidden, dtype=np.float64)]
    W = [[float(x) for x in row] for row in np.asarray(w_store, dtype=np.float64)]
    I = [[int(x) for x in row] for row in np.asarray(topk_idx)]
    L = [[float(x) for x in row] for row in np.asarray(topk_logit, dtype=np.float64)]
    n, d, v = len(H), len(H[0]), len(W)
    T = float(T)
    Wr = [1.0] * n if row_weight is None else [float(x) for x in row_weight]
    Y = [-1] * n if labels is None else [int(x) for x in labels]
    a_kl, a_ce = (1.0, 0.0) if labels is None else (float(alpha), 1.0 - float(alpha))
    row_loss, lse_all, grad_h = [], [], []
    grad_w = [[0.0] * d for _ in range(v)]
    contrib_w = [[[] for _ in range(d)] for _ in range(v)]
    for r in range(n):
        z = [math.fsum(H[r][j] * W[c][j] for j in range(d)) for c in range(v)]
        mz = max(z)
        lse = mz / T + math.log(math.fsum(math.exp((zc - mz) / T) for zc in z))
        lse1 = mz + math.log(math.fsum(math.exp(zc - mz) for zc in z))
        if Wr[r] == 0.0:
            row_loss.append(0.0)
            lse_all.append(lse)
            grad_h.append([0.0] * d)
            continue
        a = [x / T for x in L[r]]
        if teacher_lse is None:
            ma = max(a)
            ln = ma + math.log(math.fsum(math.exp(x - ma) for x in a if x != -math.inf))
        else:
            ln = float(teacher_lse[r])
        pt = [0.0 if x == -math.inf else math.exp(x - ln) for x in a]
        terms = []
        for k, c in enumerate(I[r]):
            if pt[k] > 0.0:
                terms.append(pt[k] * ((a[k] - ln) - (z[c] / T - lse)))
        ptail, S = 0.0, 0.0
        if teacher_lse is not None:
            ptail = max(0.0, 1.0 - math.fsum(pt))
            S = math.fsum(math.exp(z[c] / T - lse) for c in I[r])
            if ptail > 0.0:
                terms.append(ptail * (math.log(ptail) - math.log(1.0 - S)))
        ce = (lse1 - z[Y[r]]) if Y[r] >= 0 else 0.0
        row_loss.append(Wr[r] * (a_kl * T * T * math.fsum(terms) + a_ce * ce))
        lse_all.append(lse)
        sp = math.fsum(pt)
        G = []
        for c in range(v):
            q = math.exp(z[c] / T - lse)
            Pc = math.fsum(pt[k] for k, cc in enumerate(I[r]) if cc == c)
            g = a_kl * T * (q * sp - Pc)
            if ptail > 0.0:
                mult = sum(1 for cc in I[r] if cc == c)
                g += a_kl * T * ptail * (mult * q - q * S) / (1.0 - S)
            if Y[r] >= 0:
                g += a_ce * (math.exp(z[c] - lse1) - (1.0 if c == Y[r] else 0.0))
            G.append(grad_scale * Wr[r] * g)
        grad_h.append([math.fsum(G[c] * W[c][j] for c in range(v)) for j in range(d)])
        for c in range(v):
            for j in range(d):
                contrib_w[c][j].append(G[c] * H[r][j])
    for c in range(v):
        for j in range(d):
            grad_w[c][j] = math.fsum(contrib_w[c][j])
    return {
        "loss": math.fsum(row_loss),
        "row_loss": np.array(row_loss),
        "lse": np.array(lse_all),
        "grad_hidden": np.array(grad_h),
        "grad_w": np.array(grad_w),
    }

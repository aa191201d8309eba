"""fp64 reference of the student-renormalised top-K KL loss (a loss option).

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
imports this module and this module never imports the HIP library.

What is computed, and where it comes from
-----------------------------------------
The teacher is a cache of its K most probable (id, logit) pairs per position
("Multiverse Computing ... (iitak.ru)", third paragraph; "Wissensdestillation
mit deutlich weniger GPU-Speicher", section "Teacher-Ausgaben einmalig
zwischenspeichern"), softened by the temperature T, with the KL term taken
between the softened distributions and multiplied by T squared
("Дистилляция и сжатие моделей" (ml-book.com), section "Как это работает:
мягкие метки и температура").

The pages leave open what happens outside the K cached entries. The main loss
(``kl_oracle``) renormalises the teacher over its K entries and normalises the
student over the whole vocabulary. This module is the other plain reading:
both distributions are renormalised over the same K entries, so the loss
needs the student's logits at the cached ids only (no vocabulary-wide
log-sum-exp). Entries whose teacher logit is -inf are padding: they take part
in neither softmax. Duplicate ids inside a row act as separate entries.

Per row r, with V_r the entries of finite teacher logit, row weight w_r and
upstream scale s:

    a_k      = l_rk / T,     log p_k = a_k - logsumexp_{j in V_r} a_j
    u_k      = z_r,idx_rk / T = (h_r . W_store[idx_rk]) / T
    log q_k  = u_k - logsumexp_{j in V_r} u_j
    row_loss = w_r T^2 sum_{k in V_r} p_k (log p_k - log q_k)
    G_rk     = s w_r T (q_k sum_{j in V_r} p_j - p_k)   (= d loss / d z_r,idx_rk; 0 off V_r)
    grad_h_r = sum_k G_rk W_store[idx_rk]
    grad_W_store[v] = sum over (r, k) with idx_rk = v of G_rk h_r

Rows with w_r = 0 contribute nothing, whatever their teacher logits; any
other row needs one finite teacher logit.
"""

from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _masked_log_softmax(x, valid):
    """log softmax of each row of x over the entries where ``valid`` holds
    (-inf elsewhere). Rows without a valid entry give -inf everywhere."""
    xm = np.where(valid, x, -np.inf)
    m = np.max(xm, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        log_norm = np.log(np.sum(np.where(valid, np.exp(xm - m), 0.0), axis=1, keepdims=True))
        return np.where(valid, xm - m - log_norm, -np.inf)


def renorm_forward_backward(hidden, w_store, topk_idx, topk_logit, T: float,
                            grad_scale: float = 1.0, row_weight=None,
                            want_grads: bool = True) -> dict:
    """Loss, per-row pieces and gradients of the student-renormalised loss.

    hidden [N, d], w_store [V, d] (any float dtype; upcast exactly),
    topk_idx [N, K] integer ids in [0, V), topk_logit [N, K].
    Returns ``loss`` (math.fsum of the rows), ``row_loss`` [N], ``topk_z``
    [N, K] (raw z at the ids), ``coef`` [N, K] (G) and, when ``want_grads``,
    ``grad_hidden`` [N, d] and ``grad_w`` [V, d] (stored layout).
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
    lg = _f64(topk_logit)
    valid = np.isfinite(lg)
    live = wr != 0
    if np.any(live & ~valid.any(axis=1)):
        raise ValueError("every weighted row needs at least one finite teacher logit")
    valid &= live[:, None]                      # zero-weight rows: no entries at all

    zk = np.einsum("nd,nkd->nk", h, w[idx]) if idx.size else np.zeros(idx.shape)
    log_p = _masked_log_softmax(lg / T, valid)
    log_q = _masked_log_softmax(zk / T, valid)
    p = np.where(valid, np.exp(log_p), 0.0)
    q = np.where(valid, np.exp(log_q), 0.0)
    term = np.where(valid, p * (np.where(valid, log_p, 0.0) - np.where(valid, log_q, 0.0)), 0.0)
    row_loss = np.where(live, wr * T * T * term.sum(axis=1), 0.0)
    coef = grad_scale * wr[:, None] * T * (q * p.sum(axis=1, keepdims=True) - p)
    coef = np.where(valid, coef, 0.0)
    out = {"loss": math.fsum(row_loss.tolist()), "row_loss": row_loss, "topk_z": zk,
           "coef": coef}
    if want_grads:
        out["grad_hidden"] = np.einsum("nk,nkd->nd", coef, w[idx]) if idx.size else np.zeros((n, d))
        gw = np.zeros((v, d))
        np.add.at(gw, idx.ravel(), coef.ravel()[:, None] * np.repeat(h, idx.shape[1], axis=0))
        out["grad_w"] = gw
    return out


def renorm_brute_force(hidden, w_store, topk_idx, topk_logit, T: float,
                       grad_scale: float = 1.0, row_weight=None) -> dict:
    """The same loss written as scalar Python loops (tiny inputs only): every
    sum is math.fsum over Python floats, so a vectorisation slip in
    ``renorm_forward_backward`` cannot hide behind the same slip here."""
    H = [[float(x) for x in row] for row in np.asarray(hidden, dtype=np.float64)]
    W = [[float(x) for x in row] for row in np.asarray(w_store, dtype=np.float64)]
    I = [[int(x) for x in row] for row in np.asarray(topk_idx)]
    L = [[float(x) for x in row] for row in np.asarray(topk_logit, dtype=np.float64)]
    n, d, v = len(H), len(H[0]), len(W)
    T = float(T)
    Wr = [1.0] * n if row_weight is None else [float(x) for x in row_weight]
    row_loss, grad_h = [], []
    contrib = [[[] for _ in range(d)] for _ in range(v)]
    for r in range(n):
        ks = [k for k in range(len(I[r])) if math.isfinite(L[r][k])] if Wr[r] != 0 else []
        if not ks:
            row_loss.append(0.0)
            grad_h.append([0.0] * d)
            continue
        z = {k: math.fsum(H[r][j] * W[I[r][k]][j] for j in range(d)) for k in ks}
        ma = max(L[r][k] / T for k in ks)
        sa = math.fsum(math.exp(L[r][k] / T - ma) for k in ks)
        mu = max(z[k] / T for k in ks)
        su = math.fsum(math.exp(z[k] / T - mu) for k in ks)
        p = {k: math.exp(L[r][k] / T - ma) / sa for k in ks}
        q = {k: math.exp(z[k] / T - mu) / su for k in ks}
        kl = math.fsum(p[k] * (math.log(p[k]) - math.log(q[k])) for k in ks if p[k] > 0)
        row_loss.append(Wr[r] * T * T * kl)
        psum = math.fsum(p.values())
        g = {k: grad_scale * Wr[r] * T * (q[k] * psum - p[k]) for k in ks}
        grad_h.append([math.fsum(g[k] * W[I[r][k]][j] for k in ks) for j in range(d)])
        for k in ks:
            for j in range(d):
                contrib[I[r][k]][j].append(g[k] * H[r][j])
    grad_w = [[math.fsum(contrib[vv][j]) for j in range(d)] for vv in range(v)]
    return {"loss": math.fsum(row_loss), "row_loss": np.array(row_loss),
            "grad_hidden": np.array(grad_h), "grad_w": np.array(grad_w)}

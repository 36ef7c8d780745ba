"""Gated non-causal softmax anchor attention, fp64 (test infrastructure only).

Source: SANA-Video 2.0 abstract and summary (method section, hybrid attention):
one layer in four is a gated softmax "anchor" that restores full-rank token
interaction. The pages give no formula beyond naming it a gated softmax
attention; the readings are the textbook scaled dot-product attention with
scale 1/sqrt(D), no RoPE, and the same sigmoid output gate as the linear
layers:

    l_ij = scale * q_i . k_j
    p_ij = exp(l_ij - max_j l_ij) / sum_j exp(l_ij - max_j l_ij)
    o_i  = sigmoid(g_i) * sum_j p_ij v_j
"""
from __future__ import annotations

import numpy as np


def _sigmoid(x):
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def softmax_anchor(q, k, v, g=None, scale: float | None = None, rows=None, row_block: int = 256):
    """Softmax attention of (B, N, H, D) inputs over all keys, fp64.

    ``rows`` selects the query tokens whose outputs are computed (all if None).
    Query rows are independent, so they are processed ``row_block`` at a time
    to bound memory; every row still sees every key.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.empty((B, len(rows), H, D))
    for b in range(B):
        for h in range(H):
            kh = k[b, :, h, :]
            vh = v[b, :, h, :]
            for r0 in range(0, len(rows), row_block):
                rr = rows[r0:r0 + row_block]
                logits = scale * (q[b, rr, h, :] @ kh.T)
                logits = logits - logits.max(axis=1, keepdims=True)
                p = np.exp(logits)
                p = p / p.sum(axis=1, keepdims=True)
                out[b, r0:r0 + len(rr), h, :] = p @ vh
    if g is not None:
        out = _sigmoid(np.asarray(g, dtype=np.float64)[:, rows]) * out
    return out


def softmax_anchor_lse(q, k, scale: float | None = None, rows=None, row_block: int = 256):
    """Natural-log normaliser of every query row, lse_i = log sum_j exp(scale q_i . k_j), fp64.

    Returned as (B, H, len(rows)). With it the weights are p_ij = exp(l_ij - lse_i),
    which is what a backward pass reuses instead of recomputing the forward.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, N, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            kh = k[b, :, h, :]
            for r0 in range(0, len(rows), row_block):
                rr = rows[r0:r0 + row_block]
                logits = scale * (q[b, rr, h, :] @ kh.T)
                m = logits.max(axis=1)
                out[b, h, r0:r0 + len(rr)] = m + np.log(np.exp(logits - m[:, None]).sum(axis=1))
    return out


def softmax_anchor_block_sparse(q, k, v, blocks, counts, g=None, scale: float | None = None, q_block: int = 128,
                                k_block: int = 64, rows=None):
    """Block-sparse gated softmax anchor, fp64 (parity unpinned against the pages).

    The pages name a sparse anchor (SANA-Video 2.0 summary, efficiency
    paragraph: the last stage of its engine) without its pattern; the reading
    is a caller-given block pattern. Query row i lies in query block
    r = i // q_block; for each (b, h, r) the first counts[b, h, r] entries of
    blocks[b, h, r, :] name key blocks m, and the row attends to the keys
    m * k_block <= j < min(N, (m + 1) * k_block) of every named block (entries
    outside [0, ceil(N / k_block)) name nothing). With K_r that key set:

        o_i = sigmoid(g_i) * sum_{j in K_r} softmax_{j in K_r}(scale * q_i . k_j) v_j

    and o_i = 0 when K_r is empty. Named blocks are taken as a set.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    blocks = np.asarray(blocks)
    counts = np.asarray(counts)
    B, N, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    n_kb = -(-N // k_block)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.zeros((B, len(rows), H, D))
    for b in range(B):
        for h in range(H):
            for idx, i in enumerate(rows):
                r = i // q_block
                named = {int(m) for m in blocks[b, h, r, :counts[b, h, r]] if 0 <= m < n_kb}
                keys = np.array(sorted(j for m in named for j in range(m * k_block, min(N, (m + 1) * k_block))),
                                dtype=np.int64)
                if keys.size == 0:
                    continue
                logits = scale * (k[b, keys, h, :] @ q[b, i, h, :])
                p = np.exp(logits - logits.max())
                p = p / p.sum()
                out[b, idx, h, :] = p @ v[b, keys, h, :]
    if g is not None:
        out = _sigmoid(np.asarray(g, dtype=np.float64)[:, rows]) * out
    return out


def softmax_anchor_backward(q, k, v, do, g=None, scale: float | None = None, row_block: int = 256):
    """Gradients of the gated softmax anchor, fp64.

    Differentiates the definition at the top of this module by hand. With
    s_i = sigmoid(g_i) (1 without a gate), y_i = sum_j p_ij v_j and the
    upstream gradient dO:

        dG_i   = dO_i * y_i * s_i * (1 - s_i),   dY_i = dO_i * s_i
        dP_ij  = dY_i . v_j,                     Delta_i = dY_i . y_i = sum_j p_ij dP_ij
        dL_ij  = p_ij (dP_ij - Delta_i)          (gradient of the logit l_ij)
        dq_i   = scale sum_j dL_ij k_j,  dk_j = scale sum_i dL_ij q_i,  dv_j = sum_i p_ij dY_i

    Query rows are taken ``row_block`` at a time; the key-side sums add the
    blocks in order. Returns (dq, dk, dv, dg); dg is None without a gate.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, N, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    s = np.ones_like(q) if g is None else _sigmoid(np.asarray(g, dtype=np.float64))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dg = None if g is None else np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, :, h, :], v[b, :, h, :]
            for r0 in range(0, N, row_block):
                rr = slice(r0, min(N, r0 + row_block))
                logits = scale * (q[b, rr, h, :] @ kh.T)
                p = np.exp(logits - logits.max(axis=1, keepdims=True))
                p = p / p.sum(axis=1, keepdims=True)
                y = p @ vh
                sh = s[b, rr, h, :]
                if g is not None:
                    dg[b, rr, h, :] = do[b, rr, h, :] * y * sh * (1.0 - sh)
                dy = do[b, rr, h, :] * sh
                dp = dy @ vh.T
                delta = np.sum(dy * y, axis=1, keepdims=True)
                dl = p * (dp - delta)
                dq[b, rr, h, :] = scale * (dl @ kh)
                dk[b, :, h, :] += scale * (dl.T @ q[b, rr, h, :])
                dv[b, :, h, :] += p.T @ dy
    return dq, dk, dv, dg

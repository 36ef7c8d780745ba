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

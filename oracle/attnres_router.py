"""Block attention-residual (AttnRes) router, fp64 (test infrastructure only).

Source: SANA-Video 2.0 summary (hyper.ai), method section, subsection on hybrid
attention and block residuals, the router equation: layer l's input is a
softmax-weighted sum over its depth sources v_i (token embedding, completed
block summaries, running partial sum), with weights

    alpha_i = softmax_i( (w + phi(t))^T RMSNorm(v_i) )
    h       = sum_i alpha_i v_i

Readings: RMSNorm(v) = v / sqrt(mean_c v_c^2 + eps) with eps inside the root
and no learned gain (a gain folds into w); phi(t) is optional (the same
summary reports that dropping the timestep input from the router helped), and
is per batch element; the weighted sum uses the raw sources.
"""
from __future__ import annotations

import numpy as np


def attnres_route(sources, w, phi_t=None, eps: float = 1e-6):
    """Route S sources of shape (B, T, C); w is (C,), phi_t is (B, C) or None.

    Returns (h, alpha) with h of shape (B, T, C) and alpha of shape (B, T, S).
    """
    vs = [np.asarray(s, dtype=np.float64) for s in sources]
    B, T, C = vs[0].shape
    u = np.broadcast_to(np.asarray(w, dtype=np.float64), (B, C)).copy()
    if phi_t is not None:
        u = u + np.asarray(phi_t, dtype=np.float64)
    logits = []
    for v in vs:
        rms = np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
        normed = v / rms
        logits.append(np.einsum("btc,bc->bt", normed, u))
    logits = np.stack(logits, axis=-1)  # (B, T, S)
    logits = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(logits)
    alpha = e / e.sum(axis=-1, keepdims=True)
    h = np.zeros((B, T, C))
    for i, v in enumerate(vs):
        h += alpha[..., i:i + 1] * v
    return h, alpha

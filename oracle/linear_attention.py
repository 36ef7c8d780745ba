"""ReLU-kernel linear attention with RoPE after the ReLU, fp64 (test infrastructure only).

Source: SANA-Video notes, section 3.2 (the output equation and the
``linear_attention_with_rope`` pseudocode) and section 3.4 (the causal
equation, the constant-memory cache and Algorithm 1). Gate: the SANA-Video 2.0
abstract and summary describe the linear layers as gated without giving the
form; the reading is a sigmoid of a gate tensor G of O's shape, multiplied in
after normalisation.

Definition (per batch b and head h, tokens j = 1..N):

    phi(x)  = max(x, 0)
    a_i     = RoPE_i(phi(q_i)),   c_j = RoPE_j(phi(k_j))
    KV      = sum_j c_j^T v_j                  (D x D)
    ksum    = sum_j phi(k_j)                   (D, no RoPE)
    o_i     = (a_i KV) / (phi(q_i) . ksum + eps)
    o_i    <- sigmoid(g_i) * o_i               (if a gate is given)

eps is added to the denominator (the equation shows none; the pseudocode adds
it). The denominator carries no RoPE, so it is >= 0 and o_i is finite.
"""
from __future__ import annotations

import numpy as np

from .rope3d import Rope3D, rope3d_angles, rope3d_rotate


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    # 1 / (1 + exp(-x)), written to avoid overflow for large |x|
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def _features(q, k, rope: Rope3D | None):
    """Feature maps of the queries and keys: (phi(q), phi(k), R phi(q), R phi(k)).

    phi is the ReLU; R is the 3D rotation of each token, applied after phi. The
    unrotated features feed the denominator, the rotated ones the numerator.
    """
    pos_q = np.maximum(q, 0.0)
    pos_k = np.maximum(k, 0.0)
    if rope is None:
        return pos_q, pos_k, pos_q, pos_k
    if rope.n_tokens != q.shape[1]:
        raise ValueError("RoPE grid does not match the token count")
    theta = rope3d_angles(rope)
    return pos_q, pos_k, rope3d_rotate(pos_q, theta), rope3d_rotate(pos_k, theta)


def linear_attention(q, k, v, g=None, rope: Rope3D | None = None, eps: float = 1e-6,
                     rows=None, return_state: bool = False):
    """Bidirectional linear attention of (B, N, H, D) inputs, fp64.

    For every batch b and head h the D x D state is the sum over all tokens of
    the outer products c_j^T v_j (c_j the rotated key features), formed as one
    product of the stacked rows, and the key sum adds the unrotated features.
    Each requested row then reads both: o_i = (a_i S) / (phi(q_i) . z + eps),
    and the gate multiplies in last.

    ``rows`` optionally selects the token indices whose outputs are returned
    (the state always sums over all N tokens). With ``return_state`` the
    (KV, ksum) pair of shape (B, H, D, D) and (B, H, D) is returned as well.
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, N, H, D = q.shape
    phi_q, phi_k, rot_q, rot_k = _features(q, k, rope)
    sel = np.arange(N) if rows is None else np.asarray(rows)
    state = np.zeros((B, H, D, D))
    zsum = np.zeros((B, H, D))
    out = np.zeros((B, len(sel), H, D))
    for b in range(B):
        for h in range(H):
            c = rot_k[b, :, h, :]
            state[b, h] = c.T @ v[b, :, h, :]
            zsum[b, h] = phi_k[b, :, h, :].sum(axis=0)
            # per-row products as plain sums, so a row's value does not depend
            # on which other rows are requested
            num = np.einsum("id,de->ie", rot_q[b, sel, h, :], state[b, h])
            den = np.einsum("id,d->i", phi_q[b, sel, h, :], zsum[b, h]) + eps
            out[b, :, h, :] = num / den[:, None]
    if g is not None:
        out = _sigmoid(g[:, sel]) * out
    if return_state:
        return out, state, zsum
    return out


def linear_attention_chunked(q, k, v, chunk_tokens: int, g=None, rope: Rope3D | None = None,
                             eps: float = 1e-6, kv_in=None, ksum_in=None, rows=None):
    """Block-causal linear attention with a carried constant-memory state, fp64.

    Chunk c holds tokens [c*L, min((c+1)*L, N)). Following the causal equation
    (the own term is included) and Algorithm 1's cache update, the cache
    (sum of states, sum of phi(K)) is advanced by each chunk in order, and the
    chunk's tokens read the cache that already includes their own chunk:

        KV_c   = KV_in   + sum_{j in chunks 0..c} c_j^T v_j
        ksum_c = ksum_in + sum_{j in chunks 0..c} phi(k_j)
        o_i    = (a_i KV_c(i)) / (phi(q_i) . ksum_c(i) + eps)

    Returns (out, kv_out, ksum_out) with kv_out, ksum_out the cache after the
    last chunk. ``rows`` optionally restricts the returned outputs.
    """
    if chunk_tokens <= 0:
        raise ValueError("chunk_tokens must be positive")
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, N, H, D = q.shape
    q_relu, k_relu, q_rope, k_rope = _features(q, k, rope)
    kv = np.zeros((B, H, D, D)) if kv_in is None else np.array(kv_in, dtype=np.float64)
    k_sum = np.zeros((B, H, D)) if ksum_in is None else np.array(ksum_in, dtype=np.float64)
    out = np.zeros((B, N, H, D))
    for start in range(0, N, chunk_tokens):
        stop = min(N, start + chunk_tokens)
        kv = kv + np.einsum("bnhd,bnhe->bhde", k_rope[:, start:stop], v[:, start:stop])
        k_sum = k_sum + k_relu[:, start:stop].sum(axis=1)
        num = np.einsum("bnhd,bhde->bnhe", q_rope[:, start:stop], kv)
        den = np.einsum("bnhd,bhd->bnh", q_relu[:, start:stop], k_sum)
        out[:, start:stop] = num / (den[..., None] + eps)
    if g is not None:
        out = _sigmoid(g) * out
    if rows is not None:
        out = out[:, np.asarray(rows)]
    return out, kv, k_sum


def linear_attention_causal(q, k, v, g=None, rope: Rope3D | None = None, eps: float = 1e-6, kv_in=None,
                            ksum_in=None, rows=None):
    """Token-causal linear attention, fp64 (SANA-Video notes, section 3.4, causal equation).

    Token i sees every token j <= i, itself included, on top of an optional
    carried state:

        KV_i   = KV_in   + sum_{j <= i} c_j^T v_j
        ksum_i = ksum_in + sum_{j <= i} phi(k_j)
        o_i    = (a_i KV_i) / (phi(q_i) . ksum_i + eps)     [then the gate]

    Returns (out, kv_out, ksum_out), the state being the one after the last
    token. ``rows`` selects the outputs returned (any order); the sums are
    accumulated segment by segment between the requested rows, so memory
    stays O(D^2) however long the sequence.
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, N, H, D = q.shape
    q_relu, k_relu, q_rope, k_rope = _features(q, k, rope)
    kv = np.zeros((B, H, D, D)) if kv_in is None else np.array(kv_in, dtype=np.float64)
    k_sum = np.zeros((B, H, D)) if ksum_in is None else np.array(ksum_in, dtype=np.float64)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.zeros((B, len(rows), H, D))
    done = 0  # tokens already summed into kv, k_sum
    for idx in np.argsort(rows, kind="stable"):
        i = int(rows[idx])
        if i + 1 > done:
            kv = kv + np.einsum("bnhd,bnhe->bhde", k_rope[:, done:i + 1], v[:, done:i + 1])
            k_sum = k_sum + k_relu[:, done:i + 1].sum(axis=1)
            done = i + 1
        num = np.einsum("bhd,bhde->bhe", q_rope[:, i], kv)
        den = np.einsum("bhd,bhd->bh", q_relu[:, i], k_sum)
        out[:, idx] = num / (den[..., None] + eps)
    if done < N:
        kv = kv + np.einsum("bnhd,bnhe->bhde", k_rope[:, done:], v[:, done:])
        k_sum = k_sum + k_relu[:, done:].sum(axis=1)
    if g is not None:
        out = _sigmoid(g[:, rows]) * out
    return out, kv, k_sum


def linear_attention_backward(q, k, v, do, g=None, rope: Rope3D | None = None, eps: float = 1e-6):
    """Gradients of the bidirectional (gated) linear attention, fp64.

    Differentiates the definition at the top of this module by hand. With
    s_i = sigmoid(g_i) (1 without a gate), y_i = num_i / den_i and the upstream
    gradient dO:

        dG_i    = dO_i * y_i * s_i * (1 - s_i)
        dY_i    = dO_i * s_i
        dnum_i  = dY_i / den_i,        dden_i = -(dY_i . y_i) / den_i
        da_i    = KV dnum_i,           dKV    = sum_i a_i^T dnum_i
        dphiq_i = R_i^T da_i + dden_i ksum,   dksum = sum_i dden_i phi(q_i)
        dc_j    = dKV v_j,             dv_j   = dKV^T c_j
        dphik_j = R_j^T dc_j + dksum
        dq = dphiq * [q > 0],          dk = dphik * [k > 0]

    (R_i is the rotation of token i, so R_i^T undoes it; ReLU's derivative is
    taken as 0 at 0.) Returns (dq, dk, dv, dg); dg is None without a gate.
    """
    q, k, v, do, g = _f64(q), _f64(k), _f64(v), _f64(do), _f64(g)
    q_relu, k_relu, q_rope, k_rope = _features(q, k, rope)
    kv = np.einsum("bnhd,bnhe->bhde", k_rope, v)
    k_sum = k_relu.sum(axis=1)
    num = np.einsum("bnhd,bhde->bnhe", q_rope, kv)
    den = np.einsum("bnhd,bhd->bnh", q_relu, k_sum)[..., None] + eps
    y = num / den
    s = np.ones_like(y) if g is None else _sigmoid(g)
    dg = None if g is None else do * y * s * (1.0 - s)
    dy = do * s
    dnum = dy / den
    dden = -np.sum(dy * y, axis=-1, keepdims=True) / den
    da = np.einsum("bhde,bnhe->bnhd", kv, dnum)
    dkv = np.einsum("bnhd,bnhe->bhde", q_rope, dnum)
    dk_sum = np.einsum("bnh,bnhd->bhd", dden[..., 0], q_relu)
    dc = np.einsum("bhde,bnhe->bnhd", dkv, v)
    dv = np.einsum("bhde,bnhd->bnhe", dkv, k_rope)
    if rope is not None:
        theta = rope3d_angles(rope)
        da, dc = rope3d_rotate(da, -theta), rope3d_rotate(dc, -theta)
    dphiq = da + dden * k_sum[:, None]
    dphik = dc + dk_sum[:, None]
    dq = dphiq * (q > 0)
    dk = dphik * (k > 0)
    return dq, dk, dv, dg


def linear_attention_chunked_backward(q, k, v, do, chunk_tokens: int, g=None, rope: Rope3D | None = None,
                                      eps: float = 1e-6, kv_in=None, ksum_in=None, dkv_out=None, dksum_out=None):
    """Gradients of the block-causal variant (``linear_attention_chunked``), fp64.

    The loss is sum(dO * o) + sum(dKV_out * KV_out) + sum(dksum_out * ksum_out),
    so the gradients reaching the returned cache are inputs too (zero when not
    given). Chunk c's queries read the cache KV_c, ksum_c, which holds the
    carried state and every chunk up to c. Per chunk, with the notation of
    ``linear_attention_backward``:

        dKV_c   = sum_{i in c} a_i^T dnum_i,      dksum_c = sum_{i in c} dden_i phi(q_i)
        dphiq_i = R_i^T (KV_c dnum_i) + dden_i ksum_c

    A key of chunk c is summed into the caches of chunks c, c+1, ... and into
    the returned cache, so it sees the suffix sums

        GKV_c = dKV_out + sum_{c' >= c} dKV_c',   Gz_c = dksum_out + sum_{c' >= c} dksum_c'
        dphik_j = R_j^T (GKV_c v_j) + Gz_c,       dv_j = GKV_c^T c_j

    and the carried state gets GKV_0, Gz_0. Returns
    (dq, dk, dv, dg, dkv_in, dksum_in); dg is None without a gate.
    """
    if chunk_tokens <= 0:
        raise ValueError("chunk_tokens must be positive")
    q, k, v, do, g = _f64(q), _f64(k), _f64(v), _f64(do), _f64(g)
    B, N, H, D = q.shape
    q_relu, k_relu, q_rope, k_rope = _features(q, k, rope)
    chunks = [slice(start, min(N, start + chunk_tokens)) for start in range(0, N, chunk_tokens)]
    s = np.ones_like(q) if g is None else _sigmoid(g)
    dg = None if g is None else np.zeros((B, N, H, D))

    # query side, chunk by chunk against the cache that includes the chunk
    kv = np.zeros((B, H, D, D)) if kv_in is None else np.array(kv_in, dtype=np.float64)
    k_sum = np.zeros((B, H, D)) if ksum_in is None else np.array(ksum_in, dtype=np.float64)
    da = np.zeros((B, N, H, D))        # KV_c dnum_i, still rotated
    dz_term = np.zeros((B, N, H, D))   # dden_i ksum_c
    dkv_chunk, dks_chunk = [], []
    for sl in chunks:
        kv = kv + np.einsum("bnhd,bnhe->bhde", k_rope[:, sl], v[:, sl])
        k_sum = k_sum + k_relu[:, sl].sum(axis=1)
        num = np.einsum("bnhd,bhde->bnhe", q_rope[:, sl], kv)
        den = np.einsum("bnhd,bhd->bnh", q_relu[:, sl], k_sum)[..., None] + eps
        y = num / den
        if g is not None:
            dg[:, sl] = do[:, sl] * y * s[:, sl] * (1.0 - s[:, sl])
        dy = do[:, sl] * s[:, sl]
        dnum = dy / den
        dden = -np.sum(dy * y, axis=-1, keepdims=True) / den
        da[:, sl] = np.einsum("bhde,bnhe->bnhd", kv, dnum)
        dz_term[:, sl] = dden * k_sum[:, None]
        dkv_chunk.append(np.einsum("bnhd,bnhe->bhde", q_rope[:, sl], dnum))
        dks_chunk.append(np.einsum("bnh,bnhd->bhd", dden[..., 0], q_relu[:, sl]))

    # key side: suffix sums over chunks, from the last chunk back
    gkv = np.zeros((B, H, D, D)) if dkv_out is None else np.array(dkv_out, dtype=np.float64)
    gz = np.zeros((B, H, D)) if dksum_out is None else np.array(dksum_out, dtype=np.float64)
    dc = np.zeros((B, N, H, D))
    dz_key = np.zeros((B, N, H, D))
    dv = np.zeros((B, N, H, D))
    for ci in range(len(chunks) - 1, -1, -1):
        sl = chunks[ci]
        gkv = gkv + dkv_chunk[ci]
        gz = gz + dks_chunk[ci]
        dc[:, sl] = np.einsum("bhde,bnhe->bnhd", gkv, v[:, sl])
        dv[:, sl] = np.einsum("bhde,bnhd->bnhe", gkv, k_rope[:, sl])
        dz_key[:, sl] = gz[:, None]

    if rope is not None:
        theta = rope3d_angles(rope)
        da, dc = rope3d_rotate(da, -theta), rope3d_rotate(dc, -theta)
    dq = (da + dz_term) * (q > 0)
    dk = (dc + dz_key) * (k > 0)
    return dq, dk, dv, dg, gkv, gz

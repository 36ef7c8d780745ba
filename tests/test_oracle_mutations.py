"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign or index, a
transposed operand, a wrong prefix) in a temporary copy of ``oracle/`` and runs
``tests/test_oracle.py`` against that copy: at least one pin must fail. The
repository's oracle is never modified; everything runs on the CPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (file under oracle/, original text, planted mistake)
MUTATIONS = [
    # RoPE: sign of the rotation, frequency exponent, coordinate decoding, band order
    ("rope3d.py", "out[..., 0::2] = even * c - odd * s", "out[..., 0::2] = even * c + odd * s"),
    ("rope3d.py", "(-2.0 * k / d)", "(-1.0 * k / d)"),
    ("rope3d.py", "y = (n // Wg) % Hg", "y = (n // Hg) % Wg"),
    ("rope3d.py", "for pos, d in zip((t, y, x), rope.bands)", "for pos, d in zip((t, x, y), rope.bands)"),
    # bidirectional linear attention
    ("linear_attention.py", 'den = np.einsum("id,d->i", phi_q[b, sel, h, :], zsum[b, h]) + eps',
     'den = np.einsum("id,d->i", rot_q[b, sel, h, :], zsum[b, h]) + eps'),
    ("linear_attention.py", 'den = np.einsum("id,d->i", phi_q[b, sel, h, :], zsum[b, h]) + eps',
     'den = np.maximum(np.einsum("id,d->i", phi_q[b, sel, h, :], zsum[b, h]), eps)'),
    ("linear_attention.py", "state[b, h] = c.T @ v[b, :, h, :]", "state[b, h] = (c.T @ v[b, :, h, :]).T"),
    ("linear_attention.py", "return pos_q, pos_k, rope3d_rotate(pos_q, theta), rope3d_rotate(pos_k, theta)",
     "return pos_q, pos_k, rope3d_rotate(pos_q, theta), pos_k"),
    ("linear_attention.py", "out = _sigmoid(g[:, sel]) * out", "out = (1 - _sigmoid(g[:, sel])) * out"),
    ("linear_attention.py", "zsum[b, h] = phi_k[b, :, h, :].sum(axis=0)", "zsum[b, h] = phi_q[b, :, h, :].sum(axis=0)"),
    # chunked: exclusive instead of inclusive prefix, dropped key-sum input, wrong key sum, dropped gate
    ("linear_attention.py",
     '        num = np.einsum("bnhd,bhde->bnhe", q_rope[:, start:stop], kv)\n        den',
     '        num = np.einsum("bnhd,bhde->bnhe", q_rope[:, start:stop], '
     'kv - np.einsum("bnhd,bnhe->bhde", k_rope[:, start:stop], v[:, start:stop]))\n        den'),
    ("linear_attention.py", "k_sum = np.zeros((B, H, D)) if ksum_in is None else np.array(ksum_in, dtype=np.float64)",
     "k_sum = np.zeros((B, H, D))"),
    ("linear_attention.py", "        k_sum = k_sum + k_relu[:, start:stop].sum(axis=1)",
     "        k_sum = k_sum + q_relu[:, start:stop].sum(axis=1)"),
    ("linear_attention.py", "        out[:, start:stop] = num / (den[..., None] + eps)\n    if g",
     "        out[:, start:stop] = num / (den[..., None] + eps)\n    if False"),
    # token-causal: exclusive instead of inclusive prefix, RoPE on the denominator
    ("linear_attention.py",
     'kv = kv + np.einsum("bnhd,bnhe->bhde", k_rope[:, done:i + 1], v[:, done:i + 1])',
     'kv = kv + np.einsum("bnhd,bnhe->bhde", k_rope[:, done:i], v[:, done:i])'),
    ("linear_attention.py", 'den = np.einsum("bhd,bhd->bh", q_relu[:, i], k_sum)',
     'den = np.einsum("bhd,bhd->bh", q_rope[:, i], k_sum)'),
    # backward: no inverse rotation, gate derivative factor, denominator sign, key-sum gradient
    ("linear_attention.py", "da, dc = rope3d_rotate(da, -theta), rope3d_rotate(dc, -theta)", "da, dc = da, dc"),
    ("linear_attention.py", "dg = None if g is None else do * y * s * (1.0 - s)", "dg = None if g is None else do * y * s"),
    ("linear_attention.py", "dden = -np.sum(dy * y, axis=-1, keepdims=True) / den",
     "dden = np.sum(dy * y, axis=-1, keepdims=True) / den"),
    ("linear_attention.py", "dphik = dc + dk_sum[:, None]", "dphik = dc"),
    # chunked backward: prefix instead of suffix, chunk's own term dropped, returned-cache gradient dropped
    ("linear_attention.py", "    for ci in range(len(chunks) - 1, -1, -1):", "    for ci in range(len(chunks)):"),
    ("linear_attention.py", "        dz_key[:, sl] = gz[:, None]", "        dz_key[:, sl] = (gz - dks_chunk[ci])[:, None]"),
    ("linear_attention.py", 'dc[:, sl] = np.einsum("bhde,bnhe->bnhd", gkv, v[:, sl])',
     'dc[:, sl] = np.einsum("bhde,bnhe->bnhd", gkv - dkv_chunk[ci], v[:, sl])'),
    ("linear_attention.py",
     "gkv = np.zeros((B, H, D, D)) if dkv_out is None else np.array(dkv_out, dtype=np.float64)",
     "gkv = np.zeros((B, H, D, D))"),
    # anchor: missing scale, softmax over the wrong axis
    ("softmax_anchor.py", "logits = scale * (q[b, rr, h, :] @ kh.T)", "logits = (q[b, rr, h, :] @ kh.T)"),
    ("softmax_anchor.py", "p = p / p.sum(axis=1, keepdims=True)", "p = p / p.sum(axis=0, keepdims=True)"),
    # anchor backward: Delta dropped, key gradient unscaled, value gradient from dO instead of dY
    ("softmax_anchor.py", "dl = p * (dp - delta)", "dl = p * dp"),
    ("softmax_anchor.py", "dk[b, :, h, :] += scale * (dl.T @ q[b, rr, h, :])", "dk[b, :, h, :] += dl.T @ q[b, rr, h, :]"),
    ("softmax_anchor.py", "dv[b, :, h, :] += p.T @ dy", "dv[b, :, h, :] += p.T @ do[b, rr, h, :]"),
    # block-sparse anchor: last key of a block dropped, query block taken with the key block size
    ("softmax_anchor.py", "range(m * k_block, min(N, (m + 1) * k_block))", "range(m * k_block, min(N, (m + 1) * k_block - 1))"),
    ("softmax_anchor.py", "                r = i // q_block", "                r = i // k_block"),
    # router: RMSNorm dropped, eps dropped, sum instead of mean
    ("attnres_router.py", "normed = v / rms", "normed = v"),
    ("attnres_router.py", "np.mean(v * v, axis=-1, keepdims=True) + eps", "np.mean(v * v, axis=-1, keepdims=True)"),
    ("attnres_router.py", "np.mean(v * v, axis=-1, keepdims=True)", "np.sum(v * v, axis=-1, keepdims=True)"),
]


@pytest.mark.parametrize("fname,orig,bad", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_planted_mistake_fails_a_pin(tmp_path, fname, orig, bad):
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "test_oracle.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copy(os.path.join(ROOT, "synth.py"), tmp_path / "synth.py")
    path = tmp_path / "oracle" / fname
    src = path.read_text()
    assert orig in src, f"mutation anchor not found in oracle/{fname}: {orig!r}"
    path.write_text(src.replace(orig, bad, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle.py", "-q", "-x", "-p", "no:cacheprovider"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, f"no pin caught the planted mistake ({bad!r}):\n{r.stdout[-2000:]}"

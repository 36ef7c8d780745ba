"""3D rotary position embedding, fp64 (test infrastructure only).

Source: SANA-Video notes (Efficient Video Generation with Block Linear
Diffusion Transformer), section 3.2 and Figure 2(c): Q and K pass through the
ReLU feature map and then through a 3D RoPE; the pseudocode calls it
``apply_3d_rope(x, rope_freqs)`` without defining it. Section 4.1 says the
head dimension was enlarged so that a 3D RoPE fits.

Readings (the pages are silent on these):

* Token flattening: the notes flatten video tokens as T*H*W and reshape back
  as (B, T, H, W, ...) (section 3.3 pseudocode), so token n sits at
  n = (t * Hg + y) * Wg + x, t-major.
* Band split: the head dimension D is split into three contiguous bands
  [t | h | w] of widths (d_t, d_h, d_w) (16/24/24 for D = 64).
* Pairing: adjacent pairs (o + 2k, o + 2k + 1) inside a band starting at dim o,
  rotated by the 2x2 matrix [[cos a, -sin a], [sin a, cos a]] (the original
  rotary form).
* Frequencies: a = p * base^(-2k / d_band), k = 0 .. d_band/2 - 1, with p the
  integer coordinate of the token along the band's axis (t + t_offset, y or x),
  base = 10000.

Parity of this convention against the pages' model is unpinned; the tests pin
the implementation to the reading above.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Rope3D:
    """Grid and band description of a 3D RoPE."""

    grid: tuple  # (T, Hg, Wg)
    bands: tuple = (16, 24, 24)  # (d_t, d_h, d_w)
    base: float = 10000.0
    t_offset: int = 0  # global frame index of the first frame

    @property
    def n_tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w


def rope3d_angles(rope: Rope3D) -> np.ndarray:
    """Rotation angle of every (token, pair): array of shape (N, D/2), fp64.

    Pair p covers dims (2p, 2p+1); pairs are numbered band after band.
    """
    T, Hg, Wg = rope.grid
    n = np.arange(T * Hg * Wg, dtype=np.int64)
    t = n // (Hg * Wg) + rope.t_offset
    y = (n // Wg) % Hg
    x = n % Wg
    cols = []
    for pos, d in zip((t, y, x), rope.bands):
        k = np.arange(d // 2, dtype=np.float64)
        inv_freq = float(rope.base) ** (-2.0 * k / d)
        cols.append(pos.astype(np.float64)[:, None] * inv_freq[None, :])
    return np.concatenate(cols, axis=1)


def rope3d_rotate(x: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs of the last axis of ``x`` (B, N, H, D) by ``theta`` (N, D/2)."""
    c = np.cos(theta)[None, :, None, :]
    s = np.sin(theta)[None, :, None, :]
    even = x[..., 0::2]
    odd = x[..., 1::2]
    out = np.empty_like(x, dtype=np.float64)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out

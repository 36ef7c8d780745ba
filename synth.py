"""Seeded synthetic inputs and the workload shapes they are drawn for.

This module is shared by the tests, the bench and the smoke check. It holds
none of the method's arithmetic: it only draws normal deviates, rounds them to
bfloat16 bit patterns, and names the shapes.

Generator: numpy's PCG64 ``Generator.standard_normal(dtype=float32)``, drawn in
fixed-size blocks; block ``i`` of tensor ``k`` drawn from seed ``s`` uses
``SeedSequence(s, spawn_key=(k, i))``, so blocks are independent of each other and can be filled
by several threads while the result stays a pure function of ``(seed,
shape)``. bfloat16 values are the float32 draws rounded to nearest-even and
kept as ``uint16`` bit patterns; ``bf16_to_f32`` decodes them exactly.

The token grids stand in for the latent grids of the video pages (SANA-Video
2.0 abstract: 720p/5s and 720p/60s; SANA-Video notes, section 1.1: more than
75 000 tokens for 720p/5s).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BLOCK = 1 << 22  # elements per independently seeded block


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even) and return the uint16 bits.

    Inputs are finite normal deviates, so the NaN case is not handled.
    """
    u = x.view(np.uint32)
    bias = ((u >> 16) & 1).astype(np.uint32) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bfloat16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def randn(seed: int, shape, std: float = 1.0, dtype: str = "bf16", stream: int = 0) -> np.ndarray:
    """Seeded N(0, std^2) draws of ``shape``.

    ``stream`` separates the tensors drawn from one seed (Q, K, V, ...).
    ``dtype='f32'`` returns float32; ``dtype='bf16'`` returns uint16 bfloat16
    bit patterns (the float32 draw times ``std``, rounded to nearest-even).
    """
    shape = tuple(int(s) for s in shape)
    total = int(np.prod(shape)) if shape else 1
    out = np.empty(total, np.uint16 if dtype == "bf16" else np.float32)
    nblk = (total + BLOCK - 1) // BLOCK
    sd = np.float32(std)

    def fill(i: int) -> None:
        lo = i * BLOCK
        hi = min(total, lo + BLOCK)
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(stream, i)))
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= sd
        out[lo:hi] = _f32_to_bf16_bits(x) if dtype == "bf16" else x

    if nblk <= 1:
        for i in range(nblk):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def to_f64(x: np.ndarray) -> np.ndarray:
    """float64 view of an input: bf16 bits are decoded, floats are upcast."""
    if x.dtype == np.uint16:
        return bf16_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


@dataclass(frozen=True)
class LinearWorkload:
    """One linear-attention call: (B, N, H, D) tensors over a T x Hg x Wg grid."""

    name: str
    dtype: str  # "bf16" or "f32"
    B: int
    H: int
    grid: tuple  # (T, Hg, Wg); N = T * Hg * Wg
    gated: bool
    seed: int
    D: int = 64
    bands: tuple = (16, 24, 24)
    base: float = 10000.0
    eps: float = 1e-6
    chunk_tokens: int = 0  # 0 = bidirectional over the whole sequence

    @property
    def N(self) -> int:
        t, h, w = self.grid
        return t * h * w

    def draw(self, seed: int | None = None):
        """Q, K, V (and G if gated) as arrays of shape (B, N, H, D)."""
        s = self.seed if seed is None else seed
        shp = (self.B, self.N, self.H, self.D)
        names = ["q", "k", "v"] + (["g"] if self.gated else [])
        return {nm: randn(s, shp, dtype=self.dtype, stream=i) for i, nm in enumerate(names)}


@dataclass(frozen=True)
class AnchorWorkload:
    name: str
    B: int
    N: int
    H: int
    seed: int
    D: int = 64
    gated: bool = True

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def draw(self, seed: int | None = None):
        s = self.seed if seed is None else seed
        shp = (self.B, self.N, self.H, self.D)
        names = ["q", "k", "v"] + (["g"] if self.gated else [])
        return {nm: randn(s, shp, stream=i) for i, nm in enumerate(names)}


@dataclass(frozen=True)
class RouteWorkload:
    name: str
    B: int
    T: int
    C: int
    S: int
    seed: int
    with_phi_t: bool = True
    eps: float = 1e-6
    qstd: float = 0.02

    def draw(self, seed: int | None = None):
        s = self.seed if seed is None else seed
        srcs = [randn(s, (self.B, self.T, self.C), stream=i) for i in range(self.S)]
        w = randn(s, (self.C,), std=self.qstd, dtype="f32", stream=100)
        phi = randn(s, (self.B, self.C), std=self.qstd, dtype="f32", stream=101) if self.with_phi_t else None
        return {"v": srcs, "w": w, "phi_t": phi}


# The measured workloads. Grids, dtypes, gating and seeds as described above;
# the long-video case is chunked every 10 latent frames (36 000 tokens).
LINEAR_F32_N1024 = LinearWorkload("linear_f32_B1H1_4x16x16", "f32", 1, 1, (4, 16, 16), False, 1)
LINEAR_CFGPAIR_N32760 = LinearWorkload("linear_bf16_B2H32_21x30x52_gated", "bf16", 2, 32, (21, 30, 52), True, 2)
LINEAR_720P5S = LinearWorkload("linear_bf16_B1H32_21x45x80_gated", "bf16", 1, 32, (21, 45, 80), True, 3)
HYBRID_LINEAR = [LinearWorkload(f"hybrid_linear{i}_bf16_B1H32_21x45x80_gated", "bf16", 1, 32, (21, 45, 80), True, 40 + i)
                 for i in range(3)]
HYBRID_ANCHOR = AnchorWorkload("hybrid_anchor_bf16_B1H32_N75600_gated", 1, 75600, 32, 43)
HYBRID_ROUTES = [RouteWorkload(f"hybrid_route{i}_bf16_T75600_C2048_S4", 1, 75600, 2048, 4, 44 + i) for i in range(4)]
CHUNKED_720P60S = LinearWorkload("chunked_bf16_B1H32_241x45x80_L36000", "bf16", 1, 32, (241, 45, 80), False, 5,
                                 chunk_tokens=36000)


def block_window_pattern(B: int, H: int, N: int, half_window: int, n_global: int, q_block: int = 128,
                         k_block: int = 64):
    """A local-window block pattern for the block-sparse anchor (a stand-in: the pages give none).

    Query block r (rows [r q_block, (r+1) q_block)) names the key blocks whose
    index lies within ``half_window`` of the key block holding the query
    block's first row, plus the first ``n_global`` key blocks; the same for
    every (b, h), each list ascending and without repeats. Returns int32
    arrays blocks (B, H, nqb, max_blocks), padded with -1, and counts (B, H, nqb).
    """
    nqb, nkb = -(-N // q_block), -(-N // k_block)
    lists = []
    for r in range(nqb):
        c = (r * q_block) // k_block
        named = set(range(max(0, c - half_window), min(nkb, c + half_window + 1))) | set(range(min(n_global, nkb)))
        lists.append(sorted(named))
    width = max(len(x) for x in lists)
    blocks = np.full((B, H, nqb, width), -1, dtype=np.int32)
    counts = np.zeros((B, H, nqb), dtype=np.int32)
    for r, x in enumerate(lists):
        blocks[:, :, r, :len(x)] = x
        counts[:, :, r] = len(x)
    return blocks, counts


# Block-sparse anchor at 720p/5s: a window of +-72 key blocks (about +-1.3
# latent frames of 3 600 tokens) plus 4 global blocks, ~12% of the pairs.
SPARSE_ANCHOR_720P5S = AnchorWorkload("sparse_anchor_bf16_B1H32_N75600_window72_global4_gated", 1, 75600, 32, 48)
SPARSE_ANCHOR_WINDOW = (72, 4)

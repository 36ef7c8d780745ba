"""GPU parity of the block-sparse anchor (hla_softmax_anchor_block_sparse) against the fp64 oracle.

The oracle is ``oracle.softmax_anchor_block_sparse`` (pinned in
tests/test_oracle.py; parity against the pages is unpinned, as they give no
pattern). Cases: random patterns with empty lists, entries that name nothing,
repeated entries, counts beyond max_blocks and negative counts, ragged query
and key blocks, and work-groups whose four query blocks name different tiles;
every key block named, which must equal the dense kernel bit for bit; both
score loops (half precision and bf16 running max) on one pattern; and the
720p/5s local-window pattern on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from softmax_attention_relu_amd import hla

from gpu_common import TOL_BF16, dev, host, normwise, say

pytestmark = pytest.mark.gpu


def random_pattern(rng, B, H, N, max_blocks):
    nqb, nkb = -(-N // 128), -(-N // 64)
    blocks = np.full((B, H, nqb, max_blocks), -1, dtype=np.int32)
    counts = np.zeros((B, H, nqb), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for r in range(nqb):
                c = int(rng.integers(0, max_blocks + 1))
                named = rng.permutation(nkb)[:c]
                if c and rng.random() < 0.3:
                    named[0] = nkb + int(rng.integers(0, 5))  # names nothing
                if c > 2 and rng.random() < 0.3:
                    named[-1] = named[1]  # a repeat counts once
                blocks[b, h, r, :len(named)] = named
                counts[b, h, r] = len(named)
    # a count beyond max_blocks (clamped) and a negative count (none)
    counts[0, 0, 0] = max_blocks + 7
    if nqb > 1:
        counts[-1, -1, 1] = -3
    return blocks, counts


def run(x, blocks, counts):
    d = {k: dev(v) for k, v in x.items()}
    o = hla.hla_softmax_anchor_block_sparse(d["q"], d["k"], d["v"], torch.from_numpy(blocks).cuda(),
                                            torch.from_numpy(counts).cuda(), d.get("g"), 0.125)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("N,B,H,gated", [(1, 1, 1, True), (100, 2, 3, True), (129, 1, 2, False), (300, 2, 2, True),
                                         (1000, 1, 3, True)])
def test_sparse_anchor_random_patterns(N, B, H, gated):
    rng = np.random.default_rng(900 + N)
    names = ["q", "k", "v"] + (["g"] if gated else [])
    x = {nm: synth.randn(910 + N, (B, N, H, 64), stream=i) for i, nm in enumerate(names)}
    max_blocks = min(-(-N // 64), 6)
    blocks, counts = random_pattern(rng, B, H, N, max_blocks)
    say(f"[sparse] N={N} B={B} H={H} gated={gated} max_blocks={max_blocks}")
    o = host(run(x, blocks, counts))
    f = {k: synth.to_f64(v) for k, v in x.items()}
    ref = oracle.softmax_anchor_block_sparse(f["q"], f["k"], f["v"], blocks, np.clip(counts, 0, max_blocks),
                                             f.get("g"), 0.125)
    e = normwise(o, ref)
    say(f"[sparse] normwise {e:.3e}")
    assert e <= TOL_BF16
    # rows of query blocks that name no key give exactly zero
    empty = ref == 0
    assert np.all(o[empty] == 0)


def test_sparse_anchor_both_score_loops():
    """The sparse form takes the half-precision scores or the bf16 running max like the dense one: v * 2^44
    (beyond the |v| bound) changes the loop, which shows in the bits, and both outputs meet the bar."""
    B, N, H = 1, 700, 2
    rng = np.random.default_rng(941)
    x = {nm: synth.randn(941, (B, N, H, 64), stream=i) for i, nm in enumerate("qkvg")}
    blocks, counts = random_pattern(rng, B, H, N, 6)
    f = {k: synth.to_f64(v) for k, v in x.items()}
    ref = oracle.softmax_anchor_block_sparse(f["q"], f["k"], f["v"], blocks, np.clip(counts, 0, 6), f["g"], 0.125)
    d = {k: dev(v) for k, v in x.items()}
    bl, ct = torch.from_numpy(blocks).cuda(), torch.from_numpy(counts).cuda()
    half = hla.hla_softmax_anchor_block_sparse(d["q"], d["k"], d["v"], bl, ct, d["g"], 0.125)
    big = hla.hla_softmax_anchor_block_sparse(d["q"], d["k"], d["v"] * 2.0 ** 44, bl, ct, d["g"], 0.125)
    torch.cuda.synchronize()
    assert normwise(host(half), ref) <= TOL_BF16
    assert normwise(host(big) * 2.0 ** -44, ref) <= TOL_BF16
    assert not torch.equal(big, half * 2.0 ** 44)


def test_sparse_anchor_full_pattern_equals_dense():
    """Every key block named (in reverse order): each wave walks the dense kernel's tiles in ascending order, so
    the outputs match bitwise."""
    B, N, H = 1, 1000, 5
    x = {nm: synth.randn(930, (B, N, H, 64), stream=i) for i, nm in enumerate("qkvg")}
    nqb, nkb = -(-N // 128), -(-N // 64)
    blocks = np.tile(np.arange(nkb, dtype=np.int32)[::-1].copy(), (B, H, nqb, 1))
    counts = np.full((B, H, nqb), nkb, dtype=np.int32)
    o = run(x, blocks, counts)
    d = {k: dev(v) for k, v in x.items()}
    dense = hla.hla_softmax_anchor(d["q"], d["k"], d["v"], d["g"], 0.125)
    torch.cuda.synchronize()
    assert torch.equal(o, dense)


def test_sparse_anchor_720p5s_window_sampled_rows():
    """720p/5s with the local-window pattern (+-72 key blocks + 4 global): sampled rows of four heads."""
    w = synth.SPARSE_ANCHOR_720P5S
    x = w.draw()
    blocks, counts = synth.block_window_pattern(w.B, w.H, w.N, *synth.SPARSE_ANCHOR_WINDOW)
    say(f"[sparse] {w.name}: N={w.N} H={w.H} named blocks per query block {counts.min()}..{counts.max()}")
    o = run(x, blocks, counts)
    rows = np.unique(np.concatenate([np.linspace(0, w.N - 1, 300).astype(np.int64), [0, 127, 128, w.N - 1]]))
    heads = [0, 11, 31]
    got = host(o[:, torch.from_numpy(rows).cuda()][:, :, heads])
    for j, h in enumerate(heads):
        f = {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in x.items()}
        ref = oracle.softmax_anchor_block_sparse(f["q"], f["k"], f["v"], blocks[:, h:h + 1], counts[:, h:h + 1],
                                                 f["g"], w.scale, rows=rows)
        e = normwise(got[:, :, j:j + 1], ref)
        say(f"[sparse] head {h}: normwise {e:.3e}")
        assert e <= TOL_BF16

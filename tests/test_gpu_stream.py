"""Constant-memory streaming (SANA-Video notes, section 3.4, Algorithm 1).

A long video is generated block by block. Every denoising step of a block
attends to the block itself (bidirectionally) and to the cache, the summed
state and key sum of all finished blocks, which it only reads; after the
block's last step its keys and values are committed to the cache. With
``hla_linear_attn_chunked`` a step is one call on the block's tokens with
``kv_in``/``ksum_in`` = the cache and no ``kv_out``; the last step passes the
cache as ``kv_out``/``ksum_out`` too (updated in place).

Checked here on the 720p/60s grid (241 x 45 x 80 latent tokens, blocks of ten
frames) for a cond/uncond pair (B = 2): streamed outputs and the final cache
equal one call over the whole sequence, the fp64 oracle on sampled rows, and
the read-only steps of the first two blocks and the last see exactly the
blocks committed before them.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from softmax_attention_relu_amd import hla

from gpu_common import TOL_BF16, dev, host, normwise, say

pytestmark = pytest.mark.gpu

GRID = (241, 45, 80)
FRAMES = 10
HW = GRID[1] * GRID[2]
B, H = 2, 4


def block_inputs(c, frames):
    """Last-step inputs of block c; the first step uses a perturbed copy (keys rolled, values negated)."""
    shp = (B, frames * HW, H, 64)
    last = {nm: synth.randn(900, shp, stream=10 * c + i) for i, nm in enumerate("qkv")}
    first = dict(q=last["q"], k=np.roll(last["k"], 1000, axis=1), v=last["v"] ^ np.uint16(0x8000))
    return first, last


def test_algorithm1_stream_cfg_pair():
    nblocks = -(-GRID[0] // FRAMES)
    kv = torch.zeros((B, H, 64, 64), dtype=torch.float32, device="cuda")
    ks = torch.zeros((B, H, 64), dtype=torch.float32, device="cuda")
    outs, lasts, firsts = [], [], {}
    checked = (0, 1, nblocks - 1)
    say(f"[stream] {nblocks} blocks of {FRAMES} frames, B={B} H={H}, two steps per block")
    for c in range(nblocks):
        frames = min(FRAMES, GRID[0] - FRAMES * c)
        L = frames * HW
        rope = hla.Rope3D((frames, GRID[1], GRID[2]), t_offset=FRAMES * c)
        first, last = block_inputs(c, frames)
        # step 1: reads the cache, commits nothing
        d = {k: dev(v) for k, v in first.items()}
        o1 = hla.hla_linear_attn_chunked(d["q"], d["k"], d["v"], L, None, rope, kv_in=kv, ksum_in=ks)
        if c in checked:
            firsts[c] = (first, host(o1), host(kv), host(ks))
        # last step: reads the cache, then commits this block into it (in place)
        d = {k: dev(v) for k, v in last.items()}
        o2 = hla.hla_linear_attn_chunked(d["q"], d["k"], d["v"], L, None, rope, kv_in=kv, ksum_in=ks, kv_out=kv,
                                         ksum_out=ks)
        outs.append(o2)
        lasts.append(last)
    torch.cuda.synchronize()
    stream_out = torch.cat(outs, dim=1)
    full = {nm: np.concatenate([x[nm] for x in lasts], axis=1) for nm in "qkv"}

    # one call over the whole sequence
    d = {k: dev(v) for k, v in full.items()}
    kv1 = torch.empty_like(kv)
    ks1 = torch.empty_like(ks)
    one = hla.hla_linear_attn_chunked(d["q"], d["k"], d["v"], FRAMES * HW, None, hla.Rope3D(GRID), kv_out=kv1,
                                      ksum_out=ks1)
    torch.cuda.synchronize()
    e_one = normwise(host(stream_out), host(one))
    e_kv = normwise(host(kv), host(kv1))
    e_ks = normwise(host(ks), host(ks1))
    say(f"[stream] streamed vs one call: out {e_one:.2e} state {e_kv:.2e} key sum {e_ks:.2e}")
    # same arithmetic except the split of the state sums: states agree to fp32 rounding
    assert e_kv <= 1e-5 and e_ks <= 1e-5
    assert e_one <= TOL_BF16

    # fp64 oracle on one head, sampled rows of every block
    h = 1
    N = full["q"].shape[1]
    rows = np.unique(np.concatenate([np.linspace(0, N - 1, 600).astype(np.int64), [N - 1]]))
    f = {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in full.items()}
    ref, kv_ref, ks_ref = oracle.linear_attention_chunked(f["q"], f["k"], f["v"], FRAMES * HW, None,
                                                          oracle.Rope3D(GRID), rows=rows)
    got = host(stream_out[:, torch.from_numpy(rows).cuda(), h:h + 1])
    e_ref = normwise(got, ref)
    e_kvr = normwise(host(kv)[:, h:h + 1], kv_ref)
    e_ksr = normwise(host(ks)[:, h:h + 1], ks_ref)
    say(f"[stream] streamed vs oracle (head {h}): out {e_ref:.2e} state {e_kvr:.2e} key sum {e_ksr:.2e}")
    assert e_ref <= TOL_BF16 and e_kvr <= TOL_BF16 and e_ksr <= 1e-5

    # the read-only steps saw exactly the blocks committed before them
    for c, (first, o1, kv_in, ks_in) in firsts.items():
        frames = first["q"].shape[1] // HW
        g = {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in first.items()}
        # cache before block c from the oracle: the blocks before it (last-step inputs)
        n0 = FRAMES * HW * c
        if c == 0:
            kv0, ks0 = np.zeros((B, 1, 64, 64)), np.zeros((B, 1, 64))
        elif c == 1:
            blk = {k: v[:, :n0] for k, v in f.items()}
            _, kv0, ks0 = oracle.linear_attention_chunked(blk["q"], blk["k"], blk["v"], n0, None,
                                                          oracle.Rope3D((FRAMES, GRID[1], GRID[2])), rows=[0])
        else:  # the last block: final cache minus the block's own state
            blk = {k: v[:, n0:] for k, v in f.items()}
            _, kv_c, ks_c = oracle.linear_attention_chunked(blk["q"], blk["k"], blk["v"], N - n0, None,
                                                            oracle.Rope3D((frames, GRID[1], GRID[2]),
                                                                          t_offset=FRAMES * c), rows=[0])
            kv0, ks0 = kv_ref - kv_c, ks_ref - ks_c
        if c:
            assert normwise(kv_in[:, h:h + 1], kv0) <= TOL_BF16
        else:
            assert np.all(kv_in == 0)
        L = frames * HW
        r = np.unique(np.linspace(0, L - 1, 200).astype(np.int64))
        ref1, _, _ = oracle.linear_attention_chunked(g["q"], g["k"], g["v"], L, None,
                                                     oracle.Rope3D((frames, GRID[1], GRID[2]), t_offset=FRAMES * c),
                                                     kv_in=kv0, ksum_in=ks0, rows=r)
        e1 = normwise(o1[:, r, h:h + 1], ref1)
        say(f"[stream] block {c} read-only step vs oracle: {e1:.2e}")
        assert e1 <= TOL_BF16

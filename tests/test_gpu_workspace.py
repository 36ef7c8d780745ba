"""Workspace contents on entry do not matter.

Every call that takes a workspace is run twice on the same inputs: once with
the workspace zeroed and once with every byte 0xFF (a NaN pattern in every
float it could hold). The outputs must be equal bit for bit, so no kernel
reads a workspace byte that the same call has not written first. Shapes span
several tiles, slabs, chunks and query blocks, with ragged ends.
"""
import numpy as np
import pytest
import torch

import synth
from softmax_attention_relu_amd import hla

from gpu_common import dev, say

pytestmark = pytest.mark.gpu

B, N, H = 2, 1000, 4
GRID = (10, 10, 10)


def inputs(seed, names="qkvg"):
    return {nm: dev(synth.randn(seed, (B, N, H, 64), stream=i)) for i, nm in enumerate(names)}


def both(nbytes, call):
    """call(ws) -> tensor or tuple of tensors, with a zeroed and a 0xFF-filled workspace."""
    out = []
    for fill in (0, 255):
        ws = torch.full((max(int(nbytes), 1),), fill, dtype=torch.uint8, device="cuda")
        r = call(ws)
        torch.cuda.synchronize()
        out.append(r if isinstance(r, tuple) else (r,))
    return out


def assert_same(a, b):
    for x, y in zip(a, b):
        if x is None and y is None:
            continue
        assert torch.equal(x, y)


def test_linear_forms():
    say("[workspace] linear, chunked, causal")
    x = inputs(961)
    rope = hla.Rope3D(GRID)
    assert_same(*both(hla.hla_linear_attn_workspace(B, N, H, 64),
                      lambda ws: hla.hla_linear_attn(x["q"], x["k"], x["v"], x["g"], rope, ws=ws)))

    def chunked(ws):
        kv = torch.empty((B, H, 64, 64), dtype=torch.float32, device="cuda")
        ks = torch.empty((B, H, 64), dtype=torch.float32, device="cuda")
        o = hla.hla_linear_attn_chunked(x["q"], x["k"], x["v"], 300, x["g"], rope, kv_out=kv, ksum_out=ks, ws=ws)
        return o, kv, ks
    assert_same(*both(hla.hla_linear_attn_chunked_workspace(B, N, H, 64, 300), chunked))
    assert_same(*both(hla.hla_linear_attn_causal_workspace(B, N, H, 64),
                      lambda ws: hla.hla_linear_attn_causal(x["q"], x["k"], x["v"], x["g"], rope, ws=ws)))


def test_linear_gradients():
    say("[workspace] linear gradients")
    x = inputs(962, "qkvgd")
    rope = hla.Rope3D(GRID)
    assert_same(*both(hla.hla_linear_attn_backward_workspace(B, N, H, 64),
                      lambda ws: hla.hla_linear_attn_backward(x["q"], x["k"], x["v"], x["d"], x["g"], rope, ws=ws)))
    assert_same(*both(hla.hla_linear_attn_chunked_backward_workspace(B, N, H, 64, 300),
                      lambda ws: hla.hla_linear_attn_chunked_backward(x["q"], x["k"], x["v"], x["d"], 300, x["g"],
                                                                      rope, ws=ws)[:4]))
    kv = torch.empty((B, H, 64, 64), dtype=torch.float32, device="cuda")
    ks = torch.empty((B, H, 64), dtype=torch.float32, device="cuda")
    hla.hla_linear_attn_chunked(x["q"], x["k"], x["v"], N, None, rope, kv_out=kv, ksum_out=ks)
    assert_same(*both(hla.hla_linear_attn_backward_workspace(B, N, H, 64),
                      lambda ws: hla.hla_linear_attn_backward_saved(x["q"], x["k"], x["v"], kv, ks, x["d"], x["g"],
                                                                    rope, ws=ws)))


def test_anchor_forms():
    say("[workspace] anchor, lse, block-sparse")
    x = inputs(963)
    nbytes = hla.hla_softmax_anchor_workspace(B, N, H, 64)
    assert_same(*both(nbytes, lambda ws: hla.hla_softmax_anchor(x["q"], x["k"], x["v"], x["g"], ws=ws)))
    assert_same(*both(nbytes, lambda ws: hla.hla_softmax_anchor_lse(x["q"], x["k"], x["v"], x["g"], ws=ws)))
    rng = np.random.default_rng(963)
    nqb, nkb, mb = -(-N // 128), -(-N // 64), 5
    blocks = torch.from_numpy(rng.integers(0, nkb, size=(B, H, nqb, mb)).astype(np.int32)).cuda()
    counts = torch.from_numpy(rng.integers(0, mb + 1, size=(B, H, nqb)).astype(np.int32)).cuda()
    assert_same(*both(nbytes, lambda ws: hla.hla_softmax_anchor_block_sparse(x["q"], x["k"], x["v"], blocks, counts,
                                                                             x["g"], ws=ws)))


def test_anchor_gradients():
    say("[workspace] anchor gradients")
    x = inputs(964, "qkvgd")
    nbytes = hla.hla_softmax_anchor_backward_workspace(B, N, H, 64)
    assert_same(*both(nbytes, lambda ws: hla.hla_softmax_anchor_backward(x["q"], x["k"], x["v"], x["d"], x["g"],
                                                                         ws=ws)))
    o, lse = hla.hla_softmax_anchor_lse(x["q"], x["k"], x["v"], x["g"])
    assert_same(*both(nbytes, lambda ws: hla.hla_softmax_anchor_backward_saved(x["q"], x["k"], x["v"], o, lse,
                                                                               x["d"], x["g"], ws=ws)))

"""Library calls captured in a HIP graph replay to the eager results.

The calls issue kernels only (no memset or copy nodes), so they can be
captured once their RoPE tables are on the device and their outputs and
workspaces are allocated. The graph holds a gated linear layer with RoPE, its
allocation-free form, a block-causal call carrying state, the anchor and a
route. It is replayed three times with the program's own eager work and a
synchronisation between the replays; before each replay the outputs are
cleared, and after it every output must equal the eager call's bit for bit.
"""
import pytest
import torch

import synth
from softmax_attention_relu_amd import hla

from gpu_common import dev, say

pytestmark = pytest.mark.gpu

B, N, H = 1, 1000, 4
GRID = (10, 10, 10)


def test_captured_calls_replay_eagerly_equal():
    say("[graph] capture and replay")
    x = {nm: dev(synth.randn(971, (B, N, H, 64), stream=i)) for i, nm in enumerate("qkvg")}
    srcs = [dev(synth.randn(972, (B, N, 256), stream=i)) for i in range(4)]
    w = dev(synth.randn(973, (256,), std=0.02, dtype="f32"))
    rope = hla.Rope3D(GRID)
    q, k, v, g = x["q"], x["k"], x["v"], x["g"]

    outs = {
        "o": torch.empty_like(q), "o_na": torch.empty_like(q), "oc": torch.empty_like(q), "oa": torch.empty_like(q),
        "kv": torch.empty((B, H, 64, 64), dtype=torch.float32, device="cuda"),
        "ks": torch.empty((B, H, 64), dtype=torch.float32, device="cuda"),
        "h": torch.empty_like(srcs[0]),
    }
    ws_l = torch.empty(hla.hla_linear_attn_workspace(B, N, H, 64), dtype=torch.uint8, device="cuda")
    ws_c = torch.empty(hla.hla_linear_attn_chunked_workspace(B, N, H, 64, 300), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(hla.hla_softmax_anchor_workspace(B, N, H, 64), dtype=torch.uint8, device="cuda")

    def calls():
        hla.hla_linear_attn(q, k, v, g, rope, o=outs["o"], ws=ws_l)
        hla.hla_linear_attn_noalloc(q, k, v, g, rope, o=outs["o_na"])
        hla.hla_linear_attn_chunked(q, k, v, 300, g, rope, kv_out=outs["kv"], ksum_out=outs["ks"], o=outs["oc"],
                                    ws=ws_c)
        hla.hla_softmax_anchor(q, k, v, g, o=outs["oa"], ws=ws_a)
        hla.hla_attnres_route(srcs, w, None, h=outs["h"])

    calls()  # eager, also places the RoPE tables on the device
    torch.cuda.synchronize()
    ref = {name: t.clone() for name, t in outs.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for r in range(3):
        for t in outs.values():
            t.fill_(float("nan") if t.dtype != torch.uint8 else 0)
        a = torch.randn((1024, 1024), device="cuda")
        (a @ a).sum().item()  # eager work and a synchronisation between replays
        graph.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(t, ref[name]), (r, name)

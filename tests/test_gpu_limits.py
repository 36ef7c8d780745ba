"""GPU calls at the C ABI's size limit: B * H = 65 535 (batch, head) pairs, the most
the launch grids take (one more is rejected on the host, tests/test_abi_host.py),
with short sequences so the tensors stay small. Sampled heads, the first and the
last ones included, are compared with the fp64 oracle at the bf16 bar.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from softmax_attention_relu_amd import hla

from gpu_common import TOL_BF16, dev, host, normwise, say

pytestmark = pytest.mark.gpu

PAIRS = 65535


def sampled(H):
    return sorted({0, 1, 4097, H // 2, H - 2, H - 1})


def heads_of(x, h):
    return {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in x.items()}


def test_linear_chunked_causal_at_max_batch_heads():
    B, N, H, L = 1, 40, PAIRS, 16
    say(f"[limits] linear paths B={B} N={N} H={H}")
    x = {nm: synth.randn(900, (B, N, H, 64), stream=i) for i, nm in enumerate("qkvg")}
    d = {k: dev(v) for k, v in x.items()}
    o = hla.hla_linear_attn(d["q"], d["k"], d["v"], d["g"], None)
    kv = torch.empty((B, H, 64, 64), dtype=torch.float32, device="cuda")
    ks = torch.empty((B, H, 64), dtype=torch.float32, device="cuda")
    oc = hla.hla_linear_attn_chunked(d["q"], d["k"], d["v"], L, d["g"], None, kv_out=kv, ksum_out=ks)
    ot = hla.hla_linear_attn_causal(d["q"], d["k"], d["v"], d["g"], None)
    torch.cuda.synchronize()
    o, oc, ot, kv, ks = host(o), host(oc), host(ot), host(kv), host(ks)
    for h in sampled(H):
        f = heads_of(x, h)
        ref = oracle.linear_attention(f["q"], f["k"], f["v"], f["g"])
        ref_c, ref_kv, ref_ks = oracle.linear_attention_chunked(f["q"], f["k"], f["v"], L, f["g"])
        ref_t, _, _ = oracle.linear_attention_causal(f["q"], f["k"], f["v"], f["g"])
        assert normwise(o[:, :, h:h + 1], ref) <= TOL_BF16, h
        assert normwise(oc[:, :, h:h + 1], ref_c) <= TOL_BF16, h
        assert normwise(ot[:, :, h:h + 1], ref_t) <= TOL_BF16, h
        assert normwise(kv[:, h:h + 1], ref_kv) <= TOL_BF16, h
        assert normwise(ks[:, h:h + 1], ref_ks) <= 1e-5, h


def test_anchor_at_max_batch_heads():
    B, N, H = 5, 70, PAIRS // 5
    say(f"[limits] anchor B={B} N={N} H={H}")
    x = {nm: synth.randn(901, (B, N, H, 64), stream=i) for i, nm in enumerate("qkvg")}
    d = {k: dev(v) for k, v in x.items()}
    o = host(hla.hla_softmax_anchor(d["q"], d["k"], d["v"], d["g"]))
    torch.cuda.synchronize()
    for h in sampled(H):
        f = heads_of(x, h)
        ref = oracle.softmax_anchor(f["q"], f["k"], f["v"], f["g"], scale=0.125)
        assert normwise(o[:, :, h:h + 1], ref) <= TOL_BF16, h
    assert np.isfinite(o).all()


def test_anchor_gradients_at_max_batch_heads():
    B, N, H = 5, 70, PAIRS // 5
    say(f"[limits] anchor gradients B={B} N={N} H={H}")
    x = {nm: synth.randn(902, (B, N, H, 64), stream=i) for i, nm in enumerate(("q", "k", "v", "g", "do"))}
    d = {k: dev(v) for k, v in x.items()}
    out = [host(t) for t in hla.hla_softmax_anchor_backward(d["q"], d["k"], d["v"], d["do"], d["g"], 0.125)]
    torch.cuda.synchronize()
    for h in sampled(H):
        f = heads_of(x, h)
        ref = oracle.softmax_anchor_backward(f["q"], f["k"], f["v"], f["do"], f["g"], 0.125)
        for i, nm in enumerate(("dq", "dk", "dv", "dg")):
            assert normwise(out[i][:, :, h:h + 1], ref[i]) <= TOL_BF16, (nm, h)
    for t in out:
        assert np.isfinite(t).all()

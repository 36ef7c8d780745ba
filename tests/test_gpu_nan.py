"""NaN and Inf inputs on the GPU: what reaches the outputs.

The stated behaviour (a reading: no page says anything about non-finite
inputs) is propagation. phi = ReLU keeps NaN (phi(-Inf) = 0, phi(+Inf) = +Inf),
every sum that takes a NaN or Inf term carries it, and nothing is clamped:

- linear (bidirectional): a NaN in q_i spoils row i only; in k_j every row of
  that head (the key sum and the state); in v_j[e] column e of every row of
  that head; in g_i[e] that one element;
- block-causal: a key or value of chunk c spoils chunk c and every later chunk,
  not the earlier ones, and the returned state;
- softmax anchor: a NaN in q_i spoils row i; in k_j every row of the head; in
  v_j[e] column e of every row of the head;
- router: a NaN in any source at token t spoils h_t and alpha_t only.

Outputs that do not depend on the planted value equal the clean call's
outputs (bitwise where the kernel takes the same path; the anchor's other
rows in the spoiled query's wave take the running-max path and are compared
to the bf16 bar). These are ordinary, in-bounds launches.
"""
import numpy as np
import pytest
import torch

import synth
from softmax_attention_relu_amd import hla

from gpu_common import TOL_BF16, dev, normwise, say

pytestmark = pytest.mark.gpu

B, N, H = 1, 300, 2
GRID = (3, 10, 10)
I0, J0, H0, D0 = 123, 77, 1, 5


def inputs(seed):
    return {nm: dev(synth.randn(seed, (B, N, H, 64), stream=i)) for i, nm in enumerate("qkvg")}


def planted(x, name, tok, value, dim=D0):
    y = {k: v.clone() for k, v in x.items()}
    y[name][0, tok, H0, dim] = value
    return y


def linear(x, chunk=0, state=False):
    rope = hla.Rope3D(GRID)
    if chunk:
        kv = torch.empty((B, H, 64, 64), dtype=torch.float32, device="cuda")
        ks = torch.empty((B, H, 64), dtype=torch.float32, device="cuda")
        o = hla.hla_linear_attn_chunked(x["q"], x["k"], x["v"], chunk, x["g"], rope, kv_out=kv, ksum_out=ks)
        torch.cuda.synchronize()
        return (o, kv, ks) if state else o
    o = hla.hla_linear_attn(x["q"], x["k"], x["v"], x["g"], rope)
    torch.cuda.synchronize()
    return o


def other_heads_equal(a, b):
    keep = [h for h in range(H) if h != H0]
    return torch.equal(a[:, :, keep], b[:, :, keep])


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_linear_query(bad):
    say(f"[nan] linear q {bad}")
    x = inputs(71)
    ref, got = linear(x), linear(planted(x, "q", I0, bad))
    assert not torch.isfinite(got[0, I0, H0].float()).any()
    mask = torch.ones(N, dtype=torch.bool, device="cuda")
    mask[I0] = False
    assert torch.equal(got[0, mask], ref[0, mask])


def test_linear_key_nan_and_negative_inf():
    say("[nan] linear k")
    x = inputs(72)
    ref, got = linear(x), linear(planted(x, "k", J0, float("nan")))
    assert torch.isnan(got[0, :, H0].float()).all()
    assert other_heads_equal(got, ref)
    # phi(-Inf) = 0: the same as any negative value there
    neg = linear(planted(x, "k", J0, -1.0))
    assert torch.equal(linear(planted(x, "k", J0, float("-inf"))), neg)


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_linear_value(bad):
    say(f"[nan] linear v {bad}")
    x = inputs(73)
    ref, got = linear(x), linear(planted(x, "v", J0, bad))
    assert not torch.isfinite(got[0, :, H0, D0].float()).any()
    cols = [e for e in range(64) if e != D0]
    assert torch.equal(got[0, :, H0, cols], ref[0, :, H0, cols])
    assert other_heads_equal(got, ref)


def test_linear_gate_nan():
    say("[nan] linear g")
    x = inputs(74)
    ref, got = linear(x), linear(planted(x, "g", I0, float("nan")))
    bad = ~torch.isfinite(got.float())
    assert bad.sum().item() == 1 and bad[0, I0, H0, D0]
    assert torch.equal(torch.where(bad, ref, got), ref)


@pytest.mark.parametrize("name", ["k", "v"])
def test_chunked_spoils_own_and_later_chunks(name):
    say(f"[nan] chunked {name}")
    x = inputs(75)
    L, tok = 100, 150  # three chunks; the planted token sits in chunk 1
    ref, kv_r, ks_r = linear(x, chunk=L, state=True)
    got, kv, ks = linear(planted(x, name, tok, float("nan")), chunk=L, state=True)
    assert torch.equal(got[0, :L], ref[0, :L])  # chunk 0 does not see the token
    later = got[0, L:, H0].float()
    if name == "k":
        assert torch.isnan(later).all()
        assert torch.isnan(ks[0, H0, D0]) and torch.isnan(kv[0, H0]).any()
    else:
        assert torch.isnan(later[:, D0]).all()
        assert torch.isnan(kv[0, H0, :, D0]).all()
    assert other_heads_equal(got, ref)


def anchor(x):
    o = hla.hla_softmax_anchor(x["q"], x["k"], x["v"], x["g"])
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_anchor_query(bad):
    say(f"[nan] anchor q {bad}")
    x = inputs(76)
    ref, got = anchor(x), anchor(planted(x, "q", I0, bad))
    assert not torch.isfinite(got[0, I0, H0].float()).all()
    if bad != bad:  # NaN: the whole row
        assert torch.isnan(got[0, I0, H0].float()).all()
    mask = torch.ones(N, dtype=torch.bool, device="cuda")
    mask[I0] = False
    g, r = got[0, mask].float().cpu().numpy(), ref[0, mask].float().cpu().numpy()
    assert np.isfinite(g).all()
    assert normwise(g.astype(np.float64), r.astype(np.float64)) <= TOL_BF16


def test_anchor_key_nan():
    say("[nan] anchor k")
    x = inputs(77)
    ref, got = anchor(x), anchor(planted(x, "k", J0, float("nan")))
    assert torch.isnan(got[0, :, H0].float()).all()
    assert other_heads_equal(got, ref)


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_anchor_value(bad):
    say(f"[nan] anchor v {bad}")
    x = inputs(78)
    ref, got = anchor(x), anchor(planted(x, "v", J0, bad))
    assert not torch.isfinite(got[0, :, H0, D0].float()).any()
    cols = [e for e in range(64) if e != D0]
    assert torch.equal(got[0, :, H0, cols], ref[0, :, H0, cols])
    assert other_heads_equal(got, ref)


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_route_source(bad):
    say(f"[nan] route {bad}")
    T, C, S, t0 = 200, 256, 4, 57
    srcs = [dev(synth.randn(79, (B, T, C), stream=i)) for i in range(S)]
    w = dev(synth.randn(79, (C,), std=0.02, dtype="f32", stream=100))
    phi = dev(synth.randn(79, (B, C), std=0.02, dtype="f32", stream=101))
    h_ref, a_ref = hla.hla_attnres_route(srcs, w, phi, alpha=True)
    bad_srcs = [s.clone() for s in srcs]
    bad_srcs[2][0, t0, 11] = bad
    h, a = hla.hla_attnres_route(bad_srcs, w, phi, alpha=True)
    torch.cuda.synchronize()
    assert not torch.isfinite(h[0, t0].float()).all()
    if bad != bad:
        assert torch.isnan(h[0, t0].float()).all() and torch.isnan(a[0, t0]).all()
    mask = torch.ones(T, dtype=torch.bool, device="cuda")
    mask[t0] = False
    assert torch.equal(h[0, mask], h_ref[0, mask]) and torch.equal(a[0, mask], a_ref[0, mask])

"""Every call runs on the stream it is given.

The inputs are produced on a side stream behind a long matrix product, and the
library call is issued on that side stream with no other synchronisation. Had
any kernel run on another stream it would read the inputs before they exist
(they start as uninitialised memory); on the given stream it reads them in
order, and the outputs equal those of the same call on the default stream
bitwise. Streams keep the default priority. Forward calls and gradients, and
calls from four host threads at once.
"""
import pytest
import torch

import synth
from softmax_attention_relu_amd import hla

from gpu_common import dev, say

pytestmark = pytest.mark.gpu

B, N, H = 1, 1000, 4
GRID = (10, 10, 10)


def delayed_copies(side, tensors):
    """Copies of ``tensors`` made on ``side`` after a long product queued there first."""
    with torch.cuda.stream(side):
        a = torch.randn((4096, 4096), device="cuda")
        for _ in range(8):
            a = a @ a
            a = a / a.abs().max()
        out = [torch.empty_like(t) for t in tensors]
        for o, t in zip(out, tensors):
            o.copy_(t)
    return out


def test_linear_forms_on_a_side_stream():
    say("[streams] linear, chunked, causal")
    x = [dev(synth.randn(950, (B, N, H, 64), stream=i)) for i in range(4)]
    rope = hla.Rope3D(GRID)
    ref = hla.hla_linear_attn(*x, rope)
    ref_c = hla.hla_linear_attn_chunked(x[0], x[1], x[2], 300, x[3], rope)
    ref_t = hla.hla_linear_attn_causal(*x, rope)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    xs = delayed_copies(side, x)
    with torch.cuda.stream(side):
        o = hla.hla_linear_attn(*xs, rope, stream=side)
        oc = hla.hla_linear_attn_chunked(xs[0], xs[1], xs[2], 300, xs[3], rope, stream=side)
        ot = hla.hla_linear_attn_causal(*xs, rope, stream=side)
    side.synchronize()
    assert torch.equal(o, ref) and torch.equal(oc, ref_c) and torch.equal(ot, ref_t)


def test_anchor_and_route_on_a_side_stream():
    say("[streams] anchor, route")
    x = [dev(synth.randn(951, (B, N, H, 64), stream=i)) for i in range(4)]
    srcs = [dev(synth.randn(952, (B, N, 256), stream=i)) for i in range(4)]
    w = dev(synth.randn(953, (256,), std=0.02, dtype="f32"))
    ref = hla.hla_softmax_anchor(*x)
    ref_h, ref_a = hla.hla_attnres_route(srcs, w, None, alpha=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    xs = delayed_copies(side, x + srcs)
    with torch.cuda.stream(side):
        o = hla.hla_softmax_anchor(*xs[:4], stream=side)
        h, al = hla.hla_attnres_route(xs[4:], w, None, alpha=True, stream=side)
    side.synchronize()
    assert torch.equal(o, ref) and torch.equal(h, ref_h) and torch.equal(al, ref_a)


def test_gradients_on_a_side_stream():
    say("[streams] linear and anchor gradients")
    x = [dev(synth.randn(954, (B, N, H, 64), stream=i)) for i in range(5)]
    q, k, v, g, do = x
    rope = hla.Rope3D(GRID)
    ref_l = hla.hla_linear_attn_backward(q, k, v, do, g, rope)
    ref_c = hla.hla_linear_attn_chunked_backward(q, k, v, do, 300, g, rope)[:4]
    ref_a = hla.hla_softmax_anchor_backward(q, k, v, do, g)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    qs, ks, vs, gs, ds = delayed_copies(side, x)
    with torch.cuda.stream(side):
        gl = hla.hla_linear_attn_backward(qs, ks, vs, ds, gs, rope, stream=side)
        gc = hla.hla_linear_attn_chunked_backward(qs, ks, vs, ds, 300, gs, rope, stream=side)[:4]
        ga = hla.hla_softmax_anchor_backward(qs, ks, vs, ds, gs, stream=side)
    side.synchronize()
    for got, ref in ((gl, ref_l), (gc, ref_c), (ga, ref_a)):
        for a, b in zip(got, ref):
            assert torch.equal(a, b)


def test_calls_from_several_host_threads():
    """Four host threads, each with its own stream, outputs and workspaces, call the linear layer and the
    anchor at once; every result equals the same call made alone."""
    import threading

    say("[streams] four host threads")
    xs = [[dev(synth.randn(955 + t, (B, N, H, 64), stream=i)) for i in range(4)] for t in range(4)]
    rope = hla.Rope3D(GRID)
    refs = []
    for x in xs:
        refs.append((hla.hla_linear_attn(*x, rope), hla.hla_softmax_anchor(*x)))
    torch.cuda.synchronize()
    got = [None] * 4
    errors = []

    def work(t):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                o = hla.hla_linear_attn(*xs[t], rope, stream=st)
                oa = hla.hla_softmax_anchor(*xs[t], stream=st)
            st.synchronize()
            got[t] = (o, oa)
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for (o, oa), (r, ra) in zip(got, refs):
        assert torch.equal(o, r) and torch.equal(oa, ra)

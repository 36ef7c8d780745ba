"""GPU parity of the anchor gradients (hla_softmax_anchor_backward) against the fp64 oracle.

The oracle is ``oracle.softmax_anchor_backward`` (pinned in tests/test_oracle.py
to autograd of an independent forward and to central differences). Shapes
cover one token, tile edges (63, 64, 65 tokens), ragged multi-tile lengths and
a part-empty last work-group, with and without the gate; N = 4096 in full; and
the 720p/5s shape, where dq and dg are compared on sampled rows and dk, dv
through identities that hold at any size (sum_j dv_j = sum_i dY_i and
sum_j dk_j = 0, because every row of the weights sums to one).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from softmax_attention_relu_amd import hla

from gpu_common import TOL_BF16, dev, host, normwise, say

pytestmark = pytest.mark.gpu


def inputs(seed, B, N, H, gated):
    names = ["q", "k", "v", "do"] + (["g"] if gated else [])
    return {nm: synth.randn(seed, (B, N, H, 64), stream=i) for i, nm in enumerate(names)}


def run(x, scale=0.125):
    d = {k: dev(v) for k, v in x.items()}
    out = hla.hla_softmax_anchor_backward(d["q"], d["k"], d["v"], d["do"], d.get("g"), scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("N", [1, 63, 64, 65, 300, 1000])
@pytest.mark.parametrize("gated", [True, False])
def test_anchor_backward_small_shapes(N, gated):
    B, H = 2, 3
    x = inputs(960 + N, B, N, H, gated)
    say(f"[anchor bwd] N={N} gated={gated}")
    dq, dk, dv, dg = run(x)
    f = {k: synth.to_f64(v) for k, v in x.items()}
    ref = oracle.softmax_anchor_backward(f["q"], f["k"], f["v"], f["do"], f.get("g"), 0.125)
    checked = (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2]))
    if N == 1:
        # One key: every weight is 1, so dL = dP - Delta = dY . v - dY . y = 0 and dq, dk vanish exactly.
        # The result is the cancellation of two terms of size |dY . v|; bound the error by those terms.
        s = 1.0 if not gated else 1.0 / (1.0 + np.exp(-f["g"]))
        term = np.abs(np.sum(f["do"] * s * f["v"], axis=-1, keepdims=True))
        for nm, got, other in (("dq", dq, f["k"]), ("dk", dk, f["q"])):
            err = np.abs(host(got)).max()
            size = 0.125 * np.max(term * np.abs(other))
            say(f"[anchor bwd] {nm} (one key): {err:.3e} of term size {size:.3e}")
            assert err <= TOL_BF16 * size
        checked = checked[2:]
    for nm, got, r in checked:
        e = normwise(host(got), r)
        say(f"[anchor bwd] {nm}: {e:.3e}")
        assert e <= TOL_BF16, nm
    if gated:
        e = normwise(host(dg), ref[3])
        say(f"[anchor bwd] dg: {e:.3e}")
        assert e <= TOL_BF16
    else:
        assert dg is None


def test_anchor_backward_n4096_and_repeat():
    """One head at N = 4096 (64 tiles each way) in full; a second call is bitwise identical."""
    x = inputs(990, 1, 4096, 2, True)
    dq, dk, dv, dg = run(x)
    again = run(x)
    for a, b in zip((dq, dk, dv, dg), again):
        assert torch.equal(a, b)
    f = {k: synth.to_f64(v) for k, v in x.items()}
    ref = oracle.softmax_anchor_backward(f["q"], f["k"], f["v"], f["do"], f["g"], 0.125)
    for nm, got, r in zip(("dq", "dk", "dv", "dg"), (dq, dk, dv, dg), ref):
        e = normwise(host(got), r)
        say(f"[anchor bwd] N=4096 {nm}: {e:.3e}")
        assert e <= TOL_BF16, nm


def test_anchor_backward_720p5s():
    """720p/5s (B1 H32 N75600, gated): dq, dg on sampled rows of three heads; dk, dv by identities."""
    w = synth.HYBRID_ANCHOR
    x = w.draw()
    x["do"] = synth.randn(w.seed, (w.B, w.N, w.H, w.D), stream=4)
    say(f"[anchor bwd] {w.name}: N={w.N} H={w.H}")
    dq, dk, dv, dg = run(x, w.scale)
    rows = np.unique(np.concatenate([np.linspace(0, w.N - 1, 200).astype(np.int64), [0, 63, 64, w.N - 1]]))
    ridx = torch.from_numpy(rows).cuda()
    for h in (0, 17, 31):
        f = {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in x.items()}
        sub = {k: f[k][:, rows] for k in ("q", "do", "g")}
        rq, _, _, rg = oracle.softmax_anchor_backward(sub["q"], f["k"], f["v"], sub["do"], sub["g"], w.scale)
        e_q = normwise(host(dq[:, ridx, h:h + 1]), rq)
        e_g = normwise(host(dg[:, ridx, h:h + 1]), rg)
        # sum_j dv_j = sum_i dY_i with dY = dO sigmoid(g); sum_j dk_j = 0
        dy_sum = np.sum(f["do"] / (1.0 + np.exp(-f["g"])), axis=1)
        dv_sum = host(dv[:, :, h:h + 1].float().sum(dim=1))
        e_v = normwise(dv_sum, dy_sum)
        dkh = host(dk[:, :, h:h + 1])
        r_k = np.abs(dkh.sum(axis=1)).max() / np.abs(dkh).sum(axis=1).max()
        say(f"[anchor bwd] head {h}: dq {e_q:.3e} dg {e_g:.3e} sum dv {e_v:.3e} |sum dk|/sum|dk| {r_k:.2e}")
        assert e_q <= TOL_BF16 and e_g <= TOL_BF16 and e_v <= TOL_BF16 and r_k <= 1e-3


@pytest.mark.parametrize("N", [1, 65, 300, 1000])
@pytest.mark.parametrize("gated", [True, False])
def test_anchor_lse_and_saved_backward(N, gated):
    """hla_softmax_anchor_lse: o bitwise equal to hla_softmax_anchor, lse against the oracle's
    normaliser (max abs 1e-2: a relative error of 1e-2 in the weights); the backward from that
    saved o and lse against the oracle gradients."""
    B, H = 2, 3
    x = inputs(1100 + N, B, N, H, gated)
    d = {k: dev(v) for k, v in x.items()}
    o, lse = hla.hla_softmax_anchor_lse(d["q"], d["k"], d["v"], d.get("g"), 0.125)
    o_plain = hla.hla_softmax_anchor(d["q"], d["k"], d["v"], d.get("g"), 0.125)
    grads = hla.hla_softmax_anchor_backward_saved(d["q"], d["k"], d["v"], o, lse, d["do"], d.get("g"), 0.125)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)
    f = {k: synth.to_f64(v) for k, v in x.items()}
    lse_ref = oracle.softmax_anchor_lse(f["q"], f["k"], 0.125)
    e_lse = np.abs(host(lse) - lse_ref).max()
    say(f"[anchor saved] N={N} gated={gated}: lse max abs {e_lse:.3e}")
    assert e_lse <= 1e-2
    ref = oracle.softmax_anchor_backward(f["q"], f["k"], f["v"], f["do"], f.get("g"), 0.125)
    names = ("dq", "dk", "dv", "dg") if gated else ("dq", "dk", "dv")
    for nm, got, r in zip(names, grads, ref):
        if N == 1 and nm in ("dq", "dk"):
            # one key: dq, dk vanish; bound them by the size of the cancelling terms
            s = 1.0 if not gated else 1.0 / (1.0 + np.exp(-f["g"]))
            term = np.abs(np.sum(f["do"] * s * f["v"], axis=-1, keepdims=True))
            other = f["k"] if nm == "dq" else f["q"]
            assert np.abs(host(got)).max() <= TOL_BF16 * 0.125 * np.max(term * np.abs(other)), nm
            continue
        e = normwise(host(got), r)
        say(f"[anchor saved] N={N} {nm}: {e:.3e}")
        assert e <= TOL_BF16, nm
    if not gated:
        assert grads[3] is None


def test_anchor_saved_backward_720p5s():
    """720p/5s (B1 H32 N75600, gated): the backward from the saved forward against the recomputing
    backward (normwise) and through the identities sum_j dv_j = sum_i dY_i and sum_j dk_j = 0."""
    w = synth.HYBRID_ANCHOR
    x = w.draw()
    x["do"] = synth.randn(w.seed, (w.B, w.N, w.H, w.D), stream=4)
    d = {k: dev(v) for k, v in x.items()}
    say(f"[anchor saved] {w.name}: N={w.N} H={w.H}")
    o, lse = hla.hla_softmax_anchor_lse(d["q"], d["k"], d["v"], d["g"], w.scale)
    saved = hla.hla_softmax_anchor_backward_saved(d["q"], d["k"], d["v"], o, lse, d["do"], d["g"], w.scale)
    again = hla.hla_softmax_anchor_backward_saved(d["q"], d["k"], d["v"], o, lse, d["do"], d["g"], w.scale)
    full = hla.hla_softmax_anchor_backward(d["q"], d["k"], d["v"], d["do"], d["g"], w.scale)
    torch.cuda.synchronize()
    for a, b in zip(saved, again):
        assert torch.equal(a, b)
    for nm, a, b in zip(("dq", "dk", "dv", "dg"), saved, full):
        e = normwise(host(a), host(b).astype(np.float64))
        say(f"[anchor saved] {nm} vs recomputing backward: {e:.3e}")
        assert e <= TOL_BF16, nm
    for h in (0, 31):
        f = {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in x.items()}
        dy_sum = np.sum(f["do"] / (1.0 + np.exp(-f["g"])), axis=1)
        e_v = normwise(host(saved[2][:, :, h:h + 1].float().sum(dim=1)), dy_sum)
        dkh = host(saved[1][:, :, h:h + 1])
        r_k = np.abs(dkh.sum(axis=1)).max() / np.abs(dkh).sum(axis=1).max()
        say(f"[anchor saved] head {h}: sum dv {e_v:.3e} |sum dk|/sum|dk| {r_k:.2e}")
        assert e_v <= TOL_BF16 and r_k <= 1e-3

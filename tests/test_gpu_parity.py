"""GPU parity: libhla (through its C ABI) against the fp64 oracle.

Inputs come from the seeded generator ``synth``; the oracle decodes the same
bf16 bits. The error measure is normwise, max|got - ref| / max|ref| over the
compared outputs (outputs are zero-mean, so an elementwise relative error is
ill-posed); bars: 1e-2 for bf16 inputs, 1e-5 for float inputs. The oracle is
called head by head (heads are independent in the definition; a per-head
einsum is much faster than one over all heads).
"""
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from softmax_attention_relu_amd import hla

from gpu_common import TOL_BF16, TOL_F32, dev, host, normwise, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def tol(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def oracle_linear_per_head(x, grid, chunk=0, rows=None, heads=None, bands=(16, 24, 24), t_offset=0, kv_in=None,
                           ksum_in=None):
    """Oracle outputs of shape (B, len(rows), len(heads), 64) and the states (B, len(heads), 64, 64), (B, len(heads), 64)."""
    B, N, H, D = x["q"].shape
    heads = range(H) if heads is None else heads
    rope = None if grid is None else oracle.Rope3D(grid, bands, t_offset=t_offset)
    outs, kvs, kss = [], [], []
    for h in heads:
        f = {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in x.items()}
        g = f.get("g")
        if chunk:
            kin = None if kv_in is None else kv_in[:, h:h + 1]
            sin = None if ksum_in is None else ksum_in[:, h:h + 1]
            o, kv, ks = oracle.linear_attention_chunked(f["q"], f["k"], f["v"], chunk, g, rope, kv_in=kin,
                                                        ksum_in=sin, rows=rows)
        else:
            o, kv, ks = oracle.linear_attention(f["q"], f["k"], f["v"], g, rope, rows=rows, return_state=True)
        outs.append(o)
        kvs.append(kv)
        kss.append(ks)
    return np.concatenate(outs, axis=2), np.concatenate(kvs, axis=1), np.concatenate(kss, axis=1)


def run_linear(x, grid, chunk=0, bands=(16, 24, 24), t_offset=0, kv_in=None, ksum_in=None, want_state=False,
               rope_tables=None):
    d = {k: dev(v) for k, v in x.items()}
    rope = None
    if grid is not None:
        rope = hla.Rope3D(grid, bands, t_offset=t_offset, tables=rope_tables)
    if chunk:
        B, N, H, _ = x["q"].shape
        kin = None if kv_in is None else torch.from_numpy(kv_in.astype(np.float32)).cuda()
        sin = None if ksum_in is None else torch.from_numpy(ksum_in.astype(np.float32)).cuda()
        kvo = torch.empty((B, H, 64, 64), dtype=torch.float32, device="cuda") if want_state else None
        kso = torch.empty((B, H, 64), dtype=torch.float32, device="cuda") if want_state else None
        o = hla.hla_linear_attn_chunked(d["q"], d["k"], d["v"], chunk, d.get("g"), rope, kv_in=kin, ksum_in=sin,
                                        kv_out=kvo, ksum_out=kso)
        torch.cuda.synchronize()
        if want_state:
            return o, kvo, kso
        return o
    o = hla.hla_linear_attn(d["q"], d["k"], d["v"], d.get("g"), rope)
    torch.cuda.synchronize()
    return o


# ----------------------------------------------------------------------------
# linear attention at the measured sizes

@pytest.mark.parametrize("w", [synth.LINEAR_F32_N1024, synth.LINEAR_CFGPAIR_N32760, synth.LINEAR_720P5S],
                         ids=lambda w: w.name)
def test_linear_full_size(w):
    say(f"[parity] {w.name}: B={w.B} N={w.N} H={w.H} dtype={w.dtype} gated={w.gated}")
    x = w.draw()
    got = host(run_linear(x, w.grid))
    ref, _, _ = oracle_linear_per_head(x, w.grid)
    err = normwise(got, ref)
    per_head = max(normwise(got[:, :, h], ref[:, :, h]) for h in range(w.H))
    say(f"[parity] {w.name}: normwise {err:.3e}, worst head {per_head:.3e}")
    assert err <= tol(w.dtype)
    assert per_head <= tol(w.dtype)


def test_hybrid_linear_layer_sampled_heads():
    w = synth.HYBRID_LINEAR[0]
    say(f"[parity] {w.name}")
    x = w.draw()
    got = host(run_linear(x, w.grid))
    heads = [0, 9, 22, 31]
    ref, _, _ = oracle_linear_per_head(x, w.grid, heads=heads)
    err = normwise(got[:, :, heads], ref)
    say(f"[parity] {w.name}: heads {heads} normwise {err:.3e}")
    assert err <= TOL_BF16


def test_chunked_720p60s_sampled():
    w = synth.CHUNKED_720P60S
    say(f"[parity] {w.name}: N={w.N} L={w.chunk_tokens} (drawing inputs)")
    x = w.draw()
    o, kvo, kso = run_linear(x, w.grid, chunk=w.chunk_tokens, want_state=True)
    say("[parity] chunked: GPU done")
    rows = np.unique(np.concatenate([np.arange(0, w.N, 1013), np.arange(35990, 36010), [w.N - 3600, w.N - 1]]))
    got = host(o[:, torch.from_numpy(rows).cuda()])
    heads = [0, 17, 31]
    ref, kv_ref, ks_ref = oracle_linear_per_head(x, w.grid, chunk=w.chunk_tokens, rows=rows, heads=heads)
    err = normwise(got[:, :, heads], ref)
    kv_err = normwise(host(kvo)[:, heads], kv_ref)
    ks_err = normwise(host(kso)[:, heads], ks_ref)
    say(f"[parity] chunked: out {err:.3e} kv_out {kv_err:.3e} ksum_out {ks_err:.3e}")
    assert err <= TOL_BF16
    assert kv_err <= TOL_BF16
    assert ks_err <= 1e-5


# ----------------------------------------------------------------------------
# small and ragged shapes

GRIDS = {1: (1, 1, 1), 7: (7, 1, 1), 63: (7, 3, 3), 64: (4, 4, 4), 65: (5, 13, 1), 300: (3, 10, 10),
         1000: (10, 10, 10)}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N", sorted(GRIDS))
@pytest.mark.parametrize("rope,gated", [(True, True), (False, False), (True, False)])
def test_linear_small_shapes(dtype, N, rope, gated):
    B, H = 2, 3
    shp = (B, N, H, 64)
    names = ["q", "k", "v"] + (["g"] if gated else [])
    x = {nm: synth.randn(100 + N, shp, dtype=dtype, stream=i) for i, nm in enumerate(names)}
    grid = GRIDS[N] if rope else None
    got = host(run_linear(x, grid))
    ref, _, _ = oracle_linear_per_head(x, grid)
    err = normwise(got, ref)
    assert err <= tol(dtype), err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,L", [(300, 64), (300, 100), (300, 1), (1000, 300), (65, 1000), (1000, 17)])
def test_chunked_small_shapes(dtype, N, L):
    B, H = 1, 2
    grid = GRIDS[N]
    x = {nm: synth.randn(200 + N + L, (B, N, H, 64), dtype=dtype, stream=i) for i, nm in enumerate("qkvg")}
    kv_in = synth.randn(7, (B, H, 64, 64), dtype="f32").astype(np.float64)
    ks_in = np.abs(synth.randn(8, (B, H, 64), dtype="f32").astype(np.float64)) * 10
    o, kvo, kso = run_linear(x, grid, chunk=L, kv_in=kv_in, ksum_in=ks_in, want_state=True)
    ref, kv_ref, ks_ref = oracle_linear_per_head(x, grid, chunk=L, kv_in=kv_in, ksum_in=ks_in)
    assert normwise(host(o), ref) <= tol(dtype)
    assert normwise(host(kvo), kv_ref) <= tol(dtype)
    assert normwise(host(kso), ks_ref) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("grid,bands,chunk", [
    ((6, 10, 10), (18, 22, 24), 0),     # band widths not multiples of 8: every pair looked up alone
    ((6, 10, 10), (18, 22, 24), 250),
    ((600, 1, 1), (16, 24, 24), 0),     # 9648 table floats: too large to stage in LDS
    ((600, 1, 1), (16, 24, 24), 128),
    ((12, 5, 10), (16, 24, 24), 0),     # staged in LDS
])
def test_linear_rope_table_paths(dtype, grid, bands, chunk):
    N = grid[0] * grid[1] * grid[2]
    x = {nm: synth.randn(500 + N + chunk, (1, N, 3, 64), dtype=dtype, stream=i) for i, nm in enumerate("qkvg")}
    got = host(run_linear(x, grid, chunk=chunk, bands=bands))
    ref, _, _ = oracle_linear_per_head(x, grid, chunk=chunk, bands=bands)
    err = normwise(got, ref)
    assert err <= tol(dtype), err


def test_chunked_resume_and_aliasing():
    """Two calls carrying the state (second with t_offset, state updated in place) equal one call."""
    grid, L = (10, 10, 10), 200
    x = {nm: synth.randn(301, (1, 1000, 2, 64), stream=i) for i, nm in enumerate("qkv")}
    full, kv_full, ks_full = run_linear(x, grid, chunk=L, want_state=True)
    d = {k: dev(v) for k, v in x.items()}
    kv = torch.zeros((1, 2, 64, 64), dtype=torch.float32, device="cuda")
    ks = torch.zeros((1, 2, 64), dtype=torch.float32, device="cuda")
    outs = []
    for t0, sl in ((0, slice(0, 600)), (6, slice(600, 1000))):
        frames = (sl.stop - sl.start) // 100
        rope = hla.Rope3D((frames, 10, 10), t_offset=t0)
        q, k, v = (d[n][:, sl].contiguous() for n in "qkv")
        outs.append(hla.hla_linear_attn_chunked(q, k, v, L, None, rope, kv_in=kv, ksum_in=ks, kv_out=kv, ksum_out=ks))
    torch.cuda.synchronize()
    split = host(torch.cat(outs, dim=1))
    ref, kv_ref, ks_ref = oracle_linear_per_head(x, grid, chunk=L)
    assert normwise(split, ref) <= TOL_BF16
    assert normwise(host(kv), kv_ref) <= TOL_BF16
    assert normwise(host(ks), ks_ref) <= 1e-5
    # same arithmetic on both paths except the partial split: states agree to fp32 rounding
    assert normwise(host(kv), host(kv_full)) <= 1e-5


# ----------------------------------------------------------------------------
# edge cases and determinism

def test_linear_edge_cases_and_determinism():
    N, grid = 1000, (10, 10, 10)
    x = {nm: synth.randn(400, (1, N, 2, 64), stream=i) for i, nm in enumerate("qkv")}
    q = x["q"].copy()
    q[0, 5, 1] = synth.randn(401, (64,)) | np.uint16(0x8000)  # all-negative row -> relu(q) = 0
    x["q"] = q
    base = run_linear(x, grid)
    b = host(base)
    assert np.all(b[0, 5, 1] == 0.0)
    again = run_linear(x, grid)
    assert torch.equal(base, again), "repeat call is not bitwise identical"
    # G = 0 halves the output exactly
    xg = dict(x, g=np.zeros_like(x["q"]))
    assert torch.equal(run_linear(xg, grid), base / 2)
    # zero-angle tables reduce to no RoPE
    zero = [np.tile(np.array([1.0, 0.0], np.float32), (n, d // 2, 1)) for n, d in zip(grid, (16, 24, 24))]
    assert torch.equal(run_linear(x, grid, rope_tables=zero), run_linear(x, None))
    # a head whose keys are all negative has an empty state and key sum: o = 0 / (0 + eps) = 0 exactly,
    # in every form (bidirectional, chunked, token-causal), and the other head is untouched
    k = x["k"].copy()
    k[:, :, 0] |= np.uint16(0x8000)
    xk = dict(x, k=k)
    for o in (run_linear(xk, grid), run_linear(xk, grid, chunk=300),
              hla.hla_linear_attn_causal(*(dev(xk[n]) for n in "qkv"), None, hla.Rope3D(grid))):
        torch.cuda.synchronize()
        assert torch.count_nonzero(o[:, :, 0]).item() == 0
    assert torch.equal(run_linear(xk, grid)[:, :, 1], base[:, :, 1])
    # zero values: o = 0 exactly
    assert torch.count_nonzero(run_linear(dict(x, v=np.zeros_like(x["v"])), grid)).item() == 0


# ----------------------------------------------------------------------------
# softmax anchor

def run_anchor(x):
    d = {k: dev(v) for k, v in x.items()}
    o = hla.hla_softmax_anchor(d["q"], d["k"], d["v"], d.get("g"))
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("N", [1, 63, 64, 65, 300, 1000])
@pytest.mark.parametrize("gated", [True, False])
def test_anchor_small_shapes(N, gated):
    names = ["q", "k", "v"] + (["g"] if gated else [])
    x = {nm: synth.randn(500 + N, (2, N, 2, 64), stream=i) for i, nm in enumerate(names)}
    got = host(run_anchor(x))
    f = {k: synth.to_f64(v) for k, v in x.items()}
    ref = oracle.softmax_anchor(f["q"], f["k"], f["v"], f.get("g"), scale=0.125)
    assert normwise(got, ref) <= TOL_BF16


def test_anchor_large_logits():
    """Q scaled by 8: sharp softmax rows, exercises the reference-max refresh."""
    x = {nm: synth.randn(600, (1, 2000, 2, 64), std=8.0 if nm == "q" else 1.0, stream=i) for i, nm in enumerate("qkv")}
    got = host(run_anchor(x))
    f = {k: synth.to_f64(v) for k, v in x.items()}
    ref = oracle.softmax_anchor(f["q"], f["k"], f["v"], None, scale=0.125)
    assert normwise(got, ref) <= TOL_BF16


@pytest.mark.parametrize("q_std", [1.0, 2.0])
def test_anchor_half_and_bf16_score_paths(q_std):
    """The forward's two loops: half-precision scores where the static logit bound holds and |q|, |k|,
    |v| are within range, the bf16 running max otherwise. Power-of-two factors leave the exact result
    unchanged but move the inputs across the range bounds: v * 2^44 (|v| > 2^40), and k * 2^11 with
    q * 2^-11 (|k| > 2^10, same logits). Each output is checked against the oracle; that each factor
    changed the loop shows in the bits (the same loop would give exactly the scaled output). q_std 2
    puts the bound near its limit (b up to ~40 in log2 units)."""
    x = {nm: synth.randn(610, (1, 2000, 2, 64), std=q_std if nm == "q" else 1.0, stream=i)
         for i, nm in enumerate("qkvg")}
    f = {k: synth.to_f64(v) for k, v in x.items()}
    ref = oracle.softmax_anchor(f["q"], f["k"], f["v"], f["g"], scale=0.125)
    d = {k: dev(v) for k, v in x.items()}
    half = hla.hla_softmax_anchor(d["q"], d["k"], d["v"], d["g"], 0.125)
    big_v = hla.hla_softmax_anchor(d["q"], d["k"], d["v"] * 2.0 ** 44, d["g"], 0.125)
    big_k = hla.hla_softmax_anchor(d["q"] * 2.0 ** -11, d["k"] * 2.0 ** 11, d["v"], d["g"], 0.125)
    torch.cuda.synchronize()
    assert normwise(host(half), ref) <= TOL_BF16
    assert normwise(host(big_v) * 2.0 ** -44, ref) <= TOL_BF16
    assert normwise(host(big_k), ref) <= TOL_BF16
    assert not torch.equal(big_v, half * 2.0 ** 44)
    assert not torch.equal(big_k, half)


@pytest.mark.parametrize("scale", [0.01, 0.0625, 0.5, 2.0])
def test_anchor_scales(scale):
    """Scales other than 1/sqrt(D): small ones keep the static bound (half-precision scores), large
    ones exceed it (running max); each against the oracle at that scale."""
    x = {nm: synth.randn(620, (1, 1500, 2, 64), stream=i) for i, nm in enumerate("qkvg")}
    d = {k: dev(v) for k, v in x.items()}
    got = host(hla.hla_softmax_anchor(d["q"], d["k"], d["v"], d["g"], scale))
    torch.cuda.synchronize()
    f = {k: synth.to_f64(v) for k, v in x.items()}
    ref = oracle.softmax_anchor(f["q"], f["k"], f["v"], f["g"], scale=scale)
    assert normwise(got, ref) <= TOL_BF16


def test_anchor_loops_mixed_in_one_call():
    """One call whose work-groups take different loops: head 0 all half precision; in head 1 the rows
    600-649 are scaled by 8 (beyond the static bound), so only the 512-row work-group holding them takes
    the running max; head 2's values are scaled by 2^44 (beyond the |v| bound), all running max. Every
    head against the oracle."""
    x = {nm: synth.randn(630, (1, 1200, 3, 64), stream=i) for i, nm in enumerate("qkvg")}
    f = {k: synth.to_f64(v) for k, v in x.items()}
    f["q"][:, 600:650, 1] *= 8.0
    f["v"][:, :, 2] *= 2.0 ** 44
    d = {k: dev(v) for k, v in x.items()}  # the same power-of-two factors, exact in bf16
    d["q"][:, 600:650, 1] *= 8.0
    d["v"][:, :, 2] *= 2.0 ** 44
    got = host(hla.hla_softmax_anchor(d["q"], d["k"], d["v"], d["g"], 0.125))
    torch.cuda.synchronize()
    ref = oracle.softmax_anchor(f["q"], f["k"], f["v"], f["g"], scale=0.125)
    for h in range(3):
        assert normwise(got[:, :, h], ref[:, :, h]) <= TOL_BF16, h


def test_anchor_full_size_sampled_rows():
    w = synth.HYBRID_ANCHOR
    say(f"[parity] {w.name}: N={w.N} H={w.H}")
    x = w.draw()
    o = run_anchor(x)
    rows = np.unique(np.concatenate([np.linspace(0, w.N - 1, 512).astype(np.int64), [w.N - 1]]))
    got = host(o[:, torch.from_numpy(rows).cuda()])
    worst = 0.0
    for h in range(w.H):
        f = {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in x.items()}
        ref = oracle.softmax_anchor(f["q"], f["k"], f["v"], f["g"], scale=w.scale, rows=rows)
        worst = max(worst, normwise(got[:, :, h:h + 1], ref))
    say(f"[parity] anchor: worst head normwise {worst:.3e}")
    assert worst <= TOL_BF16


# ----------------------------------------------------------------------------
# router

def run_route(srcs, w, phi, eps=1e-6, dtype="bf16"):
    ds = [dev(s) for s in srcs]
    wd = torch.from_numpy(w).cuda()
    pd = None if phi is None else torch.from_numpy(phi).cuda()
    h, a = hla.hla_attnres_route(ds, wd, pd, eps, alpha=True)
    torch.cuda.synchronize()
    return h, a


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S,C", [(1, 64), (2, 8), (4, 2048), (5, 520), (16, 1024), (4, 4096), (3, 1032), (16, 4096)])
@pytest.mark.parametrize("with_phi", [True, False])
def test_route_small_shapes(dtype, S, C, with_phi):
    B, T = 2, 37
    srcs = [synth.randn(700 + S + C, (B, T, C), dtype=dtype, stream=i) for i in range(S)]
    w = synth.randn(701, (C,), std=0.02, dtype="f32")
    phi = synth.randn(702, (B, C), std=0.02, dtype="f32") if with_phi else None
    h, a = run_route(srcs, w, phi, dtype=dtype)
    ref_h, ref_a = oracle.attnres_route([synth.to_f64(s) for s in srcs], w.astype(np.float64),
                                        None if phi is None else phi.astype(np.float64))
    assert normwise(host(h), ref_h) <= tol(dtype)
    assert np.abs(host(a) - ref_a).max() <= (1e-5 if dtype == "bf16" else 1e-6)


def test_route_large_query_sharp_softmax():
    srcs = [synth.randn(800, (1, 64, 256), stream=i) for i in range(4)]
    w = synth.randn(801, (256,), std=3.0, dtype="f32")
    h, a = run_route(srcs, w, None)
    ref_h, ref_a = oracle.attnres_route([synth.to_f64(s) for s in srcs], w.astype(np.float64), None)
    assert normwise(host(h), ref_h) <= TOL_BF16
    assert np.abs(host(a) - ref_a).max() <= 1e-4


def test_route_full_size():
    wk = synth.HYBRID_ROUTES[0]
    say(f"[parity] {wk.name}")
    x = wk.draw()
    h, a = run_route(x["v"], x["w"], x["phi_t"])
    ref_h, ref_a = oracle.attnres_route([synth.to_f64(s) for s in x["v"]], x["w"].astype(np.float64),
                                        x["phi_t"].astype(np.float64))
    err = normwise(host(h), ref_h)
    say(f"[parity] route: h normwise {err:.3e}, alpha max abs {np.abs(host(a) - ref_a).max():.3e}")
    assert err <= TOL_BF16
    assert np.abs(host(a) - ref_a).max() <= 1e-5


# ----------------------------------------------------------------------------
# golden fixtures (oracle values stored by tests/golden/make_golden.py)

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        doc = json.load(f)
    return doc, {k: np.asarray(v).reshape(doc["shapes"][k]) for k, v in doc["outputs"].items()}


def test_golden_fixtures_on_gpu():
    doc, outs = _golden("linear_gated_2x2x3.json")
    inp = doc["inputs"]
    x = {nm: synth.randn(inp["seed"], inp["shape"], stream=s) for nm, s in inp["streams"].items()}
    assert normwise(host(run_linear(x, tuple(doc["grid"]))), outs["o"]) <= TOL_BF16

    doc, outs = _golden("chunked_5x2x2_L6.json")
    inp = doc["inputs"]
    x = {nm: synth.randn(inp["seed"], inp["shape"], stream=s) for nm, s in inp["streams"].items()}
    o, kvo, kso = run_linear(x, tuple(doc["grid"]), chunk=doc["chunk_tokens"], want_state=True)
    assert normwise(host(o), outs["o"]) <= TOL_BF16
    assert normwise(host(kvo), outs["kv_out"]) <= TOL_BF16

    doc, outs = _golden("anchor_N40.json")
    inp = doc["inputs"]
    x = {nm: synth.randn(inp["seed"], inp["shape"], stream=s) for nm, s in inp["streams"].items()}
    assert normwise(host(run_anchor(x)), outs["o"]) <= TOL_BF16

    doc, outs = _golden("route_B2T3C64S4.json")
    inp = doc["inputs"]
    shp = inp["sources"]["shape"]
    srcs = [synth.randn(inp["seed"], shp, stream=s) for s in inp["sources"]["streams"]]
    w = synth.randn(inp["seed"], (shp[2],), std=0.02, dtype="f32", stream=100)
    phi = synth.randn(inp["seed"], (shp[0], shp[2]), std=0.02, dtype="f32", stream=101)
    h, a = run_route(srcs, w, phi)
    assert normwise(host(h), outs["h"]) <= TOL_BF16

"""GPU parity of the linear-attention gradients against the fp64 oracle.

hla_linear_attn_backward is compared with ``oracle.linear_attention_backward``
and hla_linear_attn_chunked_backward with
``oracle.linear_attention_chunked_backward`` (both pinned in
tests/test_oracle.py to autograd of independent forwards and to central
differences). Shapes span several 32-token steps and parts, ragged tails and
chunks, a single token, a head count that leaves a head group part-empty,
both RoPE table paths, carried and returned cache gradients, and the 720p/5s
shape on whole heads.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from softmax_attention_relu_amd import hla

from gpu_common import TOL_BF16, dev, host, normwise, say

pytestmark = pytest.mark.gpu

GRIDS = {1: (1, 1, 1), 31: (31, 1, 1), 33: (3, 11, 1), 100: (4, 5, 5), 300: (3, 10, 10), 1000: (10, 10, 10)}
ALIGNED = (16, 24, 24)
UNALIGNED = (18, 22, 24)  # band widths not multiples of 8: per-pair table lookups


def inputs(seed, B, N, H, gated):
    names = ["q", "k", "v", "do"] + (["g"] if gated else [])
    return {nm: synth.randn(seed, (B, N, H, 64), stream=i) for i, nm in enumerate(names)}


def check(name, got, ref, tol=TOL_BF16):
    e = normwise(got, ref)
    say(f"[bwd] {name}: {e:.3e}")
    assert e <= tol, name


@pytest.mark.parametrize("N", sorted(GRIDS))
@pytest.mark.parametrize("bands,gated", [(ALIGNED, True), (None, False), (UNALIGNED, True)])
def test_backward_small_shapes(N, bands, gated):
    B, H = 2, 3
    x = inputs(800 + N, B, N, H, gated)
    d = {k: dev(v) for k, v in x.items()}
    rope = None if bands is None else hla.Rope3D(GRIDS[N], bands)
    say(f"[bwd] bidirectional N={N} bands={bands} gated={gated}")
    dq, dk, dv, dg = hla.hla_linear_attn_backward(d["q"], d["k"], d["v"], d["do"], d.get("g"), rope)
    torch.cuda.synchronize()
    f = {k: synth.to_f64(v) for k, v in x.items()}
    ref = oracle.linear_attention_backward(f["q"], f["k"], f["v"], f["do"], f.get("g"),
                                           None if bands is None else oracle.Rope3D(GRIDS[N], bands))
    if N == 1:
        # One token: o = v (phi_q . phi_k) / (phi_q . phi_k + eps) hardly depends on q or k, and dq, dk are
        # differences of two terms of size |phi_k| |v . dY| / den (resp. |phi_q| ...) that cancel to eps / den.
        # Their rounding is bounded by those terms, not by the tiny result.
        fq, fk = np.maximum(f["q"], 0), np.maximum(f["k"], 0)
        den = np.sum(fq * fk, axis=-1, keepdims=True) + 1e-6
        s = 1.0 if not gated else 1.0 / (1.0 + np.exp(-f["g"]))
        vdy = np.abs(np.sum(f["v"] * f["do"] * s, axis=-1, keepdims=True)) / den
        for nm, got, r, phi in (("dq", dq, ref[0], fk), ("dk", dk, ref[1], fq)):
            err = np.abs(host(got) - r).max()
            say(f"[bwd] {nm} (one token): error {err:.3e} of term size {np.max(phi * vdy):.3e}")
            assert err <= TOL_BF16 * np.max(phi * vdy)
        check("dv", host(dv), ref[2])
    else:
        for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            check(nm, host(got), r)
    if gated:
        check("dg", host(dg), ref[3])
    else:
        assert dg is None


@pytest.mark.parametrize("N,L,bands", [(1000, 300, ALIGNED), (1000, 32, None), (300, 7, UNALIGNED), (33, 100, ALIGNED)])
def test_chunked_backward_with_cache(N, L, bands):
    B, H = 2, 3
    x = inputs(850 + L, B, N, H, True)
    kv_in = synth.randn(851, (B, H, 64, 64), dtype="f32").astype(np.float64)
    ks_in = np.abs(synth.randn(852, (B, H, 64), dtype="f32").astype(np.float64)) * 10
    dkv_out = synth.randn(853, (B, H, 64, 64), dtype="f32").astype(np.float64) * 1e-3
    dks_out = synth.randn(854, (B, H, 64), dtype="f32").astype(np.float64) * 1e-3
    d = {k: dev(v) for k, v in x.items()}
    t32 = lambda a: torch.from_numpy(a.astype(np.float32)).cuda()
    rope = None if bands is None else hla.Rope3D(GRIDS[N], bands)
    dkv_in = torch.empty((B, H, 64, 64), dtype=torch.float32, device="cuda")
    dks_in = torch.empty((B, H, 64), dtype=torch.float32, device="cuda")
    say(f"[bwd] chunked N={N} L={L} bands={bands}")
    dq, dk, dv, dg = hla.hla_linear_attn_chunked_backward(d["q"], d["k"], d["v"], d["do"], L, d["g"], rope,
                                                          kv_in=t32(kv_in), ksum_in=t32(ks_in), dkv_out=t32(dkv_out),
                                                          dksum_out=t32(dks_out), dkv_in=dkv_in, dksum_in=dks_in)
    # the cache gradient updated in place gives the same result
    g_kv, g_ks = t32(dkv_out), t32(dks_out)
    again = hla.hla_linear_attn_chunked_backward(d["q"], d["k"], d["v"], d["do"], L, d["g"], rope,
                                                 kv_in=t32(kv_in), ksum_in=t32(ks_in), dkv_out=g_kv,
                                                 dksum_out=g_ks, dkv_in=g_kv, dksum_in=g_ks)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv, dg, dkv_in, dks_in), (*again, g_kv, g_ks)):
        assert torch.equal(a, b), "in-place cache gradient differs"
    f = {k: synth.to_f64(v) for k, v in x.items()}
    ref = oracle.linear_attention_chunked_backward(f["q"], f["k"], f["v"], f["do"], L, f["g"],
                                                   None if bands is None else oracle.Rope3D(GRIDS[N], bands),
                                                   kv_in=kv_in, ksum_in=ks_in, dkv_out=dkv_out, dksum_out=dks_out)
    for nm, got, r in zip(("dq", "dk", "dv", "dg", "dkv_in", "dksum_in"), (dq, dk, dv, dg, dkv_in, dks_in), ref):
        check(nm, host(got), r)


def test_chunked_backward_one_chunk_equals_bidirectional():
    """chunk_tokens = N and no cache: the same kernels and split, bitwise equal outputs; repeats are too."""
    N, grid = 1000, GRIDS[1000]
    x = inputs(870, 1, N, 5, True)
    d = {k: dev(v) for k, v in x.items()}
    rope = hla.Rope3D(grid)
    a = hla.hla_linear_attn_backward(d["q"], d["k"], d["v"], d["do"], d["g"], rope)
    b = hla.hla_linear_attn_chunked_backward(d["q"], d["k"], d["v"], d["do"], N, d["g"], rope)
    c = hla.hla_linear_attn_backward(d["q"], d["k"], d["v"], d["do"], d["g"], rope)
    torch.cuda.synchronize()
    for u, w, z in zip(a, b, c):
        assert torch.equal(u, w) and torch.equal(u, z)


def test_backward_full_size_whole_heads():
    """720p/5s shape (B1 H32 N75600, gated, RoPE): three whole heads against the oracle."""
    w = synth.LINEAR_720P5S
    x = w.draw()
    x["do"] = synth.randn(w.seed, (w.B, w.N, w.H, w.D), stream=4)
    say(f"[bwd] full size {w.name}: N={w.N} H={w.H}")
    d = {k: dev(v) for k, v in x.items()}
    dq, dk, dv, dg = hla.hla_linear_attn_backward(d["q"], d["k"], d["v"], d["do"], d["g"], hla.Rope3D(w.grid))
    torch.cuda.synchronize()
    rope = oracle.Rope3D(w.grid)
    for h in (0, 13, 31):
        f = {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in x.items()}
        ref = oracle.linear_attention_backward(f["q"], f["k"], f["v"], f["do"], f["g"], rope)
        for nm, got, r in zip(("dq", "dk", "dv", "dg"), (dq, dk, dv, dg), ref):
            check(f"{nm} head {h}", host(got[:, :, h:h + 1]), r)


@pytest.mark.parametrize("N,bands,gated", [(100, ALIGNED, True), (300, None, False), (1000, UNALIGNED, True),
                                           (75600, ALIGNED, True)])
def test_backward_from_saved_state(N, bands, gated):
    """hla_linear_attn_backward_saved with the state that hla_linear_attn_chunked returns for chunk = N:
    bitwise equal to hla_linear_attn_backward (same state, same kernels afterwards); on one small shape also
    against the oracle. N = 75600 is the 720p/5s layer (B1 H32)."""
    big = N == 75600
    B, H = (1, 32) if big else (2, 3)
    grid = (21, 45, 80) if big else GRIDS[N]
    x = inputs(850 + N, B, N, H, gated)
    d = {k: dev(v) for k, v in x.items()}
    rope = None if bands is None else hla.Rope3D(grid, bands)
    say(f"[bwd saved] N={N} B={B} H={H} bands={bands} gated={gated}")
    kv = torch.empty((B, H, 64, 64), dtype=torch.float32, device="cuda")
    ks = torch.empty((B, H, 64), dtype=torch.float32, device="cuda")
    o_chunk = hla.hla_linear_attn_chunked(d["q"], d["k"], d["v"], N, d.get("g"), rope, kv_out=kv, ksum_out=ks)
    o_plain = hla.hla_linear_attn(d["q"], d["k"], d["v"], d.get("g"), rope)
    saved = hla.hla_linear_attn_backward_saved(d["q"], d["k"], d["v"], kv, ks, d["do"], d.get("g"), rope)
    full = hla.hla_linear_attn_backward(d["q"], d["k"], d["v"], d["do"], d.get("g"), rope)
    torch.cuda.synchronize()
    assert torch.equal(o_chunk, o_plain)
    for nm, a, b in zip(("dq", "dk", "dv", "dg"), saved, full):
        if b is None:
            assert a is None
            continue
        assert torch.equal(a, b), nm
    if N == 100:
        f = {k: synth.to_f64(v) for k, v in x.items()}
        ref = oracle.linear_attention_backward(f["q"], f["k"], f["v"], f["do"], f.get("g"),
                                               oracle.Rope3D(grid, bands))
        for nm, got, r in zip(("dq", "dk", "dv", "dg"), saved, ref):
            check(f"saved {nm}", host(got), r)

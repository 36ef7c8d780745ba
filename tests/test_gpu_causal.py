"""GPU parity of token-causal linear attention (hla_linear_attn_causal) against the fp64 oracle.

The oracle is ``oracle.linear_attention_causal`` (the causal equation of the
SANA-Video notes, section 3.4, written out per row; pinned in
tests/test_oracle.py). Shapes span several 32-token steps and ranges, ragged
tails, a single token, carried state in and out, and the 720p/5s shape on
sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from softmax_attention_relu_amd import hla

from gpu_common import TOL_BF16, dev, host, normwise, say

pytestmark = pytest.mark.gpu

GRIDS = {1: (1, 1, 1), 5: (5, 1, 1), 31: (31, 1, 1), 32: (2, 4, 4), 33: (3, 11, 1), 64: (4, 4, 4), 100: (4, 5, 5),
         300: (3, 10, 10), 1000: (10, 10, 10)}


def run_causal(x, grid, kv_in=None, ksum_in=None, state=True):
    d = {k: dev(v) for k, v in x.items()}
    B, N, H, _ = x["q"].shape
    rope = None if grid is None else hla.Rope3D(grid)
    kin = None if kv_in is None else torch.from_numpy(kv_in.astype(np.float32)).cuda()
    sin = None if ksum_in is None else torch.from_numpy(ksum_in.astype(np.float32)).cuda()
    kvo = torch.empty((B, H, 64, 64), dtype=torch.float32, device="cuda") if state else None
    kso = torch.empty((B, H, 64), dtype=torch.float32, device="cuda") if state else None
    o = hla.hla_linear_attn_causal(d["q"], d["k"], d["v"], d.get("g"), rope, kv_in=kin, ksum_in=sin, kv_out=kvo,
                                   ksum_out=kso)
    torch.cuda.synchronize()
    return o, kvo, kso


def oracle_causal(x, grid, kv_in=None, ksum_in=None, rows=None, heads=None):
    B, N, H, _ = x["q"].shape
    heads = range(H) if heads is None else heads
    rope = None if grid is None else oracle.Rope3D(grid)
    outs, kvs, kss = [], [], []
    for h in heads:
        f = {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in x.items()}
        o, kv, ks = oracle.linear_attention_causal(
            f["q"], f["k"], f["v"], f.get("g"), rope, kv_in=None if kv_in is None else kv_in[:, h:h + 1],
            ksum_in=None if ksum_in is None else ksum_in[:, h:h + 1], rows=rows)
        outs.append(o)
        kvs.append(kv)
        kss.append(ks)
    return np.concatenate(outs, axis=2), np.concatenate(kvs, axis=1), np.concatenate(kss, axis=1)


@pytest.mark.parametrize("N", sorted(GRIDS))
@pytest.mark.parametrize("rope,gated,carry", [(True, True, False), (False, False, False), (True, False, True)])
def test_causal_small_shapes(N, rope, gated, carry):
    B, H = 2, 3
    names = ["q", "k", "v"] + (["g"] if gated else [])
    x = {nm: synth.randn(700 + N, (B, N, H, 64), stream=i) for i, nm in enumerate(names)}
    kv_in = synth.randn(701, (B, H, 64, 64), dtype="f32").astype(np.float64) if carry else None
    ks_in = np.abs(synth.randn(702, (B, H, 64), dtype="f32").astype(np.float64)) * 10 if carry else None
    grid = GRIDS[N] if rope else None
    o, kvo, kso = run_causal(x, grid, kv_in, ks_in)
    ref, kv_ref, ks_ref = oracle_causal(x, grid, kv_in, ks_in)
    assert normwise(host(o), ref) <= TOL_BF16
    assert normwise(host(kvo), kv_ref) <= TOL_BF16
    assert normwise(host(kso), ks_ref) <= 1e-5


@pytest.mark.parametrize("grid", [(600, 1, 1), (1, 2, 300), (8, 12, 10)])
def test_causal_rope_table_paths(grid):
    """RoPE table sets of up to 9 216 floats (36 KB) are read from an LDS copy (8x12x10: 656
    floats; 1x2x300: 7 264, a long w table), larger ones from global memory (600x1x1: 9 648).
    Each against the oracle, gated, with a carried state."""
    B, H = 1, 2
    N = grid[0] * grid[1] * grid[2]
    x = {nm: synth.randn(760 + N, (B, N, H, 64), stream=i) for i, nm in enumerate("qkvg")}
    kv_in = synth.randn(761, (B, H, 64, 64), dtype="f32").astype(np.float64)
    ks_in = np.abs(synth.randn(762, (B, H, 64), dtype="f32").astype(np.float64)) * 10
    floats = grid[0] * 16 + grid[1] * 24 + grid[2] * 24
    say(f"[causal] rope grid {grid}: {floats} table floats ({'global' if floats > 9216 else 'LDS'} lookups)")
    o, kvo, kso = run_causal(x, grid, kv_in, ks_in)
    ref, kv_ref, ks_ref = oracle_causal(x, grid, kv_in, ks_in)
    e = normwise(host(o), ref)
    say(f"[causal] rope grid {grid}: normwise {e:.3e}")
    assert e <= TOL_BF16
    assert normwise(host(kvo), kv_ref) <= TOL_BF16
    assert normwise(host(kso), ks_ref) <= 1e-5


def test_causal_in_place_state_determinism_and_resume():
    """kv_out == kv_in updates in place; two calls carrying the state equal one call; repeats are bitwise equal."""
    grid = (10, 10, 10)
    x = {nm: synth.randn(710, (1, 1000, 2, 64), stream=i) for i, nm in enumerate("qkvg")}
    full, kv_full, ks_full = run_causal(x, grid)
    again, _, _ = run_causal(x, grid)
    assert torch.equal(full, again), "repeat call is not bitwise identical"
    d = {k: dev(v) for k, v in x.items()}
    kv = torch.zeros((1, 2, 64, 64), dtype=torch.float32, device="cuda")
    ks = torch.zeros((1, 2, 64), dtype=torch.float32, device="cuda")
    outs = []
    for t0, sl in ((0, slice(0, 400)), (4, slice(400, 1000))):
        rope = hla.Rope3D(((sl.stop - sl.start) // 100, 10, 10), t_offset=t0)
        q, k, v, g = (d[n][:, sl].contiguous() for n in "qkvg")
        outs.append(hla.hla_linear_attn_causal(q, k, v, g, rope, kv_in=kv, ksum_in=ks, kv_out=kv, ksum_out=ks))
    torch.cuda.synchronize()
    ref, kv_ref, ks_ref = oracle_causal(x, grid)
    assert normwise(host(torch.cat(outs, dim=1)), ref) <= TOL_BF16
    assert normwise(host(kv), host(kv_full)) <= 1e-5
    assert normwise(host(ks), host(ks_full)) <= 1e-5
    assert normwise(host(kv), kv_ref) <= TOL_BF16


def test_causal_full_size_sampled_rows():
    """720p/5s shape (B1 H32 N75600, gated): sampled rows of four heads against the oracle."""
    w = synth.LINEAR_720P5S
    x = w.draw()
    say(f"[parity] causal {w.name}: N={w.N} H={w.H}")
    o, kvo, kso = run_causal(x, w.grid)
    rows = np.unique(np.concatenate([np.linspace(0, w.N - 1, 400).astype(np.int64), np.arange(40), [w.N - 1]]))
    heads = [0, 9, 22, 31]
    ref, kv_ref, ks_ref = oracle_causal(x, w.grid, rows=rows, heads=heads)
    got = host(o[:, torch.from_numpy(rows).cuda()][:, :, heads])
    e = normwise(got, ref)
    e_kv = normwise(host(kvo)[:, heads], kv_ref)
    e_ks = normwise(host(kso)[:, heads], ks_ref)
    say(f"[parity] causal: out {e:.3e} state {e_kv:.3e} key sum {e_ks:.3e}")
    assert e <= TOL_BF16 and e_kv <= TOL_BF16 and e_ks <= 1e-5

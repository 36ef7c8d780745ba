"""Write the oracle regression fixtures in this folder.

Calls only ``oracle/`` (and the seeded generator in ``synth``). The pages print
no worked numeric example, so every stored value here is the fp64 oracle's
output on a small seeded input; ``tests/test_golden.py`` checks that the
oracle still reproduces them (drift guard) and the GPU parity tests reuse them.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def _dump(name, meta, arrays):
    doc = dict(meta)
    doc["outputs"] = {k: np.asarray(v, dtype=np.float64).ravel().tolist() for k, v in arrays.items()}
    doc["shapes"] = {k: list(np.shape(v)) for k, v in arrays.items()}
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(doc, f, indent=0)


def main():
    # bidirectional, gated, bf16 inputs, grid 2x2x3, two heads
    grid, B, H, D = (2, 2, 3), 1, 2, 64
    N = 12
    ins = {nm: synth.randn(7, (B, N, H, D), stream=i) for i, nm in enumerate("qkvg")}
    f = {k: synth.to_f64(v) for k, v in ins.items()}
    o = oracle.linear_attention(f["q"], f["k"], f["v"], f["g"], oracle.Rope3D(grid), eps=1e-6)
    _dump("linear_gated_2x2x3.json", {
        "what": "bidirectional ReLU linear attention, RoPE after ReLU, RoPE-free denominator, sigmoid gate",
        "cites": "SANA-Video notes section 3.2 (equation and pseudocode); SANA-Video 2.0 abstract (gated linear layers)",
        "inputs": {"generator": "synth.randn", "seed": 7, "streams": {"q": 0, "k": 1, "v": 2, "g": 3}, "dtype": "bf16",
                   "shape": [B, N, H, D]},
        "grid": list(grid), "bands": [16, 24, 24], "base": 10000.0, "eps": 1e-6}, {"o": o})

    # chunked: grid 5x2x2 (20 tokens), chunks of 6 tokens (ragged tail of 2), no gate
    grid, N, L = (5, 2, 2), 20, 6
    ins = {nm: synth.randn(8, (B, N, H, D), stream=i) for i, nm in enumerate("qkv")}
    f = {k: synth.to_f64(v) for k, v in ins.items()}
    o, kv, ks = oracle.linear_attention_chunked(f["q"], f["k"], f["v"], L, None, oracle.Rope3D(grid), eps=1e-6)
    _dump("chunked_5x2x2_L6.json", {
        "what": "block-causal linear attention with carried (KV, ksum), own chunk inclusive",
        "cites": "SANA-Video notes section 3.4 (causal equation, constant-memory cache, Algorithm 1)",
        "inputs": {"generator": "synth.randn", "seed": 8, "streams": {"q": 0, "k": 1, "v": 2}, "dtype": "bf16",
                   "shape": [B, N, H, D]},
        "grid": list(grid), "bands": [16, 24, 24], "base": 10000.0, "eps": 1e-6, "chunk_tokens": L},
        {"o": o, "kv_out": kv, "ksum_out": ks})

    # anchor: N=40, two heads, gated, scale 1/8
    N = 40
    ins = {nm: synth.randn(9, (B, N, H, D), stream=i) for i, nm in enumerate("qkvg")}
    f = {k: synth.to_f64(v) for k, v in ins.items()}
    o = oracle.softmax_anchor(f["q"], f["k"], f["v"], f["g"], scale=0.125)
    _dump("anchor_N40.json", {
        "what": "gated non-causal softmax attention, scale 1/sqrt(64)",
        "cites": "SANA-Video 2.0 abstract and summary (periodic gated softmax anchors)",
        "inputs": {"generator": "synth.randn", "seed": 9, "streams": {"q": 0, "k": 1, "v": 2, "g": 3}, "dtype": "bf16",
                   "shape": [B, N, H, D]}, "scale": 0.125}, {"o": o})

    # router: B=2, T=3, C=64, S=4 sources, w and phi(t) ~ N(0, 0.02^2)
    Bq, T, C, S = 2, 3, 64, 4
    vs = [synth.randn(10, (Bq, T, C), stream=i) for i in range(S)]
    w = synth.randn(10, (C,), std=0.02, dtype="f32", stream=100)
    phi = synth.randn(10, (Bq, C), std=0.02, dtype="f32", stream=101)
    h, a = oracle.attnres_route([synth.to_f64(v) for v in vs], w.astype(np.float64), phi.astype(np.float64), eps=1e-6)
    _dump("route_B2T3C64S4.json", {
        "what": "AttnRes router: softmax over sources of (w+phi(t))^T RMSNorm(v_i), weighted sum of raw v_i",
        "cites": "SANA-Video 2.0 summary, method section, router equation",
        "inputs": {"generator": "synth.randn", "seed": 10, "sources": {"streams": list(range(S)), "dtype": "bf16",
                   "shape": [Bq, T, C]}, "w": {"stream": 100, "std": 0.02, "dtype": "f32"},
                   "phi_t": {"stream": 101, "std": 0.02, "dtype": "f32"}}, "eps": 1e-6}, {"h": h, "alpha": a})


if __name__ == "__main__":
    main()

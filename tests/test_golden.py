"""Drift guard: the oracle still reproduces the stored fixtures in tests/golden/."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        doc = json.load(f)
    outs = {k: np.asarray(v).reshape(doc["shapes"][k]) for k, v in doc["outputs"].items()}
    return doc, outs


def _inputs(doc, names):
    inp = doc["inputs"]
    return {nm: synth.to_f64(synth.randn(inp["seed"], inp["shape"], stream=inp["streams"][nm])) for nm in names}


def test_golden_linear():
    doc, outs = load("linear_gated_2x2x3.json")
    f = _inputs(doc, "qkvg")
    o = oracle.linear_attention(f["q"], f["k"], f["v"], f["g"], oracle.Rope3D(tuple(doc["grid"])), eps=doc["eps"])
    np.testing.assert_allclose(o, outs["o"], rtol=1e-12, atol=1e-15)


def test_golden_chunked():
    doc, outs = load("chunked_5x2x2_L6.json")
    f = _inputs(doc, "qkv")
    o, kv, ks = oracle.linear_attention_chunked(f["q"], f["k"], f["v"], doc["chunk_tokens"], None,
                                                oracle.Rope3D(tuple(doc["grid"])), eps=doc["eps"])
    np.testing.assert_allclose(o, outs["o"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(kv, outs["kv_out"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ks, outs["ksum_out"], rtol=1e-12)


def test_golden_anchor():
    doc, outs = load("anchor_N40.json")
    f = _inputs(doc, "qkvg")
    o = oracle.softmax_anchor(f["q"], f["k"], f["v"], f["g"], scale=doc["scale"])
    np.testing.assert_allclose(o, outs["o"], rtol=1e-12, atol=1e-15)


def test_golden_route():
    doc, outs = load("route_B2T3C64S4.json")
    inp = doc["inputs"]
    shp = inp["sources"]["shape"]
    vs = [synth.to_f64(synth.randn(inp["seed"], shp, stream=s)) for s in inp["sources"]["streams"]]
    w = synth.randn(inp["seed"], (shp[2],), std=0.02, dtype="f32", stream=100).astype(np.float64)
    phi = synth.randn(inp["seed"], (shp[0], shp[2]), std=0.02, dtype="f32", stream=101).astype(np.float64)
    h, a = oracle.attnres_route(vs, w, phi, eps=doc["eps"])
    np.testing.assert_allclose(h, outs["h"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(a, outs["alpha"], rtol=1e-12)

#!/usr/bin/env python3
"""Benchmark of the hybrid-attention token-mixing path on one MI355X.

One step is one 3:1 hybrid group at the 720p/5s latent shape (B=1, N=75600 =
21 x 45 x 80 tokens, H=32, D=64, bf16): three gated ReLU+3D-RoPE linear
attention layers, one gated softmax anchor and four AttnRes routes (C=2048,
S=4 sources), every call through libhla's C ABI on one stream. Inputs are
seeded synthetic tensors already resident in HBM.

Printed: one JSON line. ``value`` is the linear-attention token throughput at
the 720p/5s shape (tokens per second of one layer, B*N / median layer time);
``ms_per_step`` is the wall time of a whole group. Per-call times are the
median (and min) over the timed steps, from HIP events recorded on the stream
the library launches on. ``legs`` adds, each as the median and min of repeated
calls with a 1 GiB read before every call (outside the timed region): the
cond/uncond pair (B=2, N=32760), the token-causal and the backward passes at
720p/5s, the block-sparse anchor, the block-causal 720p/60s call (N=867600,
chunks of 36000), the same sequence streamed block by block for a cond/uncond
pair, and a plain 2 GiB device copy as the achievable ceiling. ``cpu_baseline``
times the fp64 oracle on the host cores; ``context`` quotes the pages' H100
figures (other hardware, whole model: not compared).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-legs]
    python bench.py --profile-leg LEG     # one call of one leg, for rocprofv3
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix peak


def _dev(torch, x):
    import numpy as np

    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _src_hash(*names) -> str:
    """Hash of the kernel sources and of the build script (its flags shape the code too)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "softmax_attention_relu_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, "softmax_attention_relu_amd", "build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str, grid: int, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None.

    profiles/hbm_traffic.txt holds one line per kernel and launch size:
      kernel=<name> grid=<threads> fetch_kib=<F> write_kib=<W>
      fetch_scale=<bytes per counter KiB> write_scale=<...> src=<sha>
    F and W are FETCH_SIZE and WRITE_SIZE per dispatch as the counters read
    them; the scales turn them into bytes and were measured on a copy of known
    size. A line whose src hash differs from the current kernel source is stale
    and ignored, so a changed kernel reports null until it is profiled again.
    """
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        kv = dict(re.findall(r"(\w+)=(\S+)", line))
        if kv.get("kernel") == kernel and kv.get("grid") == str(grid) and kv.get("src") == src_hash:
            return float(kv["fetch_kib"]) * float(kv["fetch_scale"]) + float(kv["write_kib"]) * float(kv["write_scale"])
    return None


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores, timed before the GPU is touched
# (worker processes are forked from a process that has not initialised the GPU).

_CPU_INPUTS = {}


def _cpu_linear_head(job):
    import oracle
    import synth

    name, h = job
    w, x = _CPU_INPUTS[name]
    f = {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in x.items()}
    oracle.linear_attention(f["q"], f["k"], f["v"], f.get("g"), oracle.Rope3D(w.grid), eps=w.eps)
    return h


def _cpu_anchor_rows(r):
    import numpy as np

    import oracle

    x = _CPU_INPUTS["anchor"]
    oracle.softmax_anchor(x["q"], x["k"], x["v"], x["g"], scale=x["scale"], rows=np.arange(r[0], r[1]))
    return r


def _cpu_route_tokens(r):
    import oracle
    import synth

    x = _CPU_INPUTS["route"]
    oracle.attnres_route([synth.to_f64(s[:, r[0]:r[1]]) for s in x["v"]], x["w"], x["phi_t"], x["eps"])
    return r


def cpu_baseline(anchor_rows: int = 16384, route_tokens: int = 75600):
    """The fp64 oracle on the host's visible cores (one worker process per core, at most 16).

    Times, on the seeded inputs of the hybrid 720p/5s group: the gated linear layer on all 32
    heads (value: tokens/s of one layer), one AttnRes route (``route_tokens`` tokens, scaled to
    the full route), and ``anchor_rows`` query rows of one anchor head against all keys,
    extrapolated to the 32 heads and all rows; then the cond/uncond pair layer and the fp32
    1024-token layer in full.
    """
    import multiprocessing as mp

    import numpy as np

    import synth

    w = synth.HYBRID_LINEAR[0]
    aw = synth.HYBRID_ANCHOR
    rw = synth.HYBRID_ROUTES[0]
    _CPU_INPUTS["linear"] = (w, w.draw())
    extra = (synth.LINEAR_CFGPAIR_N32760, synth.LINEAR_F32_N1024)
    for e in extra:
        _CPU_INPUTS[e.name] = (e, e.draw())
    a = aw.draw()
    _CPU_INPUTS["anchor"] = {k: synth.to_f64(v[:, :, 0:1]) for k, v in a.items()}
    _CPU_INPUTS["anchor"]["scale"] = aw.scale
    r = rw.draw()
    _CPU_INPUTS["route"] = {"v": r["v"], "w": r["w"].astype(np.float64), "phi_t": r["phi_t"].astype(np.float64),
                            "eps": rw.eps}
    procs = max(1, min(16, len(os.sched_getaffinity(0))))
    env_threads = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env_threads:
        os.environ[k] = "1"  # one BLAS thread per worker process
    try:
        with mp.get_context("fork").Pool(procs) as pool:
            t0 = time.perf_counter()
            pool.map(_cpu_linear_head, [("linear", h) for h in range(w.H)])
            lin_s = time.perf_counter() - t0
            extra_s = {}
            for e in extra:
                t0 = time.perf_counter()
                pool.map(_cpu_linear_head, [(e.name, h) for h in range(e.H)])
                extra_s[e.name] = time.perf_counter() - t0
            nrow = min(anchor_rows, aw.N)
            t0 = time.perf_counter()
            pool.map(_cpu_anchor_rows, [(i, min(nrow, i + 1024)) for i in range(0, nrow, 1024)])
            anc_sample_s = time.perf_counter() - t0
            ntok = min(route_tokens, rw.T)
            t0 = time.perf_counter()
            pool.map(_cpu_route_tokens, [(i, min(ntok, i + 4096)) for i in range(0, ntok, 4096)])
            route_sample_s = time.perf_counter() - t0
    finally:
        for k, v in env_threads.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    _CPU_INPUTS.clear()
    anc_s = anc_sample_s * (aw.N / nrow) * aw.H * aw.B
    route_s = route_sample_s * (rw.T / ntok)
    model = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": w.B * w.N / lin_s,
        "unit": "tokens/s",
        "cores": procs,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle in {procs} worker processes: all {w.H} heads of one 720p/5s gated linear "
                   f"layer ({lin_s:.1f} s, value), one AttnRes route over {ntok} of {rw.T} tokens "
                   f"({route_sample_s:.1f} s), and {nrow} query rows of one anchor head against all {aw.N} keys "
                   f"({anc_sample_s:.1f} s); also the cond/uncond pair layer (B=2, N=32760, "
                   f"{extra_s[extra[0].name]:.1f} s) and the fp32 1024-token layer ({extra_s[extra[1].name]:.2f} s)"),
        "linear_layer_s": lin_s,
        "other_linear_configs": {e.name: {"s": extra_s[e.name], "tokens_per_s": e.B * e.N / extra_s[e.name]}
                                 for e in extra},
        "route_s": route_s,
        "anchor_s_extrapolated": anc_s,
        "anchor_extrapolation": f"x{aw.N / nrow:.3g} rows, x{aw.H} heads",
        "hybrid_step_s_extrapolated": 3 * lin_s + anc_s + 4 * route_s,
        "cpu_model": model,
        "visible_cpus": len(os.sched_getaffinity(0)),
    }


# The pages' own figures, measured on other hardware for the whole model; printed beside the
# results as context, never compared (SANA-Video 2.0 abstract).
CONTEXT = {
    "source": "SANA-Video 2.0 abstract; 1x H100, whole DiT / pipeline, not a kernel figure",
    "h100_compiled_dit_forward_speedup_vs_full_softmax_720p60s": 3.2,
    "h100_pipeline_latency_720p5s_s": 13.06,
}


LEGS = ("hybrid", "cfgpair", "causal", "backward", "backward_saved", "anchor_backward", "anchor_backward_saved",
        "sparse_anchor", "chunked", "stream", "copy")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true")
    ap.add_argument("--profile-leg", choices=LEGS,
                    help="for rocprofv3 runs: build one leg's inputs, run its call once, print no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs the path on one GPU; --gpus above 1 is not supported"}),
              flush=True)
        return 2

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline and not args.profile_leg:
        log("[bench] cpu baseline: fp64 oracle on the host cores (before the GPU is used)")
        cpu = cpu_baseline()
        log(f"[bench] cpu baseline done: {cpu['sample']}")

    import numpy as np
    import torch

    import synth
    from softmax_attention_relu_amd import hla

    hla.lib()  # fails loudly if libhla.so is missing
    torch.cuda.set_device(0)
    dev = lambda x: _dev(torch, x)  # noqa: E731
    prof = args.profile_leg
    run_legs = not args.no_legs

    # 1 GiB read between timed iterations (outside the timed region) evicts L2 and the MALL. A read
    # leaves clean lines behind; a write would leave dirty ones whose write-back lands in the timed call.
    flush_buf = torch.ones(1 << 28, dtype=torch.int32, device="cuda")

    def flush():
        flush_buf.sum()

    def timed(fn, reps, cold=True):
        """Median and min (ms) of ``reps`` calls, each between HIP events on the current stream."""
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            if cold:
                flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)), float(np.min(ts))

    out = {}

    # ---------------- the hybrid 720p/5s group: inputs resident in HBM before timing
    if prof in (None, "hybrid", "causal", "backward", "backward_saved", "anchor_backward",
                "anchor_backward_saved"):
        log("[bench] drawing and uploading the hybrid group's inputs")
        lin = []
        for w in synth.HYBRID_LINEAR:
            x = {k: dev(v) for k, v in w.draw().items()}
            x["o"] = torch.empty_like(x["q"])
            x["rope"] = hla.Rope3D(w.grid, w.bands, w.base)
            x["ws"] = torch.empty(hla.hla_linear_attn_workspace(w.B, w.N, w.H, w.D), dtype=torch.uint8,
                                  device="cuda")
            lin.append((w, x))
        aw = synth.HYBRID_ANCHOR
        anc = {k: dev(v) for k, v in aw.draw().items()}
        anc["o"] = torch.empty_like(anc["q"])
        anc["ws"] = torch.empty(hla.hla_softmax_anchor_workspace(aw.B, aw.N, aw.H, aw.D), dtype=torch.uint8,
                                device="cuda")
        routes = []
        for rw in synth.HYBRID_ROUTES:
            r = rw.draw()
            rr = {"v": [dev(x) for x in r["v"]], "w": dev(r["w"]), "phi": dev(r["phi_t"])}
            rr["h"] = torch.empty_like(rr["v"][0])
            routes.append((rw, rr))
        torch.cuda.synchronize()
        w0 = synth.HYBRID_LINEAR[0]
        tokh = w0.B * w0.N * w0.H

    names = [f"linear{i}" for i in range(3)] + ["anchor"] + [f"route{i}" for i in range(4)]

    def step(ev=None):
        # hybrid group in model order: route -> mixer, three linear layers then the anchor
        for i in range(4):
            rw, rr = routes[i]
            if ev is not None:
                ev[f"route{i}"][0].record()
            hla.hla_attnres_route(rr["v"], rr["w"], rr["phi"], rw.eps, h=rr["h"])
            if ev is not None:
                ev[f"route{i}"][1].record()
            if i < 3:
                w, x = lin[i]
                if ev is not None:
                    ev[f"linear{i}"][0].record()
                hla.hla_linear_attn(x["q"], x["k"], x["v"], x["g"], x["rope"], w.eps, o=x["o"], ws=x["ws"])
                if ev is not None:
                    ev[f"linear{i}"][1].record()
            else:
                if ev is not None:
                    ev["anchor"][0].record()
                hla.hla_softmax_anchor(anc["q"], anc["k"], anc["v"], anc["g"], aw.scale, o=anc["o"], ws=anc["ws"])
                if ev is not None:
                    ev["anchor"][1].record()

    if prof is None:
        log(f"[bench] warmup {args.warmup} steps")
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        # K steps back to back: each step reads ~10 GB of distinct tensors, so every call starts cold
        log(f"[bench] timing {args.steps} steps")
        evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            step(evs[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = wall * 1e3 / args.steps
        calls = {n: [e[n][0].elapsed_time(e[n][1]) for e in evs] for n in names}
        per = {n: float(np.median(v)) for n, v in calls.items()}
        per_min = {n: float(np.min(v)) for n, v in calls.items()}
        log("[bench] per-call median ms: " + ", ".join(f"{n} {v:.3f}" for n, v in per.items()))

        lin_ms = float(np.median(sum((calls[f"linear{i}"] for i in range(3)), [])))
        lin_min = float(np.min(sum((calls[f"linear{i}"] for i in range(3)), [])))
        lin_bytes = tokh * 64 * 2 * 5  # Q, K, V, G read + O written, bf16
        lin_gbs = lin_bytes / (lin_ms * 1e-3) / 1e9
        anc_ms, anc_min = per["anchor"], per_min["anchor"]
        anc_flops = 4.0 * aw.B * aw.H * aw.N * aw.N * aw.D
        anc_tflops = anc_flops / (anc_ms * 1e-3) / 1e12
        rt_all = sum((calls[f"route{i}"] for i in range(4)), [])
        rt_ms, rt_min = float(np.median(rt_all)), float(np.min(rt_all))
        rw0 = synth.HYBRID_ROUTES[0]
        rt_bytes = rw0.B * rw0.T * rw0.C * 2 * (rw0.S + 1)
        rt_gbs = rt_bytes / (rt_ms * 1e-3) / 1e9

        # anchor_fwd_kernel launches 1024 threads per 512 query rows of one head
        anchor_threads = -(-aw.N // 512) * aw.B * aw.H * 1024
        anchor_traffic = _traffic("anchor_fwd_kernel", anchor_threads, _src_hash("anchor.hip"))
        out = {
            "metric": "linear-attn tokens/s & HBM GB/s at 720p/5s shape; anchor MFMA util %",
            "value": w0.B * w0.N / (lin_ms * 1e-3),
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": ms_per_step,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16 tensors; router queries N(0,0.02^2) fp32)",
            "config": {"workload": "hybrid 3:1 group at 720p/5s: 3 gated linear layers + 1 gated softmax anchor "
                                   "+ 4 AttnRes routes", "B": 1, "N": 75600, "grid": [21, 45, 80], "H": 32, "D": 64,
                       "route_C": 2048, "route_S": 4, "parallelism": "single GPU"},
            "timing": "per call: median (and min) over the timed steps, HIP events on the library's stream; legs: "
                      "median and min of repeated calls, a 1 GiB read before each outside the timed region",
            "linear_hbm_gbs": lin_gbs,
            "linear_hbm_frac": lin_gbs / HBM_PEAK_GBS,
            "linear_ms": lin_ms,
            "linear_ms_min": lin_min,
            "anchor_mfma_util_pct": 100.0 * anc_tflops / BF16_PEAK_TFLOPS,
            "anchor_ms": anc_ms,
            "anchor_ms_min": anc_min,
            "route_hbm_gbs": rt_gbs,
            "route_ms": rt_ms,
            "route_ms_min": rt_min,
            "per_call_ms": per,
            "per_call_ms_min": per_min,
            "roofline": {"bound": "mfma", "kernel": "anchor_fwd (call incl. the V-transpose pre-pass)",
                         "achieved": anc_tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": anc_tflops / BF16_PEAK_TFLOPS, "traffic": anchor_traffic},
            "rooflines": {
                "linear_attn": {"bound": "hbm", "achieved": lin_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": lin_gbs / HBM_PEAK_GBS, "algorithmic_bytes": lin_bytes},
                "attnres_route": {"bound": "hbm", "achieved": rt_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": rt_gbs / HBM_PEAK_GBS, "algorithmic_bytes": rt_bytes},
            },
            "context": CONTEXT,
        }
    elif prof == "hybrid":
        log("[bench] profile leg: one hybrid step")
        step()
        torch.cuda.synchronize()
        return 0

    legs = out.setdefault("legs", {}) if prof is None else {}

    def leg_on(name):
        return prof == name or (prof is None and run_legs)

    def record(name, fn, reps, **info):
        if prof is not None:
            log(f"[bench] profile leg {name}: one call")
            fn()
            torch.cuda.synchronize()
            return None
        med, mn = timed(fn, reps)
        legs[name] = {"ms": med, "ms_min": mn, **info}
        log(f"[bench] {name}: {med:.3f} ms (min {mn:.3f})")
        return legs[name]

    def hbm(entry, nbytes, tokens):
        if entry is not None:
            ms = entry["ms"]
            entry.update({"tokens_per_s": tokens / (ms * 1e-3), "hbm_gbs": nbytes / (ms * 1e-3) / 1e9,
                          "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": nbytes})

    # ---------------- token-causal: the first 720p/5s linear layer's inputs, causal
    if leg_on("causal"):
        cq = lin[0][1]
        cws = torch.empty(hla.hla_linear_attn_causal_workspace(w0.B, w0.N, w0.H, w0.D), dtype=torch.uint8,
                          device="cuda")
        co = torch.empty_like(cq["q"])
        e = record("causal_720p5s", lambda: hla.hla_linear_attn_causal(cq["q"], cq["k"], cq["v"], cq["g"],
                                                                        cq["rope"], w0.eps, o=co, ws=cws), 10,
                   N=w0.N)
        hbm(e, tokh * 64 * 2 * 5, w0.B * w0.N)
        del cws, co

    # ---------------- backward: gradients of the first 720p/5s linear layer (gated, RoPE)
    if leg_on("backward") or leg_on("backward_saved"):
        bx = lin[0][1]
        bdo = dev(synth.randn(w0.seed, (w0.B, w0.N, w0.H, w0.D), stream=4))
        bws = torch.empty(hla.hla_linear_attn_backward_workspace(w0.B, w0.N, w0.H, w0.D), dtype=torch.uint8,
                          device="cuda")
        bouts = [torch.empty_like(bx["q"]) for _ in range(4)]
        # algorithmic: Q, K, V, G, dO read once and dQ, dK, dV, dG written once
        bw_bytes = tokh * 64 * 2 * 9
        # what the four-kernel schedule moves: K, V (state) + Q, G, dO in, dQ, dG, dnum out + Q, dnum (gradient
        # state) + K, V in, dK, dV out, bf16; plus dden fp32 written and read
        bw_sched = tokh * 64 * 2 * 16 + tokh * 4 * 2
        if leg_on("backward"):
            e = record("backward_720p5s", lambda: hla.hla_linear_attn_backward(
                bx["q"], bx["k"], bx["v"], bdo, bx["g"], bx["rope"], w0.eps, dq=bouts[0], dk=bouts[1], dv=bouts[2],
                dg=bouts[3], ws=bws), 10, N=w0.N)
            hbm(e, bw_bytes, w0.B * w0.N)
            if e is not None:
                e.update({"schedule_bytes": bw_sched, "schedule_gbs": bw_sched / (e["ms"] * 1e-3) / 1e9})
        if leg_on("backward_saved"):
            # given the forward's state (hla_linear_attn_chunked with chunk = N returns it): the first
            # state build is skipped, K and V are read once fewer
            bkv = torch.empty((w0.B, w0.H, w0.D, w0.D), dtype=torch.float32, device="cuda")
            bks = torch.empty((w0.B, w0.H, w0.D), dtype=torch.float32, device="cuda")
            hla.hla_linear_attn_chunked(bx["q"], bx["k"], bx["v"], w0.N, bx["g"], bx["rope"], w0.eps, kv_out=bkv,
                                        ksum_out=bks)
            e = record("backward_saved_720p5s", lambda: hla.hla_linear_attn_backward_saved(
                bx["q"], bx["k"], bx["v"], bkv, bks, bdo, bx["g"], bx["rope"], w0.eps, dq=bouts[0], dk=bouts[1],
                dv=bouts[2], dg=bouts[3], ws=bws), 10, N=w0.N)
            hbm(e, bw_bytes, w0.B * w0.N)
            if e is not None:
                bs_sched = bw_sched - tokh * 64 * 2 * 2
                e.update({"schedule_bytes": bs_sched, "schedule_gbs": bs_sched / (e["ms"] * 1e-3) / 1e9})
            del bkv, bks
        del bws, bouts, bdo

    # ---------------- anchor backward: gradients of the 720p/5s anchor (gated)
    if leg_on("anchor_backward") or leg_on("anchor_backward_saved"):
        ado = dev(synth.randn(aw.seed, (aw.B, aw.N, aw.H, aw.D), stream=4))
        aws = torch.empty(hla.hla_softmax_anchor_backward_workspace(aw.B, aw.N, aw.H, aw.D), dtype=torch.uint8,
                          device="cuda")
        agrads = [torch.empty_like(anc["q"]) for _ in range(4)]
        # algorithmic: the five N x N products of the gradient (S, dP, dV, dK, dQ), 10 N^2 D per head
        ab_alg = 10.0 * aw.B * aw.H * float(aw.N) ** 2 * aw.D

        def flops(e, sched):
            if e is not None:
                e.update({"N": aw.N, "algorithmic_flop": ab_alg, "schedule_flop": sched,
                          "algorithmic_tflops": ab_alg / (e["ms"] * 1e-3) / 1e12,
                          "mfma_frac": ab_alg / (e["ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                          "schedule_tflops": sched / (e["ms"] * 1e-3) / 1e12})

        if leg_on("anchor_backward"):
            # the schedule recomputes the forward (4) and S, dP in both gradient kernels: 18 N^2 D
            e = record("anchor_backward_720p5s", lambda: hla.hla_softmax_anchor_backward(
                anc["q"], anc["k"], anc["v"], ado, anc["g"], aw.scale, *agrads, ws=aws), 3)
            flops(e, 18.0 * aw.B * aw.H * float(aw.N) ** 2 * aw.D)
        if leg_on("anchor_backward_saved"):
            # from a saved forward (its gated output and row normalisers): 14 N^2 D scheduled
            ao, alse = hla.hla_softmax_anchor_lse(anc["q"], anc["k"], anc["v"], anc["g"], aw.scale)
            e = record("anchor_backward_saved_720p5s", lambda: hla.hla_softmax_anchor_backward_saved(
                anc["q"], anc["k"], anc["v"], ao, alse, ado, anc["g"], aw.scale, *agrads, ws=aws), 3)
            flops(e, 14.0 * aw.B * aw.H * float(aw.N) ** 2 * aw.D)
            del ao, alse
        del ado, aws, agrads

    if prof in (None, "hybrid", "causal", "backward", "backward_saved", "anchor_backward",
                "anchor_backward_saved"):
        del lin, routes, anc
        torch.cuda.empty_cache()

    # ---------------- block-sparse anchor: 720p/5s with a local-window pattern
    if leg_on("sparse_anchor"):
        sw = synth.SPARSE_ANCHOR_720P5S
        sx = {k: dev(v) for k, v in sw.draw().items()}
        sb, sc = synth.block_window_pattern(sw.B, sw.H, sw.N, *synth.SPARSE_ANCHOR_WINDOW)
        # query-key pairs visited: rows of each query block x keys of its named blocks
        rows_per_qb = np.minimum(128, sw.N - 128 * np.arange(sb.shape[2]))
        keys_per_blk = np.minimum(64, sw.N - 64 * np.arange(-(-sw.N // 64)))
        pairs = float(sum(int(rows_per_qb[r]) * int(keys_per_blk[sb[b, h, r, :sc[b, h, r]]].sum())
                          for b in range(sw.B) for h in range(sw.H) for r in range(sb.shape[2])))
        sbt, sct = torch.from_numpy(sb).cuda(), torch.from_numpy(sc).cuda()
        so = torch.empty_like(sx["q"])
        sws = torch.empty(hla.hla_softmax_anchor_workspace(sw.B, sw.N, sw.H, sw.D), dtype=torch.uint8, device="cuda")
        e = record("sparse_anchor_720p5s", lambda: hla.hla_softmax_anchor_block_sparse(
            sx["q"], sx["k"], sx["v"], sbt, sct, sx["g"], sw.scale, o=so, ws=sws), 5, N=sw.N,
            pattern="window +-72 key blocks + 4 global (64-key blocks, 128-row query blocks)",
            density=pairs / (sw.B * sw.H * float(sw.N) ** 2))
        if e is not None:
            tf = 4.0 * sw.D * pairs / (e["ms"] * 1e-3) / 1e12
            e.update({"visited_pair_tflops": tf, "mfma_frac": tf / BF16_PEAK_TFLOPS})
        del sx, so, sws, sbt, sct
        torch.cuda.empty_cache()

    # ---------------- cond/uncond pair: B = 2, N = 32 760 (21 x 30 x 52), gated, RoPE
    if leg_on("cfgpair"):
        pw = synth.LINEAR_CFGPAIR_N32760
        log("[bench] cond/uncond pair leg: drawing inputs")
        px = {k: dev(v) for k, v in pw.draw().items()}
        po = torch.empty_like(px["q"])
        prope = hla.Rope3D(pw.grid, pw.bands, pw.base)
        pws = torch.empty(hla.hla_linear_attn_workspace(pw.B, pw.N, pw.H, pw.D), dtype=torch.uint8, device="cuda")
        e = record("cfgpair_linear_32760", lambda: hla.hla_linear_attn(px["q"], px["k"], px["v"], px["g"], prope,
                                                                      pw.eps, o=po, ws=pws), 20, B=pw.B, N=pw.N)
        hbm(e, pw.B * pw.N * pw.H * 64 * 2 * 5, pw.B * pw.N)
        del px, po, pws
        torch.cuda.empty_cache()

    # ---------------- block-causal 720p/60s
    if leg_on("chunked"):
        cw = synth.CHUNKED_720P60S
        log("[bench] chunked 720p/60s leg: drawing inputs")
        cx = {k: dev(v) for k, v in cw.draw().items()}
        cx["o"] = torch.empty_like(cx["q"])
        rope = hla.Rope3D(cw.grid, cw.bands, cw.base)
        ws = torch.empty(hla.hla_linear_attn_chunked_workspace(cw.B, cw.N, cw.H, cw.D, cw.chunk_tokens),
                         dtype=torch.uint8, device="cuda")
        kv = torch.zeros((cw.B, cw.H, 64, 64), dtype=torch.float32, device="cuda")
        ks = torch.zeros((cw.B, cw.H, 64), dtype=torch.float32, device="cuda")
        e = record("chunked_720p60s", lambda: hla.hla_linear_attn_chunked(
            cx["q"], cx["k"], cx["v"], cw.chunk_tokens, None, rope, cw.eps, kv_out=kv, ksum_out=ks, o=cx["o"], ws=ws),
            5, N=cw.N, chunk_tokens=cw.chunk_tokens)
        hbm(e, cw.B * cw.N * cw.H * 64 * 2 * 4, cw.B * cw.N)  # Q, K, V read + O written
        del cx, ws
        torch.cuda.empty_cache()

    # ---------------- streaming: the 720p/60s sequence block by block (ten frames per block), two
    # denoising calls per block that read the cache, the second also commits the block; a
    # cond/uncond pair (B = 2). Every block has its own inputs (seeded draws on the device).
    if leg_on("stream"):
        cw = synth.CHUNKED_720P60S
        sb, nsteps, frames = 2, 2, 10
        hw = cw.grid[1] * cw.grid[2]
        nblk = -(-cw.grid[0] // frames)
        log("[bench] streaming 720p/60s leg (B=2, two steps per block): drawing inputs")
        gen = torch.Generator(device="cuda")
        gen.manual_seed(6)
        blocks = []
        for bi in range(nblk):
            L = min(frames, cw.grid[0] - frames * bi) * hw
            x = {nm: torch.randn((sb, L, cw.H, 64), generator=gen, device="cuda", dtype=torch.bfloat16)
                 for nm in "qkv"}
            x["o"] = torch.empty_like(x["q"])
            x["rope"] = hla.Rope3D((L // hw, cw.grid[1], cw.grid[2]), cw.bands, cw.base, t_offset=frames * bi)
            blocks.append((L, x))
        lmax = frames * hw
        ws = torch.empty(hla.hla_linear_attn_chunked_workspace(sb, lmax, cw.H, cw.D, lmax), dtype=torch.uint8,
                         device="cuda")
        kv = torch.zeros((sb, cw.H, 64, 64), dtype=torch.float32, device="cuda")
        ks = torch.zeros((sb, cw.H, 64), dtype=torch.float32, device="cuda")

        def stream_pass():
            for L, x in blocks:
                for d in range(nsteps):
                    commit = d == nsteps - 1
                    hla.hla_linear_attn_chunked(x["q"], x["k"], x["v"], L, None, x["rope"], cw.eps, kv_in=kv,
                                                ksum_in=ks, kv_out=kv if commit else None,
                                                ksum_out=ks if commit else None, o=x["o"], ws=ws)

        e = record("stream_720p60s_cfg_pair", stream_pass, 3, B=sb, N=cw.N, blocks=nblk, steps_per_block=nsteps,
                   calls=nblk * nsteps)
        hbm(e, nsteps * sb * cw.N * cw.H * 64 * 2 * 4, nsteps * sb * cw.N)  # per call: Q, K, V + O
        del blocks, ws
        torch.cuda.empty_cache()

    # ---------------- the achievable ceiling: a plain device-to-device copy (the HIP runtime's copy kernel)
    if leg_on("copy"):
        src = torch.empty(1 << 31, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        e = record("copy_2GiB", lambda: dst.copy_(src), 10, bytes_moved=2 * src.numel())
        if e is not None:
            e["gbs"] = 2 * src.numel() / (e["ms"] * 1e-3) / 1e9
            e["frac"] = e["gbs"] / HBM_PEAK_GBS
        del src, dst

    if prof is not None:
        return 0
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

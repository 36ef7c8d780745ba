#!/usr/bin/env python3
"""Benchmark of the hybrid-attention token-mixing path on one MI355X.

One step is one 3:1 hybrid group at the 720p/5s latent shape (B=1, N=75600 =
21 x 45 x 80 tokens, H=32, D=64, bf16): three gated ReLU+3D-RoPE linear
attention layers, one gated softmax anchor and four AttnRes routes (C=2048,
S=4 sources), every call through libhla's C ABI on one stream. Inputs are
seeded synthetic tensors already resident in HBM.

Printed: one JSON line. ``value`` is the linear-attention token throughput at
the 720p/5s shape (tokens per second of one layer, B*N / mean layer time);
``ms_per_step`` is the wall time of a whole group. Per-call times come from
HIP events recorded on the stream the library launches on. ``legs`` adds, timed
the same way: the token-causal and the backward (gradient) pass of the first
720p/5s linear layer, the block-causal 720p/60s case (N=867600, chunks of
36000) and the same sequence streamed block by block for a cond/uncond pair.
``cpu_baseline`` times the fp64 oracle on a bounded sample of the linear
layer (a few heads) on the host cores.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-legs]
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


def cpu_baseline(heads: int):
    """fp64 oracle on ``heads`` heads of the 720p/5s linear layer; tokens/s scaled to all 32 heads."""
    import resource

    import numpy as np

    import oracle
    import synth

    w = synth.HYBRID_LINEAR[0]
    x = w.draw()
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    for h in range(heads):
        f = {k: synth.to_f64(v[:, :, h:h + 1]) for k, v in x.items()}
        oracle.linear_attention(f["q"], f["k"], f["v"], f["g"], oracle.Rope3D(w.grid), eps=w.eps)
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    per_layer = wall * w.H / heads
    model = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": w.B * w.N / per_layer,
        "unit": "tokens/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle, {heads} of {w.H} heads of one 720p/5s gated linear layer "
                   f"(N={w.N}), {wall:.1f} s wall"
                   + ("" if heads == w.H else f", scaled x{w.H / heads:g} to the full layer")),
        "cpu_seconds": round(cpu, 2),
        "cpu_model": model,
        "visible_cpus": len(os.sched_getaffinity(0)),
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--profile-pass", action="store_true",
                    help="for rocprofv3 counter runs: one untimed step, then a 1 GiB device copy whose "
                         "counter reading calibrates bytes; prints no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs the path on one GPU; --gpus above 1 is not supported"}),
              flush=True)
        return 2

    import numpy as np
    import torch

    import synth
    from softmax_attention_relu_amd import hla

    hla.lib()  # fails loudly if libhla.so is missing
    torch.cuda.set_device(0)
    dev = lambda x: _dev(torch, x)  # noqa: E731

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    # ---------------- inputs, resident in HBM before timing
    log("[bench] drawing and uploading inputs")
    lin = []
    for w in synth.HYBRID_LINEAR:
        x = {k: dev(v) for k, v in w.draw().items()}
        x["o"] = torch.empty_like(x["q"])
        x["rope"] = hla.Rope3D(w.grid, w.bands, w.base)
        x["ws"] = torch.empty(hla.hla_linear_attn_workspace(w.B, w.N, w.H, w.D), dtype=torch.uint8, device="cuda")
        lin.append((w, x))
    aw = synth.HYBRID_ANCHOR
    anc = {k: dev(v) for k, v in aw.draw().items()}
    anc["o"] = torch.empty_like(anc["q"])
    anc["ws"] = torch.empty(hla.hla_softmax_anchor_workspace(aw.B, aw.N, aw.H, aw.D), dtype=torch.uint8,
                            device="cuda")
    routes = []
    for rw in synth.HYBRID_ROUTES:
        r = rw.draw()
        rr = {"v": [dev(s) for s in r["v"]], "w": dev(r["w"]), "phi": dev(r["phi_t"])}
        rr["h"] = torch.empty_like(rr["v"][0])
        routes.append((rw, rr))
    torch.cuda.synchronize()

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

    if args.profile_pass:
        log("[bench] profile pass: one step, one token-causal call, one backward call, one 720p/60s chunked call, "
            "then a 1 GiB copy (calibration)")
        step()
        torch.cuda.synchronize()
        if not args.no_legs:
            cw0, cx0 = lin[0]
            hla.hla_linear_attn_causal(cx0["q"], cx0["k"], cx0["v"], cx0["g"], cx0["rope"], cw0.eps)
            torch.cuda.synchronize()
            bdo = dev(synth.randn(cw0.seed, (cw0.B, cw0.N, cw0.H, cw0.D), stream=4))
            hla.hla_linear_attn_backward(cx0["q"], cx0["k"], cx0["v"], bdo, cx0["g"], cx0["rope"], cw0.eps)
            torch.cuda.synchronize()
            del bdo
        if not args.no_legs:
            del lin, routes
            torch.cuda.empty_cache()
            cw = synth.CHUNKED_720P60S
            cx = {k: dev(v) for k, v in cw.draw().items()}
            ws = torch.empty(hla.hla_linear_attn_chunked_workspace(cw.B, cw.N, cw.H, cw.D, cw.chunk_tokens),
                             dtype=torch.uint8, device="cuda")
            hla.hla_linear_attn_chunked(cx["q"], cx["k"], cx["v"], cw.chunk_tokens, None,
                                        hla.Rope3D(cw.grid, cw.bands, cw.base), cw.eps, ws=ws)
            torch.cuda.synchronize()
            del cx, ws
            torch.cuda.empty_cache()
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] profile pass done")
        return 0

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

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
    per = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs])) for n in names}
    log("[bench] per-call ms: " + ", ".join(f"{n} {v:.3f}" for n, v in per.items()))

    w0 = synth.HYBRID_LINEAR[0]
    tokh = w0.B * w0.N * w0.H
    lin_ms = float(np.mean([per[f"linear{i}"] for i in range(3)]))
    lin_bytes = tokh * 64 * 2 * 5  # Q, K, V, G read + O written, bf16
    lin_gbs = lin_bytes / (lin_ms * 1e-3) / 1e9
    anc_ms = per["anchor"]
    anc_flops = 4.0 * aw.B * aw.H * aw.N * aw.N * aw.D
    anc_tflops = anc_flops / (anc_ms * 1e-3) / 1e12
    rt_ms = float(np.mean([per[f"route{i}"] for i in range(4)]))
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
        "linear_hbm_gbs": lin_gbs,
        "linear_hbm_frac": lin_gbs / HBM_PEAK_GBS,
        "linear_ms": lin_ms,
        "anchor_mfma_util_pct": 100.0 * anc_tflops / BF16_PEAK_TFLOPS,
        "anchor_ms": anc_ms,
        "route_hbm_gbs": rt_gbs,
        "route_ms": rt_ms,
        "per_call_ms": per,
        "roofline": {"bound": "mfma", "kernel": "anchor_fwd_kernel (call incl. V-transpose pre-pass)",
                     "achieved": anc_tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": anc_tflops / BF16_PEAK_TFLOPS, "traffic": anchor_traffic},
        "rooflines": {
            "linear_attn": {"bound": "hbm", "achieved": lin_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": lin_gbs / HBM_PEAK_GBS, "algorithmic_bytes": lin_bytes},
            "attnres_route": {"bound": "hbm", "achieved": rt_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": rt_gbs / HBM_PEAK_GBS, "algorithmic_bytes": rt_bytes},
        },
    }

    # ---------------- token-causal leg: the first 720p/5s linear layer's inputs, causal
    if not args.no_legs:
        cq = lin[0][1]
        cws = torch.empty(hla.hla_linear_attn_causal_workspace(w0.B, w0.N, w0.H, w0.D), dtype=torch.uint8,
                          device="cuda")
        crope = hla.Rope3D(w0.grid, w0.bands, w0.base)
        co = torch.empty_like(cq["q"])

        def causal_call():
            hla.hla_linear_attn_causal(cq["q"], cq["k"], cq["v"], cq["g"], crope, w0.eps, o=co, ws=cws)

        causal_call()
        torch.cuda.synchronize()
        times = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            causal_call()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        ca_ms = float(np.mean(times))
        out.setdefault("legs", {})["causal_720p5s"] = {
            "N": w0.N, "ms": ca_ms, "tokens_per_s": w0.B * w0.N / (ca_ms * 1e-3),
            "hbm_gbs": lin_bytes / (ca_ms * 1e-3) / 1e9, "hbm_frac": lin_bytes / (ca_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": lin_bytes}
        log(f"[bench] token-causal 720p/5s: {ca_ms:.3f} ms")
        del cws, co

    # ---------------- backward leg: gradients of the first 720p/5s linear layer (gated, RoPE)
    if not args.no_legs:
        bx = lin[0][1]
        bdo = dev(synth.randn(w0.seed, (w0.B, w0.N, w0.H, w0.D), stream=4))
        bws = torch.empty(hla.hla_linear_attn_backward_workspace(w0.B, w0.N, w0.H, w0.D), dtype=torch.uint8,
                          device="cuda")
        bouts = [torch.empty_like(bx["q"]) for _ in range(4)]

        def bwd_call():
            hla.hla_linear_attn_backward(bx["q"], bx["k"], bx["v"], bdo, bx["g"], bx["rope"], w0.eps, dq=bouts[0],
                                         dk=bouts[1], dv=bouts[2], dg=bouts[3], ws=bws)

        bwd_call()
        torch.cuda.synchronize()
        times = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            bwd_call()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        bw_ms = float(np.mean(times))
        # algorithmic: Q, K, V, G, dO read once and dQ, dK, dV, dG written once
        bw_bytes = tokh * 64 * 2 * 9
        # what the four-kernel schedule moves: K, V (state) + Q, G, dO in, dQ, dG, dnum out + Q, dnum (gradient
        # state) + K, V in, dK, dV out, bf16; plus dden fp32 written and read
        bw_sched = tokh * 64 * 2 * 16 + tokh * 4 * 2
        out.setdefault("legs", {})["backward_720p5s"] = {
            "N": w0.N, "ms": bw_ms, "tokens_per_s": w0.B * w0.N / (bw_ms * 1e-3),
            "hbm_gbs": bw_bytes / (bw_ms * 1e-3) / 1e9, "hbm_frac": bw_bytes / (bw_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": bw_bytes, "schedule_bytes": bw_sched,
            "schedule_gbs": bw_sched / (bw_ms * 1e-3) / 1e9}
        log(f"[bench] backward 720p/5s: {bw_ms:.3f} ms")
        # the same gradients given the forward's state (hla_linear_attn_chunked with chunk = N returns it):
        # the first state build is skipped, K and V are read once fewer
        bkv = torch.empty((w0.B, w0.H, w0.D, w0.D), dtype=torch.float32, device="cuda")
        bks = torch.empty((w0.B, w0.H, w0.D), dtype=torch.float32, device="cuda")
        hla.hla_linear_attn_chunked(bx["q"], bx["k"], bx["v"], w0.N, bx["g"], bx["rope"], w0.eps, kv_out=bkv,
                                    ksum_out=bks)

        def bwd_saved_call():
            hla.hla_linear_attn_backward_saved(bx["q"], bx["k"], bx["v"], bkv, bks, bdo, bx["g"], bx["rope"], w0.eps,
                                               dq=bouts[0], dk=bouts[1], dv=bouts[2], dg=bouts[3], ws=bws)

        bwd_saved_call()
        torch.cuda.synchronize()
        times = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            bwd_saved_call()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        bs_ms = float(np.mean(times))
        bs_sched = bw_sched - tokh * 64 * 2 * 2
        out["legs"]["backward_saved_720p5s"] = {
            "N": w0.N, "ms": bs_ms, "tokens_per_s": w0.B * w0.N / (bs_ms * 1e-3),
            "hbm_gbs": bw_bytes / (bs_ms * 1e-3) / 1e9, "hbm_frac": bw_bytes / (bs_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": bw_bytes, "schedule_bytes": bs_sched,
            "schedule_gbs": bs_sched / (bs_ms * 1e-3) / 1e9}
        log(f"[bench] backward from the saved state 720p/5s: {bs_ms:.3f} ms")
        del bws, bouts, bdo, bkv, bks

    # ---------------- anchor backward leg: gradients of the 720p/5s anchor (gated)
    if not args.no_legs:
        ado = dev(synth.randn(aw.seed, (aw.B, aw.N, aw.H, aw.D), stream=4))
        aws = torch.empty(hla.hla_softmax_anchor_backward_workspace(aw.B, aw.N, aw.H, aw.D), dtype=torch.uint8,
                          device="cuda")
        agrads = [torch.empty_like(anc["q"]) for _ in range(4)]

        def abwd_call():
            hla.hla_softmax_anchor_backward(anc["q"], anc["k"], anc["v"], ado, anc["g"], aw.scale, *agrads, ws=aws)

        abwd_call()
        torch.cuda.synchronize()
        times = []
        for _ in range(2):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            abwd_call()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        ab_ms = float(np.mean(times))
        # algorithmic: the five N x N products of the gradient (S, dP, dV, dK, dQ), 10 N^2 D per head; the
        # schedule recomputes the forward (4) and S, dP in both gradient kernels: 18 N^2 D
        ab_alg = 10.0 * aw.B * aw.H * float(aw.N) ** 2 * aw.D
        ab_sched = 18.0 * aw.B * aw.H * float(aw.N) ** 2 * aw.D
        out.setdefault("legs", {})["anchor_backward_720p5s"] = {
            "N": aw.N, "ms": ab_ms, "algorithmic_flop": ab_alg, "schedule_flop": ab_sched,
            "algorithmic_tflops": ab_alg / (ab_ms * 1e-3) / 1e12,
            "mfma_frac": ab_alg / (ab_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "schedule_tflops": ab_sched / (ab_ms * 1e-3) / 1e12}
        log(f"[bench] anchor backward 720p/5s: {ab_ms:.1f} ms")
        # the same gradients from a saved forward (its gated output and row normalisers): the
        # second forward pass becomes an elementwise preparation, 14 N^2 D scheduled
        ao, alse = hla.hla_softmax_anchor_lse(anc["q"], anc["k"], anc["v"], anc["g"], aw.scale)

        def abwd_saved_call():
            hla.hla_softmax_anchor_backward_saved(anc["q"], anc["k"], anc["v"], ao, alse, ado, anc["g"], aw.scale,
                                                  *agrads, ws=aws)

        abwd_saved_call()
        torch.cuda.synchronize()
        times = []
        for _ in range(2):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            abwd_saved_call()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        as_ms = float(np.mean(times))
        as_sched = 14.0 * aw.B * aw.H * float(aw.N) ** 2 * aw.D
        out["legs"]["anchor_backward_saved_720p5s"] = {
            "N": aw.N, "ms": as_ms, "algorithmic_flop": ab_alg, "schedule_flop": as_sched,
            "algorithmic_tflops": ab_alg / (as_ms * 1e-3) / 1e12,
            "mfma_frac": ab_alg / (as_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "schedule_tflops": as_sched / (as_ms * 1e-3) / 1e12}
        log(f"[bench] anchor backward from the saved forward 720p/5s: {as_ms:.1f} ms")
        del ado, aws, agrads, ao, alse

    # ---------------- block-sparse anchor leg: 720p/5s with a local-window pattern
    if not args.no_legs:
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

        def sparse_call():
            hla.hla_softmax_anchor_block_sparse(sx["q"], sx["k"], sx["v"], sbt, sct, sx["g"], sw.scale, o=so, ws=sws)

        sparse_call()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            sparse_call()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        sp_ms = float(np.mean(times))
        sp_tf = 4.0 * sw.D * pairs / (sp_ms * 1e-3) / 1e12
        out.setdefault("legs", {})["sparse_anchor_720p5s"] = {
            "N": sw.N, "pattern": "window +-72 key blocks + 4 global (64-key blocks, 128-row query blocks)",
            "density": pairs / (sw.B * sw.H * float(sw.N) ** 2), "ms": sp_ms, "visited_pair_tflops": sp_tf,
            "mfma_frac": sp_tf / BF16_PEAK_TFLOPS}
        log(f"[bench] sparse anchor 720p/5s: {sp_ms:.3f} ms, density {pairs / (sw.B * sw.H * float(sw.N) ** 2):.3f}, "
            f"{sp_tf:.0f} TFLOP/s on visited pairs")
        del sx, so, sws, sbt, sct

    # ---------------- block-causal 720p/60s leg
    if not args.no_legs:
        del lin, routes
        torch.cuda.empty_cache()
        cw = synth.CHUNKED_720P60S
        log("[bench] chunked 720p/60s leg: drawing inputs")
        cx = {k: dev(v) for k, v in cw.draw().items()}
        cx["o"] = torch.empty_like(cx["q"])
        rope = hla.Rope3D(cw.grid, cw.bands, cw.base)
        ws = torch.empty(hla.hla_linear_attn_chunked_workspace(cw.B, cw.N, cw.H, cw.D, cw.chunk_tokens),
                         dtype=torch.uint8, device="cuda")
        kv = torch.zeros((cw.B, cw.H, 64, 64), dtype=torch.float32, device="cuda")
        ks = torch.zeros((cw.B, cw.H, 64), dtype=torch.float32, device="cuda")

        def call():
            hla.hla_linear_attn_chunked(cx["q"], cx["k"], cx["v"], cw.chunk_tokens, None, rope, cw.eps,
                                        kv_out=kv, ksum_out=ks, o=cx["o"], ws=ws)

        call()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        c_ms = float(np.mean(times))
        c_bytes = cw.B * cw.N * cw.H * 64 * 2 * 4  # Q, K, V read + O written
        out.setdefault("legs", {})["chunked_720p60s"] = {
            "N": cw.N, "chunk_tokens": cw.chunk_tokens, "ms": c_ms, "tokens_per_s": cw.B * cw.N / (c_ms * 1e-3),
            "hbm_gbs": c_bytes / (c_ms * 1e-3) / 1e9, "hbm_frac": c_bytes / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": c_bytes}
        log(f"[bench] chunked: {c_ms:.3f} ms")
        del cx, ws
        torch.cuda.empty_cache()

        # ---------------- streaming leg: the 720p/60s sequence block by block (ten frames per
        # block), two denoising calls per block that read the cache, the second also commits the
        # block; a cond/uncond pair (B = 2). Block inputs are drawn once and reused by every block.
        sb, steps, frames = 2, 2, 10
        hw = cw.grid[1] * cw.grid[2]
        nblk = -(-cw.grid[0] // frames)
        log("[bench] streaming 720p/60s leg (B=2, two steps per block): drawing inputs")
        blk = {}
        for L in sorted({min(frames, cw.grid[0] - frames * b) * hw for b in range(nblk)}):
            blk[L] = {nm: dev(synth.randn(6, (sb, L, cw.H, 64), stream=i)) for i, nm in enumerate("qkv")}
            blk[L]["o"] = torch.empty_like(blk[L]["q"])
        ropes = [hla.Rope3D((min(frames, cw.grid[0] - frames * b), cw.grid[1], cw.grid[2]), cw.bands, cw.base,
                            t_offset=frames * b) for b in range(nblk)]
        lmax = frames * hw
        ws = torch.empty(hla.hla_linear_attn_chunked_workspace(sb, lmax, cw.H, cw.D, lmax), dtype=torch.uint8,
                         device="cuda")
        kv = torch.zeros((sb, cw.H, 64, 64), dtype=torch.float32, device="cuda")
        ks = torch.zeros((sb, cw.H, 64), dtype=torch.float32, device="cuda")

        def stream_pass():
            for b in range(nblk):
                L = ropes[b].grid[0] * hw
                x = blk[L]
                for d in range(steps):
                    commit = d == steps - 1
                    hla.hla_linear_attn_chunked(x["q"], x["k"], x["v"], L, None, ropes[b], cw.eps, kv_in=kv,
                                                ksum_in=ks, kv_out=kv if commit else None,
                                                ksum_out=ks if commit else None, o=x["o"], ws=ws)

        stream_pass()
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            stream_pass()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        s_ms = float(np.mean(times))
        s_bytes = steps * sb * cw.N * cw.H * 64 * 2 * 4  # per call: Q, K, V read + O written
        out["legs"]["stream_720p60s_cfg_pair"] = {
            "B": sb, "N": cw.N, "blocks": nblk, "steps_per_block": steps, "calls": nblk * steps, "ms": s_ms,
            "tokens_per_s": steps * sb * cw.N / (s_ms * 1e-3), "hbm_gbs": s_bytes / (s_ms * 1e-3) / 1e9,
            "hbm_frac": s_bytes / (s_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": s_bytes}
        log(f"[bench] streaming: {s_ms:.3f} ms for {nblk * steps} calls")
        del blk, ws
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_heads} heads")
        out["cpu_baseline"] = cpu_baseline(args.cpu_heads)

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Benchmark of the W4A16 group-quantized projection hot path on one MI355X.

One step is one 512-token prefill pass through the projections of one decoder layer
(hidden 2560, 32 query heads and 8 key/value heads of dimension 128, MLP 9728: q, k, v, o,
gate, up, down at M = 512, where the down projection's K = 9728 exercises split-K), followed
by the vocabulary head (2560 -> 151936) applied to the last row only (logits_to_keep = 1,
which dispatches to the matvec path).  These are the per-projection prefill shapes that
tiny-llm's "Week 2 Day 6: SIMD-Matrix Prefill" benchmarks in Task 5 and its Benchmark
Analysis, with Task 4's last-row slice before the vocabulary projection.  Inputs are seeded
synthetic data (the pages' Qwen3-4B weights are not available): x ~ N(0, 1) in bf16,
W ~ N(0, 0.02) quantized to 4-bit affine groups of 128.

All inputs are resident in HBM before the timed region.  Weight sets rotate over several
device copies so that weight reads miss the 256 MB last-level cache.  Output: one JSON line.

    python bench.py [--gpus 1] [--steps 30] [--warmup 5] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 qmm TFLOP/s + % roofline at M=128/512 prefill; qmv GB/s at M=1"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
PEAK_INT8_TOPS = 5000.0       # MI355X dense int8 MFMA
M_PREFILL = 512
LAYER = ["q", "k", "v", "o", "gate", "up", "down"]
DOMINANT = ("gate", "up")     # largest projections: the roofline kernel
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qmm_prefill512_gate_up_traffic.json")
KERNEL_SOURCES = ["w4a16_group_quantized_qmv_amd/csrc/qmm.hip", "w4a16_group_quantized_qmv_amd/csrc/device_common.h"]


def flops(M, N, K):
    return 2.0 * M * N * K


def algo_bytes(M, N, K):
    """Algorithmic bytes: packed codes + bf16 scale and bias per group + x + y."""
    return N * K / 2 + N * K / 32 + 2.0 * M * K + 2.0 * M * N


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per dominant-kernel launch from the committed counter summary, or None when
    the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def build_inputs(torch, copies):
    import numpy as np
    from w4a16_group_quantized_qmv_amd import synth
    dev = torch.device("cuda", 0)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    projections = []
    for name in LAYER:
        idx = synth.shape_index(4, name)
        K, N = synth.LAYER_SHAPES[name]
        wq, s, b = synth.weights(4, idx, N, K)
        x = synth.activations(4, idx, M_PREFILL, K)
        projections.append({"name": name, "M": M_PREFILL, "N": N, "K": K, "keep": 0,
                            "host": {"x": x, "wq": wq, "scales": s, "biases": b},
                            "x": bf16(x), "w": [(torch.from_numpy(wq.view(np.int32)).to(dev), bf16(s), bf16(b))]})
    vidx = synth.shape_index(5, "vocab")
    K, N = synth.VOCAB_SHAPE
    wq, s, b = synth.weights(5, vidx, N, K)
    x = synth.activations(5, vidx, M_PREFILL, K)
    projections.append({"name": "vocab_last_row", "M": 1, "N": N, "K": K, "keep": 1,
                        "host": {"x": x, "wq": wq, "scales": s, "biases": b},
                        "x": bf16(x), "w": [(torch.from_numpy(wq.view(np.int32)).to(dev), bf16(s), bf16(b))]})
    for p in projections:        # extra device copies of every weight set (same values)
        base = p["w"][0]
        for _ in range(copies - 1):
            p["w"].append(tuple(t.clone() for t in base))
    return projections


VOCAB_SAMPLE_COLS = 151936 // 4


def cpu_baseline(projections):
    """The oracle, untuned, on a bounded sample of one step: the seven 512-row projections in
    full and the last vocab row over the first quarter of the vocabulary columns."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    total_flops = 0.0
    t0 = time.perf_counter()
    for p in projections:
        h = p["host"]
        x = h["x"][-p["keep"]:] if p["keep"] else h["x"]
        n = p["N"] if not p["keep"] else VOCAB_SAMPLE_COLS
        O.reference(x, h["wq"][:n], h["scales"][:n], h["biases"][:n])
        total_flops += flops(x.shape[0], n, p["K"])
    dt = time.perf_counter() - t0
    return {"value": total_flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": "the seven 512-row layer projections in full and the last vocab row over the first "
                      f"{VOCAB_SAMPLE_COLS} of 151936 columns: unpack + fp32 dequant + fp64 GEMM "
                      "(reference() including the abs-mass), wall clock, rate scaled to the sample's FLOPs",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--copies", type=int, default=3, help="device copies of the weights, rotated per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the measurements beyond the step (for profiler runs of the step alone)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="before the timed region, copy a 256 MiB buffer three times (reference for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the projection kernels run on a single MI355X "
              "(column- or row-sharding across GPUs is not implemented).", file=sys.stderr)
        sys.exit(2)

    import torch
    import w4a16_group_quantized_qmv_amd as w4
    w4.load()                                   # raises when the HIP library is not built
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    projections = build_inputs(torch, args.copies)
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    # prepared calls: one per (projection, weight copy); y buffers shared across copies
    calls = []
    for c in range(args.copies):
        row = []
        for p in projections:
            x = p["x"][-p["keep"]:] if p["keep"] else p["x"]
            wq, s, b = p["w"][c]
            prev = calls[0][len(row)].y if calls else None
            row.append(w4.PreparedLinear(x, wq, s, b, y=prev))
        calls.append(row)
    plans = [call.plan for call in calls[0]]

    dom_idx = [j for j, p in enumerate(projections) if p["name"] in DOMINANT]
    assert dom_idx == list(range(dom_idx[0], dom_idx[0] + len(dom_idx))), "dominant projections must be adjacent"

    def step(i, per_call_events=None, dom_events=None):
        """One pass over the eight projections.  per_call_events brackets every call (breakdown
        pass); dom_events brackets only the adjacent gate/up launches (timed pass), so the timed
        stream carries two event records per step instead of sixteen."""
        row = calls[i % args.copies]
        for j, call in enumerate(row):
            if per_call_events is not None:
                per_call_events[j][0].record()
            elif dom_events is not None and j == dom_idx[0]:
                dom_events[0].record()
            call()
            if per_call_events is not None:
                per_call_events[j][1].record()
            elif dom_events is not None and j == dom_idx[-1]:
                dom_events[1].record()

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: the steps back to back on one stream, events only around gate/up
    n = len(projections)
    dom_ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(i, dom_events=dom_ev[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    dom_us = sum(e[0].elapsed_time(e[1]) for e in dom_ev) * 1e3 / (args.steps * len(dom_idx))

    # breakdown pass (not timed as a whole): events around every call
    bsteps = max(3, min(args.steps, 10))
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(n)]
          for _ in range(bsteps)]
    for i in range(bsteps):
        step(i, per_call_events=ev[i])
    torch.cuda.synchronize()
    per = []
    for j, p in enumerate(projections):
        us = sorted(ev[i][j][0].elapsed_time(ev[i][j][1]) * 1e3 for i in range(bsteps))
        avg = sum(us) / len(us)
        f, by = flops(p["M"], p["N"], p["K"]), algo_bytes(p["M"], p["N"], p["K"])
        pl = plans[j]
        per.append({"name": p["name"], "M": p["M"], "N": p["N"], "K": p["K"], "avg_us": round(avg, 3),
                    "median_us": round(us[len(us) // 2], 3), "TFLOP/s": round(f / avg / 1e6, 2),
                    "GB/s": round(by / avg / 1e3, 1),
                    "path": "qmv" if pl["path"] == 1 else "qmm", "variant": pl["variant"],
                    "tile": [pl["tile_m"], pl["tile_n"]], "split_k": pl["split_k"]})
    step_flops = sum(flops(p["M"], p["N"], p["K"]) for p in projections)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    dom = [per[j] for j in dom_idx]
    dom_flops = flops(M_PREFILL, *synth_shape("gate"))
    achieved = dom_flops / dom_us / 1e6
    traffic = load_traffic()
    vocab = per[-1]
    vocab_bytes = algo_bytes(1, vocab["N"], vocab["K"])

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill512_layer_projections+vocab_last_row", "M": M_PREFILL,
                   "projections": {p["name"]: [p["K"], p["N"]] for p in projections}, "group": 128,
                   "weight_copies": args.copies, "logits_to_keep": 1},
        "roofline": {"bound": "mfma",
                     "kernel": f"qmm {dom[0]['tile'][0]}x{dom[0]['tile'][1]} tile (gate/up, M=512, K=2560, N=9728)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flops_per_launch": dom_flops, "avg_launch_us": round(dom_us, 3),
                     "timing": "HIP events around the adjacent gate and up launches of every timed step "
                               "(on the launch stream), divided by the two launches"},
        "breakdown_timing": "separate pass after the timed region: HIP events around every call",
        "qmv_vocab_last_row": {"GB/s": round(vocab_bytes / vocab["avg_us"] / 1e3, 1),
                               "frac_hbm": round(vocab_bytes / vocab["avg_us"] / 1e3 / PEAK_HBM_GBPS, 4),
                               "avg_us": vocab["avg_us"], "bytes": vocab_bytes},
        "breakdown": per,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    if not args.no_next_rows:
        gs = torch.cuda.Stream()         # graph capture needs a stream other than the null stream
        with torch.cuda.stream(gs):
            result["next_rows"] = next_rows(torch, w4, projections, args.copies)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on one step", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(projections)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def time_call(torch, fns, reps, trials=5):
    """Microseconds per call on the GPU: ``reps`` calls (rotating over ``fns``, one per weight
    copy) are captured in one HIP graph on the current stream (the calls must have been prepared
    on it) and replayed ``trials`` times between HIP events on that stream; the median replay
    divided by ``reps``.  Replaying a graph removes the host's launch cost between calls, so short
    kernels are timed back to back as a model's decode step would issue them."""
    stream = torch.cuda.current_stream()
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            fns[i % len(fns)]()
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(trials):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        b.synchronize()
        per.append(a.elapsed_time(b) * 1e3 / reps)
    del g
    return sorted(per)[len(per) // 2]


ROTATE_BYTES = 600 << 20   # weight bytes cycled per timed case: over twice the 256 MB last-level cache


def rotation(w, min_bytes=ROTATE_BYTES):
    """The weight set ``w`` (wq, scales, biases) and enough device clones of it that one pass over
    them reads at least ``min_bytes``, so every call's weights come from HBM."""
    nbytes = sum(t.numel() * t.element_size() for t in w)
    n = max(2, -(-min_bytes // nbytes))
    return [w] + [tuple(t.clone() for t in w) for _ in range(n - 1)]


def ws_for(torch, nbytes, device):
    return torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=device) if nbytes else None


def next_rows(torch, w4, projections, copies, reps=20):
    """Measurements of the rows beyond the step, each case timed alone on the current (side)
    stream from a HIP graph over a weight rotation of more than 512 MB:
      * the fused gate/up + SwiGLU pair at the step's 512 rows against the two projections and
        against gate, up, then a framework-style bf16 SiLU and product;
      * the skinny path (16 and 32 rows) against the 64-row tiles on the gate and down shapes;
      * W4A8 (int8 activations) against W4A16 on the step's seven projections;
      * the 4096-row prefill of gate / up / down and the vocabulary head over all rows;
      * the 128-row prefill of the seven layer projections (and their sum as one layer);
      * decode rows (M = 1, 4) on the four decode shapes, and the width-generic matvec at
        1, 2, 3, 4 and 8 bits."""
    from w4a16_group_quantized_qmv_amd import synth
    by = {p["name"]: p for p in projections}
    dev = by["gate"]["x"].device
    out = {}

    def timed(fns):
        return time_call(torch, fns, max(reps, len(fns)))

    # fused gate / up + SwiGLU
    gate, up = by["gate"], by["up"]
    x = gate["x"]
    M, N, K = gate["M"], gate["N"], gate["K"]
    rot_g, rot_u = rotation(gate["w"][0]), rotation(up["w"][0])
    n = min(len(rot_g), len(rot_u))
    h = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fused = [w4.PreparedGateUp(x, rot_g[c], rot_u[c], h=h) for c in range(n)]
    g_out, u_out = torch.empty_like(h), torch.empty_like(h)
    sep_g = [w4.PreparedLinear(x, *rot_g[c], y=g_out) for c in range(n)]
    sep_u = [w4.PreparedLinear(x, *rot_u[c], y=u_out) for c in range(n)]

    def unfused(c):       # the unfused epilogue as a framework runs it: bf16 SiLU, then the product
        return lambda: (sep_g[c](), sep_u[c](), torch.nn.functional.silu(g_out).mul_(u_out))

    t_fused = timed(fused)
    t_sep = timed([(lambda c=c: (sep_g[c](), sep_u[c]())) for c in range(n)])
    t_unfused = timed([unfused(c) for c in range(n)])
    f2 = 2 * flops(M, N, K)
    out["fused_gate_up_swiglu"] = {
        "M": M, "N": N, "K": K, "plan": {k: fused[0].plan[k] for k in ("tile_m", "tile_n", "split_k", "variant")},
        "fused_us": round(t_fused, 3), "gate_plus_up_us": round(t_sep, 3),
        "unfused_gate_up_silu_mul_us": round(t_unfused, 3),
        "speedup_vs_unfused": round(t_unfused / t_fused, 3), "TFLOP/s": round(f2 / t_fused / 1e6, 2),
        "frac_mfma": round(f2 / t_fused / 1e6 / PEAK_BF16_TFLOPS, 4)}
    del fused, sep_g, sep_u, rot_g, rot_u

    # skinny rows
    skinny = []
    for name in ("gate", "down"):
        p = by[name]
        rot = rotation(p["w"][0])
        for m in (16, 32):
            xs = p["x"][:m]
            y = torch.empty((m, p["N"]), dtype=torch.bfloat16, device=dev)
            pa = w4.w4a16_plan(m, p["N"], p["K"], 128, w4.PATH_AUTO, 0)
            pt = w4.w4a16_plan(m, p["N"], p["K"], 128, w4.PATH_QMM, 0)
            wa, wt = ws_for(torch, pa["workspace_bytes"], dev), ws_for(torch, pt["workspace_bytes"], dev)
            auto = [w4.PreparedLinear(xs, *w, y=y, workspace=wa) for w in rot]
            tiled = [w4.PreparedLinear(xs, *w, y=y, path="qmm", workspace=wt) for w in rot]
            t_a, t_t = timed(auto), timed(tiled)
            b = algo_bytes(m, p["N"], p["K"])
            skinny.append({"name": name, "M": m, "N": p["N"], "K": p["K"], "tile_m": pa["tile_m"],
                           "split_k": pa["split_k"], "skinny_us": round(t_a, 3),
                           "tiled64_us": round(t_t, 3), "GB/s": round(b / t_a / 1e3, 1),
                           "frac_hbm": round(b / t_a / 1e3 / PEAK_HBM_GBPS, 4)})
        del rot
    out["skinny"] = skinny

    # W4A8 against W4A16 on the step's projections
    w4a8 = []
    for name in LAYER:
        p = by[name]
        rot = rotation(p["w"][0])
        y = torch.empty((p["M"], p["N"]), dtype=torch.bfloat16, device=dev)
        w8 = ws_for(torch, w4.w4a8_linear_workspace_bytes(p["M"], p["N"], p["K"]), dev)
        w16 = ws_for(torch, w4.w4a16_workspace_bytes(p["M"], p["N"], p["K"]), dev)
        t8 = timed([w4.PreparedW4A8(p["x"], *w, y=y, workspace=w8) for w in rot])
        t16 = timed([w4.PreparedLinear(p["x"], *w, y=y, workspace=w16) for w in rot])
        f = flops(p["M"], p["N"], p["K"])
        w4a8.append({"name": name, "M": p["M"], "N": p["N"], "K": p["K"],
                     "split_k": w4.w4a8_plan(p["M"], p["N"], p["K"])["split_k"],
                     "w4a8_us": round(t8, 3), "w4a16_us": round(t16, 3), "w4a8_TOP/s": round(f / t8 / 1e6, 2),
                     "frac_int8_mfma": round(f / t8 / 1e6 / PEAK_INT8_TOPS, 4)})
        del rot
    out["w4a8"] = w4a8

    # 4096-row prefill: gate / up / down and the vocabulary head over all rows
    long_rows = []
    for name, src in (("gate", "gate"), ("up", "up"), ("down", "down"), ("vocab_all_rows", "vocab_last_row")):
        p = by[src]
        sname = "vocab" if src == "vocab_last_row" else src
        xl = torch.from_numpy(synth.activations(5, synth.shape_index(5, sname), 4096, p["K"]).view("int16"))
        xl = xl.view(torch.bfloat16).to(dev)
        rot = rotation(p["w"][0])
        pl = w4.w4a16_plan(4096, p["N"], p["K"])
        y = torch.empty((4096, p["N"]), dtype=torch.bfloat16, device=dev)
        wsb = ws_for(torch, pl["workspace_bytes"], dev)
        fns = [w4.PreparedLinear(xl, *w, y=y, workspace=wsb) for w in rot]
        t = time_call(torch, fns, max(len(fns), 4 if src == "vocab_last_row" else reps))
        f = flops(4096, p["N"], p["K"])
        long_rows.append({"name": name, "M": 4096, "N": p["N"], "K": p["K"], "tile_m": pl["tile_m"],
                          "exact_codes": pl["variant"] >= 10, "avg_us": round(t, 3),
                          "TFLOP/s": round(f / t / 1e6, 2), "frac_mfma": round(f / t / 1e6 / PEAK_BF16_TFLOPS, 4)})
        del fns, rot, y, xl
    out["prefill4096"] = long_rows

    # 128-row prefill: the seven layer projections, each alone
    short_rows = []
    for name in LAYER:
        p = by[name]
        xs = torch.from_numpy(synth.activations(3, synth.shape_index(3, name), 128, p["K"]).view("int16"))
        xs = xs.view(torch.bfloat16).to(dev)
        rot = rotation(p["w"][0])
        pl = w4.w4a16_plan(128, p["N"], p["K"])
        y = torch.empty((128, p["N"]), dtype=torch.bfloat16, device=dev)
        wsb = ws_for(torch, pl["workspace_bytes"], dev)
        t = timed([w4.PreparedLinear(xs, *w, y=y, workspace=wsb) for w in rot])
        f = flops(128, p["N"], p["K"])
        short_rows.append({"name": name, "M": 128, "N": p["N"], "K": p["K"], "tile": [pl["tile_m"], pl["tile_n"]],
                           "split_k": pl["split_k"], "avg_us": round(t, 3), "TFLOP/s": round(f / t / 1e6, 2),
                           "frac_mfma": round(f / t / 1e6 / PEAK_BF16_TFLOPS, 4)})
        del rot, y, xs
    layer_flops = sum(flops(128, r["N"], r["K"]) for r in short_rows)
    out["prefill128"] = {"projections": short_rows,
                         "layer_TFLOP/s": round(layer_flops / sum(r["avg_us"] for r in short_rows) / 1e6, 2)}

    # decode rows on the four decode shapes
    decode = []
    for i, (K, N) in enumerate(synth.DECODE_SHAPES):
        wq, sc, bi = synth.weights(2, i, N, K)
        w0 = (torch.from_numpy(wq.view("int32")).to(dev), torch.from_numpy(sc.view("int16")).view(torch.bfloat16).to(dev),
              torch.from_numpy(bi.view("int16")).view(torch.bfloat16).to(dev))
        rot = rotation(w0)
        for m in (1, 4):
            xd = torch.from_numpy(synth.activations(2, i, m, K).view("int16")).view(torch.bfloat16).to(dev)
            y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            pl = w4.w4a16_plan(m, N, K)
            t = timed([w4.PreparedLinear(xd, *w, y=y) for w in rot])
            b = algo_bytes(m, N, K)
            decode.append({"K": K, "N": N, "M": m, "variant": pl["variant"], "avg_us": round(t, 3),
                           "GB/s": round(b / t / 1e3, 1), "frac_hbm": round(b / t / 1e3 / PEAK_HBM_GBPS, 4)})
        del rot
    out["decode"] = decode

    # width-generic matvec on the 2560 -> 9728 shape
    bits_rows = []
    K, N = synth.DECODE_SHAPES[0]
    for bits in (1, 2, 3, 4, 8):
        pr = synth.random_problem(40 + bits, 4, N, K, bits=bits)
        w0 = (torch.from_numpy(pr["wq"].view("int32")).to(dev),
              torch.from_numpy(pr["scales"].view("int16")).view(torch.bfloat16).to(dev),
              torch.from_numpy(pr["biases"].view("int16")).view(torch.bfloat16).to(dev))
        rot = rotation(w0)
        xb = torch.from_numpy(pr["x"].view("int16")).view(torch.bfloat16).to(dev)
        for m in (1, 4):
            y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            xm = xb[:m]
            t = timed([(lambda w=w: w4.qmv_affine(xm, *w, bits=bits, y=y)) for w in rot])
            b = N * K * bits / 8 + N * K / 32 + 2.0 * m * K + 2.0 * m * N
            bits_rows.append({"bits": bits, "K": K, "N": N, "M": m, "avg_us": round(t, 3),
                              "GB/s": round(b / t / 1e3, 1), "frac_hbm": round(b / t / 1e3 / PEAK_HBM_GBPS, 4)})
        del rot
    out["qmv_affine_bits"] = bits_rows
    out["timing"] = ("after the timed region: each case alone, its calls over a weight rotation of more than "
                     "512 MB replayed from a HIP graph on a side stream, median of 5 replays")
    return out


def synth_shape(name):
    from w4a16_group_quantized_qmv_amd import synth
    K, N = synth.LAYER_SHAPES[name]
    return N, K


if __name__ == "__main__":
    main()

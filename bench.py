#!/usr/bin/env python3
"""Benchmark of the W4A16 group-quantized projection hot path on one MI355X.

One step is one 512-token prefill pass through the projections of one decoder layer
(hidden 2560, 32 query heads and 8 key/value heads of dimension 128, MLP 9728: q, k, v, o,
gate, up, down at M = 512, where the down projection's K = 9728 exercises split-K), in layer
order and launched as a serving stack would: q, k and v read the same input and run as one
grouped launch; gate and up read the same input and run as the fused gate / up + SwiGLU pair,
whose output h = silu(gate) * up is the down projection's input), followed
by the vocabulary head (2560 -> 151936) applied to the last row only (logits_to_keep = 1,
which dispatches to the matvec path).  These are the per-projection prefill shapes that
tiny-llm's "Week 2 Day 6: SIMD-Matrix Prefill" benchmarks in Task 5 and its Benchmark
Analysis, with Task 4's last-row slice before the vocabulary projection.  Inputs are seeded
synthetic data (the pages' Qwen3-4B weights are not available): x ~ N(0, 1) in bf16,
W ~ N(0, 0.02) quantized to 4-bit affine groups of 128.

All inputs are resident in HBM before the timed region.  Weight sets rotate over several
device copies so that weight reads miss the 256 MB last-level cache.  Output: one JSON line.

    python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--no-cpu-baseline] [--no-next-rows]

Besides the step's throughput the line carries: the dominant kernel's roofline (the fused
gate / up pair's tile kernel, from its own start and end timestamps in every timed step), the
same run's measured ceilings (torch's
bf16 GEMM through hipBLASLt on the same shapes, and device copy / read rates), every timed
shape's fraction of the roof that binds it (min(MFMA peak, arithmetic intensity x HBM
bandwidth)), and the CPU oracle on a bounded sample of the step.
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
INPUT_OF = {"k": "q", "v": "q", "up": "gate"}   # projections that read another's input
GROUPED = ("q", "k", "v")     # one grouped launch in the step (same input)
FUSED = ("gate", "up")        # one fused gate / up + SwiGLU launch; its h is down's input
DOMINANT = "gate|up"          # the largest launch of the step: the roofline kernel
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qmm_prefill512_gate_up_traffic.json")
KERNEL_SOURCES = ["w4a16_group_quantized_qmv_amd/csrc/qmm.hip", "w4a16_group_quantized_qmv_amd/csrc/device_common.h"]


def flops(M, N, K):
    return 2.0 * M * N * K


def algo_bytes(M, N, K):
    """Algorithmic bytes: packed codes + bf16 scale and bias per group + x + y."""
    return N * K / 2 + N * K / 32 + 2.0 * M * K + 2.0 * M * N


def roof(M, N, K, achieved_tflops):
    """Roofline of one projection: arithmetic intensity (flop per algorithmic byte), the roof that
    binds it (MFMA peak or AI x HBM bandwidth, whichever is lower) and the achieved fraction."""
    ai = flops(M, N, K) / algo_bytes(M, N, K)
    hbm_roof = ai * PEAK_HBM_GBPS / 1e3          # TFLOP/s that HBM can feed at this intensity
    bound = "mfma" if PEAK_BF16_TFLOPS <= hbm_roof else "hbm"
    r = min(PEAK_BF16_TFLOPS, hbm_roof)
    return {"AI": round(ai, 1), "bound": bound, "roof_TFLOP/s": round(r, 1),
            "roofline_frac": round(achieved_tflops / r, 4)}


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
    shared = {}
    for name in LAYER:
        idx = synth.shape_index(4, name)
        K, N = synth.LAYER_SHAPES[name]
        wq, s, b = synth.weights(4, idx, N, K)
        # one input per group of projections that read the same activations in a layer: q, k and
        # v read the attention input, gate and up the MLP input
        src = INPUT_OF.get(name, name)
        if src not in shared:
            xs = synth.activations(4, synth.shape_index(4, src), M_PREFILL, K)
            shared[src] = (xs, bf16(xs))
        x, xd = shared[src]
        projections.append({"name": name, "M": M_PREFILL, "N": N, "K": K, "keep": 0,
                            "host": {"x": x, "wq": wq, "scales": s, "biases": b},
                            "x": xd, "w": [(torch.from_numpy(wq.view(np.int32)).to(dev), bf16(s), bf16(b))]})
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(projections):
    """The oracle, untuned, on a bounded sample of one step: the seven 512-row projections in
    full and the last vocab row over the first quarter of the vocabulary columns.  Timed: the
    oracle's definition of the projection -- unpack, fp32 dequantization (``dequant_f32``) and
    the fp64 GEMM ``x64 @ w64.T`` over the same column chunks as ``reference`` -- without the
    absolute-mass GEMM that ``reference`` adds for the tolerance, so the rate counts the one
    GEMM that is timed."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    affinity = len(os.sched_getaffinity(0))
    total_flops = 0.0
    t0 = time.perf_counter()
    for p in projections:
        h = p["host"]
        x = h["x"][-p["keep"]:] if p["keep"] else h["x"]
        n = p["N"] if not p["keep"] else VOCAB_SAMPLE_COLS
        x64 = O.bf16_to_f64(x)
        for c0 in range(0, n, 8192):
            c1 = min(n, c0 + 8192)
            w64 = O.dequant_f32(h["wq"][c0:c1], h["scales"][c0:c1], h["biases"][c0:c1], p["K"]).astype(np.float64)
            _ = x64 @ w64.T
        total_flops += flops(x.shape[0], n, p["K"])
    dt = time.perf_counter() - t0
    return {"value": total_flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads or affinity),
            "kind": "oracle",
            "sample": "the seven 512-row layer projections in full and the last vocab row over the first "
                      f"{VOCAB_SAMPLE_COLS} of 151936 columns: the oracle's unpack + fp32 dequant + fp64 GEMM "
                      "(dequant_f32, x64 @ w64.T in 8192-column chunks), wall clock, rate = sample FLOPs / time",
            "seconds": round(dt, 3), "cpu_model": cpu_model(), "affinity_cores": affinity,
            "blas_threads": blas_threads}


READ_FLOOR_SHAPES = ((1024, 2560), (4096, 2560), (9728, 2560), (151936, 2560))


def read_floor_key(N, K):
    """The measured read floor that stands for a matvec shape (the transposed 13 MB shape shares
    its partner's)."""
    return f"read_{max(N, K)}x{min(N, K)}_us" if N * K == 9728 * 2560 else f"read_{N}x{K}_us"


def measured_ceilings(torch, reps=50):
    """This run's own denominators on the same GPU: torch's bf16 GEMM (hipBLASLt) on the gate
    shape (K = 2560, N = 9728) at 512 and 4096 rows, a 1 GiB device-to-device copy (read +
    write) and a 1 GiB streaming read (the package's read probe, libw4a16_probe.so: 16-byte
    non-temporal loads, four in flight per thread, 2048 workgroups)."""
    import ctypes
    dev = torch.device("cuda", 0)
    out = {}

    def timed(fn, n):
        for _ in range(5):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / n          # us per call

    g = torch.Generator(device=dev)
    g.manual_seed(1)
    for M in (512, 4096):
        a = torch.randn((M, 2560), generator=g, device=dev).to(torch.bfloat16)
        w = torch.randn((9728, 2560), generator=g, device=dev).to(torch.bfloat16)
        us = timed(lambda: torch.nn.functional.linear(a, w), reps)
        out[f"bf16_gemm_M{M}_TFLOP/s"] = round(flops(M, 9728, 2560) / us / 1e6, 1)
        del a, w
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    us = timed(lambda: dst.copy_(src), 10)
    out["copy_GB/s"] = round(2 * (1 << 30) / us / 1e3, 1)
    probe = ctypes.CDLL(os.path.join(ROOT, "w4a16_group_quantized_qmv_amd", "libw4a16_probe.so"))
    probe.w4a16_probe_stream_read.restype = ctypes.c_int
    probe.w4a16_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_void_p]
    blocks = 2048
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def read():
        st = probe.w4a16_probe_stream_read(src.data_ptr(), 1 << 30, sink.data_ptr(), blocks, hs)
        assert st == 0, st
    us = timed(read, 10)
    out["read_GB/s"] = round((1 << 30) / us / 1e3, 1)
    # the same probe over the bytes of each matvec shape (N x K; 2560 x 9728 moves the bytes of
    # 9728 x 2560 to within 0.1%), each call on the next window of the 1 GiB buffer so that it
    # comes from HBM, replayed from a HIP graph as the matvec timings are
    gs = torch.cuda.Stream()
    with torch.cuda.stream(gs):
        hg = ctypes.c_void_p(gs.cuda_stream)
        for name, nbytes in ((f"{N}x{K}", algo_bytes(1, N, K)) for N, K in READ_FLOOR_SHAPES):
            nb = int(nbytes) // 256 * 256
            windows = max(2, (1 << 30) // nb)
            nblk = max(1, min(blocks, -(-nb // (256 * 64))))
            calls = [lambda off=(i % windows) * nb: probe.w4a16_probe_stream_read(src.data_ptr() + off, nb,
                                                                                 sink.data_ptr(), nblk, hg)
                     for i in range(max(20, windows))]
            us = time_call(torch, calls, len(calls))
            out[f"read_{name}_us"] = round(us, 3)
            out[f"read_{name}_GB/s"] = round(nb / us / 1e3, 1)
    del src, dst, sink
    torch.cuda.synchronize()
    out["how"] = ("torch.nn.functional.linear in bf16 (x [M, 2560] by W [9728, 2560]), Tensor.copy_ of 1 GiB, "
                  "the streaming-read probe over 1 GiB; HIP events, mean over back-to-back calls; read_<size>: the "
                  "probe over one matvec's algorithmic bytes, graph-replayed over successive windows of 1 GiB")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--copies", type=int, default=3, help="device copies of the weights, rotated per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the measurements beyond the step (for profiler runs of the step alone)")
    ap.add_argument("--profile-decode", action="store_true",
                    help="only run the decode matvecs (M = 1 and 4 on the four decode shapes, and the vocab "
                         "head's last row) a few times each with plain launches, for profiler runs, then exit")
    ap.add_argument("--profile-long", action="store_true",
                    help="only run the 4096-row gate, up and down projections a few times each with plain "
                         "launches, for profiler runs, then exit")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured ceilings (torch bf16 GEMM, copy and read rates)")
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
    if args.profile_decode:
        profile_decode(torch, w4)
        return
    if args.profile_long:
        profile_long(torch, w4)
        return
    t_gen = time.perf_counter()
    projections = build_inputs(torch, args.copies)
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    # launch units of the step, in layer order: q|k|v (one grouped call), o, gate|up (the fused
    # SwiGLU pair; its output h is the down projection's input), down, the vocabulary head's last
    # row.  Prepared once per weight copy, outputs shared across copies.
    by_name = {p["name"]: p for p in projections}
    units = [[by_name[n] for n in GROUPED], [by_name["o"]], [by_name[n] for n in FUSED], [by_name["down"]],
             [by_name["vocab_last_row"]]]
    unit_names = ["|".join(p["name"] for p in u) for u in units]
    calls = []
    for c in range(args.copies):
        row = []
        h = None
        for u, name in zip(units, unit_names):
            prev = calls[0][len(row)] if calls else None
            if name == "q|k|v":
                row.append(w4.PreparedGrouped(u[0]["x"], [p["w"][c] for p in u], ys=prev.ys if prev else None))
            elif name == "gate|up":
                row.append(w4.PreparedGateUp(u[0]["x"], u[0]["w"][c], u[1]["w"][c], h=prev.h if prev else None))
                h = row[-1].h
            else:
                p = u[0]
                x = h if name == "down" else (p["x"][-p["keep"]:] if p["keep"] else p["x"])
                wq, s, b = p["w"][c]
                row.append(w4.PreparedLinear(x, wq, s, b, y=prev.y if prev else None))
        calls.append(row)
    plans = [call.plan for call in calls[0]]

    dom_idx = [unit_names.index(DOMINANT)]
    assert dom_idx == list(range(dom_idx[0], dom_idx[0] + len(dom_idx))), "dominant projections must be adjacent"

    def step(i, starts=None, ends=None, kernel_events=None):
        """One pass over the step's launch units (q|k|v grouped, o, gate|up, down, vocab).  ``starts`` /
        ``ends`` map a call's index to a HIP event recorded on the stream just before / after it:
        every call in the breakdown pass, the fused gate|up call in the timed pass.
        ``kernel_events`` maps a call's index to an event pair that its tile kernel's own start and
        end timestamps go to (w4a16_time_next_launch)."""
        row = calls[i % args.copies]
        for j, call in enumerate(row):
            if kernel_events is not None and j in kernel_events:
                w4.w4a16_time_next_launch(*kernel_events[j])
            if starts is not None and j in starts:
                starts[j].record()
            call()
            if ends is not None and j in ends:
                ends[j].record()

    ceilings = measured_ceilings(torch) if not args.no_ceilings else None
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

    def event_pair():
        return [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]

    # timed region: the steps back to back on one stream; in every step the fused gate|up call is
    # bracketed by two events on the stream, and its tile kernel puts its own start and end
    # timestamps on two more (the HIP handles exist once each event has been recorded)
    n = len(units)
    dom_ev = [event_pair() for _ in range(args.steps)]
    dom_kev = [event_pair() for _ in range(args.steps)]
    for e in dom_kev:
        e[0].record()
        e[1].record()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(i, {dom_idx[0]: dom_ev[i][0]}, {dom_idx[-1]: dom_ev[i][1]}, {dom_idx[0]: dom_kev[i]})
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    dom_bracket_us = [e[0].elapsed_time(e[1]) * 1e3 for e in dom_ev]
    dom_kernel_us = [e[0].elapsed_time(e[1]) * 1e3 for e in dom_kev]
    dom_bracket = sum(dom_bracket_us) / len(dom_bracket_us)
    # every kernel span must lie inside the events recorded around its call; otherwise the
    # kernel timestamps were not taken and the bracket is reported instead
    kernel_spans_ok = all(0.0 < k <= b for k, b in zip(dom_kernel_us, dom_bracket_us))
    dom_us = sum(dom_kernel_us) / len(dom_kernel_us) if kernel_spans_ok else dom_bracket

    # breakdown passes (not timed as a whole): events around every call; then, in a pass of its
    # own (arming the request costs host time that would open gaps inside the brackets), every
    # call's contraction kernel (the tile or matvec kernel; not a slice sum) timestamped by itself
    bsteps = max(3, min(args.steps, 10))
    ev = [{j: event_pair() for j in range(n)} for _ in range(bsteps)]
    for i in range(bsteps):
        step(i, {j: e[0] for j, e in ev[i].items()}, {j: e[1] for j, e in ev[i].items()})
    torch.cuda.synchronize()
    kev = [{j: event_pair() for j in range(n)} for _ in range(bsteps)]
    for e in (e for row in kev for pair in row.values() for e in pair):
        e.record()
    torch.cuda.synchronize()
    for i in range(bsteps):
        step(i, kernel_events=kev[i])
    torch.cuda.synchronize()
    per = []
    for j, u in enumerate(units):
        us = sorted(ev[i][j][0].elapsed_time(ev[i][j][1]) * 1e3 for i in range(bsteps))
        kus = sorted(kev[i][j][0].elapsed_time(kev[i][j][1]) * 1e3 for i in range(bsteps))
        avg = sum(us) / len(us)
        kavg = sum(kus) / len(kus)
        M, K, N = u[0]["M"], u[0]["K"], sum(p["N"] for p in u)
        f = sum(flops(p["M"], p["N"], p["K"]) for p in u)
        # one x for the unit (grouped projections read it once)
        by = sum(algo_bytes(p["M"], p["N"], p["K"]) for p in u) - 2.0 * M * K * (len(u) - 1)
        pl = plans[j]
        path = {1: "qmv", w4.PATH_GROUPED: "qmm grouped", w4.PATH_GATE_UP: "qmm gate/up + SwiGLU"}.get(pl["path"], "qmm")
        per.append({"name": unit_names[j], "M": M, "N": N, "K": K, "avg_us": round(avg, 3),
                    "median_us": round(us[len(us) // 2], 3), "kernel_us": round(kavg, 3),
                    "TFLOP/s": round(f / avg / 1e6, 2),
                    "GB/s": round(by / avg / 1e3, 1),
                    "path": path, "variant": pl["variant"],
                    "tile": [pl["tile_m"], pl["tile_n"]], "split_k": pl["split_k"],
                    **roof(M, N, K, f / avg / 1e6)})
    step_flops = sum(flops(p["M"], p["N"], p["K"]) for p in projections)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    dom = [per[j] for j in dom_idx]
    dom_flops = sum(flops(p["M"], p["N"], p["K"]) for p in units[dom_idx[0]])
    achieved = dom_flops / dom_us / 1e6
    traffic = load_traffic()
    vocab = per[-1]
    vocab_bytes = algo_bytes(1, vocab["N"], vocab["K"])
    # the matvec's kernel span (its own pass) must be positive and not longer than the calls'
    # event brackets; otherwise the bracket is used
    vocab_kernel_ok = 0.0 < vocab["kernel_us"] <= vocab["avg_us"] * 1.05
    vocab_us = vocab["kernel_us"] if vocab_kernel_ok else vocab["avg_us"]

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill512_layer_projections+vocab_last_row", "M": M_PREFILL,
                   "projections": {p["name"]: [p["K"], p["N"]] for p in projections}, "group": 128,
                   "launches": unit_names, "weight_copies": args.copies, "logits_to_keep": 1},
        "roofline": {"bound": "mfma",
                     "kernel": f"qmm gate/up + SwiGLU pair, {dom[0]['tile'][0]}x{dom[0]['tile'][1]} tiles of h "
                               "(M=512, K=2560, N=9728 per projection)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flops_per_launch": dom_flops, "avg_launch_us": round(dom_us, 3),
                     "launches": len(dom_kernel_us),
                     "avg_call_bracket_us": round(dom_bracket, 3),
                     "frac_of_measured_bf16_gemm": (round(achieved / ceilings["bf16_gemm_M512_TFLOP/s"], 4)
                                                    if ceilings else None),
                     "the_measured_bf16_gemm": "torch.nn.functional.linear on one of the pair's projections (same "
                                               "per-projection shape)",
                     "timing": ("the tile kernel's own start and end timestamps (hipExtLaunchKernel events, armed "
                                "by w4a16_time_next_launch) in every timed step, mean over the timed steps; "
                                "avg_call_bracket_us: events recorded on the stream just before and after the "
                                "same calls, which also span the dispatch and the end-of-kernel cache flush"
                                if kernel_spans_ok else
                                "FALLBACK: a kernel timestamp span did not lie inside its call's events, so "
                                "avg_launch_us is the mean of the events recorded on the stream around each "
                                "timed call")},
        "measured_ceiling": ceilings,
        "breakdown_timing": "separate pass after the timed region: HIP events around every call (avg_us, "
                            "median_us, and the rates); kernel_us: the call's tile or matvec kernel alone, from "
                            "its own timestamps",
        "qmv_vocab_last_row": {"GB/s": round(vocab_bytes / vocab_us / 1e3, 1),
                               "frac_of_measured_read_floor": (round(ceilings[read_floor_key(vocab["N"], vocab["K"])]
                                                                     / vocab_us, 4) if ceilings else None),
                               "frac_hbm": round(vocab_bytes / vocab_us / 1e3 / PEAK_HBM_GBPS, 4),
                               "frac_of_measured_read": (round(vocab_bytes / vocab_us / 1e3 /
                                                               ceilings["read_GB/s"], 4) if ceilings else None),
                               "kernel_us": vocab["kernel_us"], "avg_call_us": vocab["avg_us"],
                               "GB/s_call": round(vocab_bytes / vocab["avg_us"] / 1e3, 1), "bytes": vocab_bytes,
                               "timing": ("the matvec kernel's own timestamps in the breakdown pass (mean of its "
                                          "calls); GB/s_call: events around the same calls" if vocab_kernel_ok else
                                          "FALLBACK: the kernel span exceeded the calls' event brackets, so the rates "
                                          "use the brackets")},
        "breakdown": per,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    if not args.no_next_rows:
        gs = torch.cuda.Stream()         # graph capture needs a stream other than the null stream
        with torch.cuda.stream(gs):
            result["next_rows"] = next_rows(torch, w4, projections, args.copies)
        if ceilings:
            for row in result["next_rows"]["decode"]:
                floor = ceilings.get(read_floor_key(row["N"], row["K"]))
                row["frac_of_measured_read"] = round(floor / row["avg_us"], 4) if floor else None
        # the metric's qmv part: the decode matvec at M = 1 on the largest decode shape
        m1 = [r for r in result["next_rows"]["decode"] if r["M"] == 1]
        if m1:
            top = max(m1, key=lambda r: (r["N"] * r["K"], r["N"]))
            result["qmv_decode_M1"] = {
                "shape": f"{top['K']}->{top['N']}", "GB/s": top["GB/s"], "frac_hbm": top["frac_hbm"],
                "frac_of_measured_read": top.get("frac_of_measured_read"), "avg_us": top["avg_us"],
                "all_M1": {f"{r['K']}->{r['N']}": r["GB/s"] for r in m1},
                "timing": "graph-replayed launches over a weight rotation of more than 512 MB (next_rows.decode)"}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on one step", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(projections)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def profile_decode(torch, w4, calls=5):
    """The decode matvecs alone, with plain stream launches (no graph), so a profiler attributes
    kernel durations and counters to each shape by its launch grid: M = 1 and 4 on 2560 -> 9728,
    9728 -> 2560, 2560 -> 4096, 2560 -> 1024, then the vocabulary head's last row (2560 ->
    151936, M = 1).  Each shape runs ``calls`` passes over a weight rotation of more than twice
    the last-level cache, one launch per weight copy, so every launch reads its weights from HBM."""
    import numpy as np
    from w4a16_group_quantized_qmv_amd import synth
    dev = torch.device("cuda", 0)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    cases = [(2, i, K, N) for i, (K, N) in enumerate(synth.DECODE_SHAPES)]
    cases.append((5, synth.shape_index(5, "vocab"), *synth.VOCAB_SHAPE))
    for cfg, idx, K, N in cases:
        wq, s, b = synth.weights(cfg, idx, N, K)
        rot = rotation((torch.from_numpy(wq.view(np.int32)).to(dev), bf16(s), bf16(b)))
        for m in ((1, 4) if cfg == 2 else (1,)):
            x = bf16(synth.activations(cfg, idx, m, K))
            prepared = [w4.PreparedLinear(x, *w) for w in rot]
            for _ in range(calls):
                for call in prepared:
                    call()
            torch.cuda.synchronize()
            plan = prepared[0].plan
            print(f"[profile-decode] M={m} K={K} N={N} plan variant {plan['variant']} grid {plan['grid_x']} "
                  f"x {plan['block_threads']} threads, {calls} x {len(rot)} launches", file=sys.stderr, flush=True)
            del prepared
        del rot
        torch.cuda.synchronize()


def profile_long(torch, w4, calls=3):
    """The 4096-row prefill projections alone (gate 2560 -> 9728, up 2560 -> 9728, down 9728 ->
    2560, the synthetic inputs of the long-prefill workload), each ``calls`` times with plain
    stream launches, so a profiler attributes kernel durations and counters to each by its grid."""
    import numpy as np
    from w4a16_group_quantized_qmv_amd import synth
    dev = torch.device("cuda", 0)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    for name in ("gate", "up", "down"):
        idx = synth.shape_index(5, name)
        K, N = synth.LAYER_SHAPES[name]
        wq, s, b = synth.weights(5, idx, N, K)
        x = bf16(synth.activations(5, idx, 4096, K))
        call = w4.PreparedLinear(x, torch.from_numpy(wq.view(np.int32)).to(dev), bf16(s), bf16(b))
        for _ in range(calls):
            call()
        torch.cuda.synchronize()
        plan = call.plan
        print(f"[profile-long] {name} M=4096 K={K} N={N} plan variant {plan['variant']} tile {plan['tile_m']}x"
              f"{plan['tile_n']} split {plan['split_k']} grid {plan['grid_x']}", file=sys.stderr, flush=True)
        del call, x


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
      * q, k and v as one grouped launch against three launches (512 and 128 rows);
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

    # q, k and v (one input) as one grouped launch against three launches, at 512 and 128 rows
    qkv = [by[n] for n in GROUPED]
    rots = [rotation(p["w"][0]) for p in qkv]
    n = min(len(r) for r in rots)
    rows_out = []
    for rows in (M_PREFILL, 128):
        xq = qkv[0]["x"][:rows]
        ys = [torch.empty((rows, p["N"]), dtype=torch.bfloat16, device=dev) for p in qkv]
        grouped = [w4.PreparedGrouped(xq, [r[c] for r in rots], ys=ys) for c in range(n)]
        sep = [[w4.PreparedLinear(xq, *r[c], y=y) for r, y in zip(rots, ys)] for c in range(n)]
        t_grp = timed(grouped)
        t_sep = timed([(lambda c=c: [f() for f in sep[c]]) for c in range(n)])
        f3 = sum(flops(rows, p["N"], p["K"]) for p in qkv)
        pl = grouped[0].plan
        rows_out.append({"M": rows, "N": [p["N"] for p in qkv], "K": qkv[0]["K"],
                         "plan": {k: pl[k] for k in ("tile_m", "tile_n", "split_k", "variant")},
                         "grouped_us": round(t_grp, 3), "three_launches_us": round(t_sep, 3),
                         "speedup": round(t_sep / t_grp, 3), "TFLOP/s": round(f3 / t_grp / 1e6, 2),
                         **roof(rows, sum(p["N"] for p in qkv), qkv[0]["K"], f3 / t_grp / 1e6)})
        del grouped, sep, ys
    out["qkv_grouped"] = rows_out
    del rots

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
                          "TFLOP/s": round(f / t / 1e6, 2), "frac_mfma": round(f / t / 1e6 / PEAK_BF16_TFLOPS, 4),
                          **roof(4096, p["N"], p["K"], f / t / 1e6)})
        del fns, rot, y, xl
    out["prefill4096"] = long_rows

    # 128-row prefill and the ragged 509-row prefill: the seven layer projections, each alone
    for rows, cfg, key in ((128, 3, "prefill128"), (509, 4, "prefill509")):
        short_rows = []
        for name in LAYER:
            p = by[name]
            xs = torch.from_numpy(synth.activations(cfg, synth.shape_index(cfg, name), rows, p["K"]).view("int16"))
            xs = xs.view(torch.bfloat16).to(dev)
            rot = rotation(p["w"][0])
            pl = w4.w4a16_plan(rows, p["N"], p["K"])
            y = torch.empty((rows, p["N"]), dtype=torch.bfloat16, device=dev)
            wsb = ws_for(torch, pl["workspace_bytes"], dev)
            t = timed([w4.PreparedLinear(xs, *w, y=y, workspace=wsb) for w in rot])
            f = flops(rows, p["N"], p["K"])
            short_rows.append({"name": name, "M": rows, "N": p["N"], "K": p["K"],
                               "tile": [pl["tile_m"], pl["tile_n"]], "split_k": pl["split_k"],
                               "avg_us": round(t, 3), "TFLOP/s": round(f / t / 1e6, 2),
                               "frac_mfma": round(f / t / 1e6 / PEAK_BF16_TFLOPS, 4),
                               **roof(rows, p["N"], p["K"], f / t / 1e6)})
            del rot, y, xs
        layer_flops = sum(flops(rows, r["N"], r["K"]) for r in short_rows)
        # the same layer launched as the step launches it: q|k|v grouped, o, the fused gate|up pair
        # (its h feeding down), down; weights rotated per call
        xa = torch.from_numpy(synth.activations(cfg, synth.shape_index(cfg, "q"), rows, by["q"]["K"]).view("int16"))
        xa = xa.view(torch.bfloat16).to(dev)
        xo = torch.from_numpy(synth.activations(cfg, synth.shape_index(cfg, "o"), rows, by["o"]["K"]).view("int16"))
        xo = xo.view(torch.bfloat16).to(dev)
        xg = torch.from_numpy(synth.activations(cfg, synth.shape_index(cfg, "gate"), rows,
                                                by["gate"]["K"]).view("int16")).view(torch.bfloat16).to(dev)
        rots = {n: rotation(by[n]["w"][0]) for n in LAYER}
        nrot = min(len(r) for r in rots.values())
        ys = [torch.empty((rows, by[n]["N"]), dtype=torch.bfloat16, device=dev) for n in GROUPED]
        yo = torch.empty((rows, by["o"]["N"]), dtype=torch.bfloat16, device=dev)
        h = torch.empty((rows, by["gate"]["N"]), dtype=torch.bfloat16, device=dev)
        yd = torch.empty((rows, by["down"]["N"]), dtype=torch.bfloat16, device=dev)
        seq = []
        for c in range(nrot):
            fns = [w4.PreparedGrouped(xa, [rots[n][c] for n in GROUPED], ys=ys),
                   w4.PreparedLinear(xo, *rots["o"][c], y=yo),
                   w4.PreparedGateUp(xg, rots["gate"][c], rots["up"][c], h=h),
                   w4.PreparedLinear(h, *rots["down"][c], y=yd)]
            seq.append(lambda fns=fns: [f() for f in fns])
        t_layer = timed(seq)
        out[key] = {"projections": short_rows,
                    "layer_TFLOP/s": round(layer_flops / sum(r["avg_us"] for r in short_rows) / 1e6, 2),
                    "layer_as_launched_us": round(t_layer, 3),
                    "layer_as_launched_TFLOP/s": round(layer_flops / t_layer / 1e6, 2),
                    "layer_as_launched": "q|k|v grouped, o, gate|up fused with SwiGLU (h feeds down), down; "
                                         "one graph of the four calls per weight copy"}
        del seq, rots, ys, yo, h, yd, xa, xo, xg

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
                           "GB/s": round(b / t / 1e3, 1), "frac_hbm": round(b / t / 1e3 / PEAK_HBM_GBPS, 4),
                           **roof(m, N, K, flops(m, N, K) / t / 1e6)})
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

#!/usr/bin/env python3
"""Throughput of block-quantized MUL_MAT on one MI355X (gfx950).

One step = one decode token of a TinyLLaMA-shaped model through libqmm:
22 decoder layers of Q4_0 weights (Wq, Wk, Wv, Wo, Wgate, Wup, Wdown: seven
GEMVs per layer, each layer with its own weights, 548 MB in all, more than
twice the 256 MB Infinity Cache) followed by the 32000 x 2048 Q8_0 LM head.
The step is captured once into a HIP graph and replayed, the way a decode
loop is driven.  `value` is the step's algorithmic bytes (packed weights +
activations + outputs) per second.

Also reported on the same JSON line:
  * prefill: the Q4_0 x bf16 GEMM 5632 x 2048 x 512 in TFLOP/s;
  * breakdown: the 512 x 512 Q8_0 GEMV, the fp16 5632 x 2048 GEMV (1 and 8
    tokens) and the Q8_0 LM head with 1, 2, 4 and 8 tokens (GB/s, rotating
    weight copies);
  * roofline: the dominant kernel (the Q4_0 FFN gate/up GEMV, 5632 x 2048)
    timed per launch with HIP events, beside the rocprofv3 average of the
    same kernel and the read ceiling of a launch of the same bytes;
  * context: the streaming-read ceiling of one launch at each decode size
    (libqmm's stream_read kernel) and the shader clock under load;
  * cpu_baseline: the CPU oracle (1 thread and all host threads, median of 3)
    on each workload, bounded samples of the large ones.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "quantized mul_mat GB/s (decode GEMV) & TFLOP/s (prefill), % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
# MI355X dense bf16 matrix cores: 256 CUs x 2.4 GHz x 4096 flop per clock per CU
BF16_PEAK_TFLOPS = 2516.6
HERE = os.path.dirname(os.path.abspath(__file__))
# HBM traffic of the dominant kernel, from hardware counters (see traffic_probe)
TRAFFIC_FILE = os.path.join(HERE, "profiles", "gemv_q4_0_gate_up_hbm_traffic.md")
# the dominant kernel's device code: its source file and the header it includes
GEMV_SOURCES = [os.path.join(HERE, "quantized_matmul_ggml_amd", "csrc", f) for f in ("gemv.hip", "wave_reduce.h")]
COPY_PROBE_BYTES = 256 << 20   # calibration copy: 256 MiB read + 256 MiB written


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip prefill/breakdown legs")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="only launch the prefill GEMM (Q4_0 5632 x 2048 x 512) 20 times, for "
                         "hardware-counter runs (rocprofv3 --pmc MfmaUtil MfmaFlopsBF16)")
    ap.add_argument("--mf-probe", action="store_true",
                    help="launch only the matrix-core decode GEMV (for counter runs) and exit")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only launch the copy calibration kernel and the dominant GEMV, for "
                         "hardware-counter runs (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


class Graph:
    """A captured sequence of library calls, replayed on the current stream."""

    def __init__(self, fn):
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()                               # warm the path outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            fn()
        torch.cuda.synchronize()

    def __call__(self):
        self.g.replay()


def timed(fn, steps, warmup):
    """ms per call of fn over exactly `steps` calls, synchronized on both sides."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall = time.perf_counter()
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall
    return t0.elapsed_time(t1) / steps, wall


def per_launch_ms(launches):
    """Average GPU duration of each launch in `launches` (callables that
    enqueue one kernel on the current stream), measured with an event pair
    around each launch.  A spin kernel holds the queue first so that the
    host enqueues everything before the GPU starts: the events then bracket
    the kernel alone, not the host's launch latency."""
    import torch
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in launches]
    torch.cuda._sleep(int(2.4e9 * 0.05))      # ~50 ms at 2.4 GHz
    for (a, b), fn in zip(evs, launches):
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    if args.traffic_probe:
        traffic_probe()
        return
    if args.mf_probe:
        mf_probe()
        return
    if args.gemm_probe:
        gemm_probe()
        return

    import torch
    sys.path.insert(0, HERE)
    import quantized_matmul_ggml_amd as Q
    from quantized_matmul_ggml_amd import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    # ------------------------------------------------------------ decode step
    log("quantizing 22 Q4_0 decoder layers and the Q8_0 LM head on the GPU")
    layers = []
    for l in range(WL.LAYERS):
        mats = {}
        for t, (name, M, K, _) in enumerate(WL.LAYER):
            w = WL.weights_device(WL.seed(3, t, l), M, K, dev)
            mats[name] = Q.quantize(w, Q.Q4_0)
            del w
        layers.append(mats)
    xs = [WL.activations_device(WL.seed(3, 7 + s), 1, k, dev) for s, k in enumerate(WL.LAYER_X_K)]
    ys = {name: torch.empty((1, M), device=dev) for name, M, _, _ in WL.LAYER}
    lm = Q.quantize(WL.weights_device(WL.seed(4, 0), WL.VOCAB, WL.HIDDEN, dev), Q.Q8_0)
    x_lm = WL.activations_device(WL.seed(4, 1), 1, WL.HIDDEN, dev)
    y_lm = torch.empty((1, WL.VOCAB), device=dev)
    torch.cuda.synchronize()

    def gemv_bytes(w, n):
        return w.M * Q.row_size(w.type, w.K) + 4 * n * w.K + 4 * n * w.M

    layer_bytes = sum(gemv_bytes(layers[0][name], 1) for name, *_ in WL.LAYER)
    step_bytes = WL.LAYERS * layer_bytes + gemv_bytes(lm, 1)

    # Three ways to run the same 155 products:
    #  * per_matrix: one qmm_gemv launch per weight matrix (155 launches);
    #  * dependent: the launches a real decoder layer allows, since each group
    #    needs the previous group's output: [Wq Wk Wv] share x and go in one
    #    batch, then Wo, then [Wgate Wup] in one batch, then Wdown (89 launches);
    #  * grouped: the layer as the workload defines it, every projection with
    #    its own independent input: the six K = 2048 projections in one batch,
    #    Wdown in another (45 launches).
    def step_per_matrix():
        for L in layers:
            for name, _, _, slot in WL.LAYER:
                Q.gemv(L[name], xs[slot], out=ys[name])
        Q.gemv(lm, x_lm, out=y_lm)

    def dependent(xs, ys, x_lm, y_lm):
        def step():
            for L in layers:
                Q.gemv_batch([(L[n], xs[0], ys[n]) for n in ("wq", "wk", "wv")])
                Q.gemv(L["wo"], xs[1], out=ys["wo"])
                Q.gemv_batch([(L[n], xs[2], ys[n]) for n in ("wgate", "wup")])
                Q.gemv(L["wdown"], xs[3], out=ys["wdown"])
            Q.gemv(lm, x_lm, out=y_lm)
        return step

    step_dependent = dependent(xs, ys, x_lm, y_lm)

    # the dependent schedule for 8 sequences decoded together: 8 tokens per
    # launch, every launch on the matrix-core kernels
    NB = 8
    xs8 = [WL.activations_device(WL.seed(3, 20 + s), NB, k, dev) for s, k in enumerate(WL.LAYER_X_K)]
    ys8 = {name: torch.empty((NB, M), device=dev) for name, M, _, _ in WL.LAYER}
    x_lm8 = WL.activations_device(WL.seed(4, 2), NB, WL.HIDDEN, dev)
    y_lm8 = torch.empty((NB, WL.VOCAB), device=dev)
    step_dependent_8 = dependent(xs8, ys8, x_lm8, y_lm8)
    step_bytes_8 = (WL.LAYERS * sum(gemv_bytes(layers[0][name], NB) for name, *_ in WL.LAYER)
                    + gemv_bytes(lm, NB))

    def step_grouped():
        for L in layers:
            Q.gemv_batch([(L[name], xs[slot], ys[name]) for name, _, _, slot in WL.LAYER[:6]])
            Q.gemv(L["wdown"], xs[3], out=ys["wdown"])
        Q.gemv(lm, x_lm, out=y_lm)

    # dependent, with the gate/up pair fused with its SwiGLU epilogue (one
    # 5632-vector written instead of two)
    def fused(xs, ys, h_ffn, x_lm, y_lm):
        def step():
            for L in layers:
                Q.gemv_batch([(L[n], xs[0], ys[n]) for n in ("wq", "wk", "wv")])
                Q.gemv(L["wo"], xs[1], out=ys["wo"])
                Q.gemv_swiglu(L["wgate"], L["wup"], xs[2], out=h_ffn)
                Q.gemv(L["wdown"], xs[3], out=ys["wdown"])
            Q.gemv(lm, x_lm, out=y_lm)
        return step

    h_ffn = torch.empty((1, WL.FFN), device=dev)
    step_fused = fused(xs, ys, h_ffn, x_lm, y_lm)
    step_fused_8 = fused(xs8, ys8, torch.empty((NB, WL.FFN), device=dev), x_lm8, y_lm8)
    fused_bytes = step_bytes - WL.LAYERS * (4 * WL.HIDDEN + 4 * WL.FFN)
    fused_bytes_8 = step_bytes_8 - WL.LAYERS * NB * (4 * WL.HIDDEN + 4 * WL.FFN)

    variants = {}
    for vname, fn, launches, nbytes, ntok in (
            ("per_matrix", step_per_matrix, 7 * WL.LAYERS + 1, step_bytes, 1),
            ("dependent", step_dependent, 4 * WL.LAYERS + 1, step_bytes, 1),
            ("grouped", step_grouped, 2 * WL.LAYERS + 1, step_bytes, 1),
            ("dependent_swiglu_fused", step_fused, 4 * WL.LAYERS + 1, fused_bytes, 1),
            ("dependent_8_tokens", step_dependent_8, 4 * WL.LAYERS + 1, step_bytes_8, NB),
            ("dependent_swiglu_fused_8_tokens", step_fused_8, 4 * WL.LAYERS + 1, fused_bytes_8, NB)):
        log(f"decode step [{vname}]: capturing {launches} launches into a HIP graph")
        graph = Graph(fn)
        ms_v, wall_v = timed(graph, args.steps, args.warmup)
        variants[vname] = {"ms": ms_v, "wall": wall_v, "launches": launches, "tokens": ntok,
                           "gbs": nbytes / (ms_v * 1e-3) / 1e9}
        log(f"decode step [{vname}] {ms_v * 1e3:.1f} us  {variants[vname]['gbs']:.0f} GB/s  "
            f"{ntok * 1e3 / ms_v:.0f} tokens/s")
    head = "dependent"
    ms, wall = variants[head]["ms"], variants[head]["wall"]
    value = variants[head]["gbs"]

    # dominant kernel of the step: the batched gate/up GEMV (2 x 5632 x 2048,
    # 52 % of a layer's bytes).  Its average launch duration: HIP events on
    # the launch stream around replays of a graph of the 22 layers' launches
    # back to back (each launch reads weights no other launch has touched
    # since the previous replay), divided by the launches.
    gate_graph = Graph(lambda: [Q.gemv_batch([(L[n], xs[2], ys[n]) for n in ("wgate", "wup")])
                                for L in layers])
    g_ms, _ = timed(gate_graph, args.steps, args.warmup)
    kern_ms = g_ms / len(layers)
    kern_bytes = gemv_bytes(layers[0]["wgate"], 1) + gemv_bytes(layers[0]["wup"], 1)
    achieved = kern_bytes / (kern_ms * 1e-3) / 1e9
    log(f"gate/up batched GEMV {kern_ms * 1e3:.2f} us/launch  {achieved:.0f} GB/s")

    # the same pair fused with its SwiGLU epilogue, timed the same way
    sw_graph = Graph(lambda: [Q.gemv_swiglu(L["wgate"], L["wup"], xs[2], out=h_ffn) for L in layers])
    s_ms, _ = timed(sw_graph, args.steps, args.warmup)
    sw_ms = s_ms / len(layers)
    sw_bytes = kern_bytes - 4 * WL.HIDDEN - 4 * WL.FFN
    sw_gbs = sw_bytes / (sw_ms * 1e-3) / 1e9
    log(f"gate/up SwiGLU fused GEMV {sw_ms * 1e3:.2f} us/launch  {sw_gbs:.0f} GB/s")

    # context: the read ceiling of one launch of the same bytes, the decode
    # step's ceiling given its launches (each launch at the read ceiling of
    # its bytes), and the shader clock under load
    ceiling = ReadCeiling(Q, dev, args)
    layer_launch_bytes = [
        sum(gemv_bytes(layers[0][n], 1) for n in ("wq", "wk", "wv")),
        gemv_bytes(layers[0]["wo"], 1),
        kern_bytes,
        gemv_bytes(layers[0]["wdown"], 1)]
    step_ceiling_us = (WL.LAYERS * sum(ceiling(b)["us"] for b in layer_launch_bytes)
                       + ceiling(gemv_bytes(lm, 1))["us"])
    asym = ceiling(1 << 30)
    clocks = clock_leg(Q)
    inner = block_gemm_probe_leg(Q)
    rec = stored_kernel_record()

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "tinyllama_decode_token: 22 x Q4_0 layer (2048/256/256/2048/5632/5632 x 2048, "
                        "2048 x 5632) + Q8_0 LM head 32000 x 2048, batch 1",
            "layers": WL.LAYERS, "bytes_per_step": step_bytes,
            "launches_per_step": variants[head]["launches"],
            "driver": "hip graph replay; [Wq Wk Wv] and [Wgate Wup] as one batched launch each",
            "decode_tokens_per_s": round(1e3 / ms, 1),
            "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
            "step_read_ceiling": {
                "what": "the step's 89 launches each at the read ceiling of its bytes",
                "us": round(step_ceiling_us, 1),
                "gbs": round(step_bytes / (step_ceiling_us * 1e-6) / 1e9, 1),
                "frac_of_it": round(step_ceiling_us / (ms * 1e3), 4)},
            "read_ceiling_1gib_gbs": asym["gbs"],
            "sclk_mhz_under_load": clocks,
            "block_gemm_inner_loop": inner,
            "wall_s_timed_region": round(wall, 4),
            "variants": {k: {"us": round(v["ms"] * 1e3, 1), "gbs": round(v["gbs"], 1),
                             "launches": v["launches"], "tokens_per_launch": v["tokens"],
                             "tokens_per_s": round(v["tokens"] * 1e3 / v["ms"], 1)}
                         for k, v in variants.items()},
            "swiglu_fused_gate_up": ceiling.attach({"kernel": "Q4_0 gate/up 2 x 5632 x 2048 + SwiGLU, batch 1",
                                     "avg_launch_us": round(sw_ms * 1e3, 3), "bytes_per_launch": sw_bytes,
                                     "gbs": round(sw_gbs, 1),
                                     "frac_of_hbm_peak": round(sw_gbs / HBM_PEAK_GBS, 4)}, sw_bytes, sw_gbs),
        },
        "roofline": ceiling.attach({
            "kernel": "Q4_0 batched GEMV [Wgate, Wup] 2 x 5632 x 2048, batch 1",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(),
            "avg_launch_us": round(kern_ms * 1e3, 3), "bytes_per_launch": kern_bytes,
            "timing": "HIP events around graph replays of the 22 layers' launches, divided by the launches",
            "rocprof_avg_us": rec and rec["avg_us"],
            "frac_rocprof": rec and round(kern_bytes / (rec["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        }, kern_bytes, achieved),
    }

    if not args.no_extras:
        result["prefill"] = prefill_leg(Q, WL, dev, args)
        result["breakdown"] = breakdown_leg(Q, WL, dev, args, gemv_bytes, ceiling)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_leg(WL)

    print(json.dumps(result), flush=True)


def gemv_source_hash():
    import hashlib
    h = hashlib.sha256()
    for path in GEMV_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch of the dominant kernel as the hardware counters
    measured them (FETCH_SIZE + WRITE_SIZE, each scaled by what the same
    counter reads for a copy of known size), or None when no measurement is
    stored or the GEMV source has changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = [l for l in f if l.startswith("traffic-record: ")]
    except OSError:
        return None
    if not lines:
        return None
    rec = json.loads(lines[-1][len("traffic-record: "):])
    if rec.get("gemv_source_sha256") != gemv_source_hash():
        log("stored HBM traffic is stale (GEMV source changed): reporting null")
        return None
    return rec["traffic_bytes_per_launch"]


KERNEL_STATS_FILE = os.path.join(HERE, "profiles", "gemv_q4_0_decode_step_kernel_stats.md")


def stored_kernel_record():
    """The rocprofv3 average duration of the dominant kernel (the gate/up
    batch launch) from the committed kernel trace, or None when there is
    none or the GEMV source changed since it was taken."""
    try:
        with open(KERNEL_STATS_FILE) as f:
            lines = [l for l in f if l.startswith("kernel-record: ")]
    except OSError:
        return None
    if not lines:
        return None
    rec = json.loads(lines[-1][len("kernel-record: "):])
    if rec.get("gemv_source_sha256") != gemv_source_hash():
        log("stored kernel trace is stale (GEMV source changed): rocprof figure null")
        return None
    return rec


def traffic_probe():
    """Launches for the hardware-counter runs: three copies of COPY_PROBE_BYTES
    (a plain device-to-device copy, the counters' calibration), then the
    dominant kernel, the batched Q4_0 [Wgate, Wup] GEMV, over 22 layers' weights
    twice (each launch reads weights that are not in L2)."""
    import torch
    sys.path.insert(0, HERE)
    import quantized_matmul_ggml_amd as Q
    from quantized_matmul_ggml_amd import workloads as WL
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    src = torch.ones(COPY_PROBE_BYTES // 4, device=dev)
    dst = torch.empty_like(src)
    gate_up = [(n, M, K) for t, (n, M, K, _) in enumerate(WL.LAYER) if n in ("wgate", "wup")]
    layers = []
    for l in range(WL.LAYERS):
        layers.append([Q.quantize(WL.weights_device(WL.seed(3, t, l), M, K, dev), Q.Q4_0)
                       for t, (n, M, K, _) in enumerate(WL.LAYER) if n in ("wgate", "wup")])
    x = WL.activations_device(WL.seed(3, 9), 1, WL.HIDDEN, dev)
    ys = [torch.empty((1, M), device=dev) for _, M, _ in gate_up]
    torch.cuda.synchronize()
    log(f"traffic probe: gemv source sha256 {gemv_source_hash()}")
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(2):
        for L in layers:
            Q.gemv_batch([(w, x, y) for w, y in zip(L, ys)])
    torch.cuda.synchronize()
    log(f"traffic probe done: 3 copies of {COPY_PROBE_BYTES} B, {2 * WL.LAYERS} gate/up launches")


def mf_probe():
    """The matrix-core decode GEMV alone, for counter runs: the Q4_0 down
    projection 2048 x 5632 at 8 tokens (one 12-wave launch per matrix) over
    22 distinct matrices, twice, then the Q8_0 LM head 32000 x 2048 at 8
    tokens over 4 copies, twice."""
    import torch
    sys.path.insert(0, HERE)
    import quantized_matmul_ggml_amd as Q
    from quantized_matmul_ggml_amd import workloads as WL
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wd = [Q.quantize(WL.weights_device(WL.seed(3, 6, l), WL.HIDDEN, WL.FFN, dev), Q.Q4_0) for l in range(WL.LAYERS)]
    lm = [Q.quantize(WL.weights_device(WL.seed(4, 0, r), WL.VOCAB, WL.HIDDEN, dev), Q.Q8_0) for r in range(4)]
    xd = WL.activations_device(WL.seed(3, 10), 8, WL.FFN, dev)
    xl = WL.activations_device(WL.seed(4, 1), 8, WL.HIDDEN, dev)
    yd = torch.empty((8, WL.HIDDEN), device=dev)
    yl = torch.empty((8, WL.VOCAB), device=dev)
    torch.cuda.synchronize()
    for _ in range(2):
        for w in wd:
            Q.gemv(w, xd, out=yd)
    torch.cuda.synchronize()
    for _ in range(2):
        for w in lm:
            Q.gemv(w, xl, out=yl)
    torch.cuda.synchronize()
    log(f"mf probe done: {2 * WL.LAYERS} down-projection launches, 8 LM-head launches, 8 tokens each")


def gemm_probe():
    """The prefill GEMM alone, 20 launches, for matrix-core counter runs."""
    import torch
    sys.path.insert(0, HERE)
    import quantized_matmul_ggml_amd as Q
    from quantized_matmul_ggml_amd import workloads as WL
    dev = torch.device("cuda:0")
    M, K, N = WL.FFN, WL.HIDDEN, 512
    w = Q.quantize(WL.weights_device(WL.seed(5, 0), M, K, dev), Q.Q4_0)
    x = WL.activations_device(WL.seed(5, 1), N, K, dev).to(torch.bfloat16)
    y = torch.empty((N, M), device=dev)
    for _ in range(20):
        Q.gemm(w, x, out=y)
    torch.cuda.synchronize()
    log(f"gemm probe: 20 launches of Q4_0 {M} x {K} x bf16 {N}")


class ReadCeiling:
    """Streaming-read ceiling of ONE launch of a given size: libqmm's
    stream_read kernel reading `size` bytes, rotating over distinct slices of
    a 2 GiB pool (no launch finds its bytes in a cache), graph-replayed and
    timed with HIP events per launch like the GEMVs; the fastest of a few
    grid sizes.  Sizes are measured on first request and remembered."""

    POOL = (1 << 31) + (64 << 20)

    def __init__(self, Q, dev, args):
        import torch
        self.Q, self.args = Q, args
        self.pool = torch.empty(self.POOL, dtype=torch.uint8, device=dev)
        self.pool.fill_(0x5A)
        self.sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
        self.memo = {}

    def __call__(self, size):
        n = (int(size) + 15) // 16 * 16
        if n in self.memo:
            return self.memo[n]
        copies = max(2, min(64, self.POOL // n))
        slices = [self.pool[i * n:(i + 1) * n] for i in range(copies)]
        best = None
        for wgs in (512, 1024, 2048, 4096):
            g = Graph(lambda: [self.Q.stream_read(sl, self.sink, workgroups=wgs) for sl in slices])
            ms, _ = timed(g, max(3, self.args.steps // 4), 2)
            per = ms / copies
            if best is None or per < best[0]:
                best = (per, wgs)
        r = {"bytes": n, "us": round(best[0] * 1e3, 3), "gbs": round(n / (best[0] * 1e-3) / 1e9, 1),
             "workgroups": best[1]}
        log(f"read ceiling {n} B: {r['us']:.2f} us/launch  {r['gbs']:.0f} GB/s ({best[1]} workgroups)")
        self.memo[n] = r
        return r

    def attach(self, entry, nbytes, gbs):
        """Add the same-size read ceiling and the fraction of it to entry."""
        c = self(nbytes)
        entry["read_ceiling_gbs"] = c["gbs"]
        entry["frac_of_read_ceiling"] = round(gbs / c["gbs"], 4)
        return entry


def clock_leg(Q):
    """Shader clock (MHz) under a VALU chain and under a matrix-instruction
    chain on 4 waves of every CU (libqmm's clock probe)."""
    import torch
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    cus = props.multi_processor_count
    r = {"valu_mhz": round(Q.clock_probe(workgroups=cus, iters=20000, mode=0), 1),
         "mfma_mhz": round(Q.clock_probe(workgroups=cus, iters=20000, mode=1), 1)}
    log(f"shader clock under load: VALU {r['valu_mhz']} MHz, bf16 MFMA {r['mfma_mhz']} MHz")
    return r


def block_gemm_probe_leg(Q):
    """The inner loop of a block-quantized GEMM on the matrix cores (libqmm's
    probe, one and two waves per SIMD on every CU): per round four 32 x 32
    output tiles each advance by one 32-block of K, with bf16 operands
    (scale already in the weights) or int8 operands whose int32 tiles are
    rescaled per block on the vector ALUs (by the weight scale, or by the
    weight and the activation scale).  The int8 route's cap for a prefill
    GEMM over Q8_0 activations."""
    import torch
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    out = {}
    for mode, name in ((2, "bf16"), (3, "int8_weight_scale"), (4, "int8_weight_and_activation_scale")):
        row = {}
        for wps in (1, 2):
            Q.mfma_probe(mode, workgroups=cus * wps, iters=200)
            r = Q.mfma_probe(mode, workgroups=cus * wps, iters=4000)
            # a SIMD runs wps waves' rounds by the time its slowest wave ends
            row[f"{wps}_wave_per_simd"] = {"cycles_per_round_per_wave": round(r["cycles_per_round"], 1),
                                           "simd_cycles_per_round": round(r["cycles_per_round_max"] / wps, 1)}
        row["tflops_1_wave_per_simd"] = round(Q.mfma_probe(mode, workgroups=cus, iters=4000)["tflops"], 1)
        out[name] = row
        log(f"block-GEMM inner loop {name}: {row}")
    return out


def prefill_leg(Q, WL, dev, args):
    import torch
    M, K, N = WL.FFN, WL.HIDDEN, 512
    w = Q.quantize(WL.weights_device(WL.seed(5, 0), M, K, dev), Q.Q4_0)
    x = WL.activations_device(WL.seed(5, 1), N, K, dev).to(torch.bfloat16)
    y = torch.empty((N, M), device=dev)
    reps = 10
    graph = Graph(lambda: [Q.gemm(w, x, out=y) for _ in range(reps)])
    ms, _ = timed(graph, max(2, args.steps // 2), 2)
    per = ms / reps
    flops = 2.0 * M * K * N
    tf = flops / (per * 1e-3) / 1e12
    durs = per_launch_ms([lambda: Q.gemm(w, x, out=y)] * 20)
    kern = sum(durs) / len(durs)
    log(f"prefill GEMM {per * 1e3:.1f} us  {tf:.0f} TFLOP/s (per-launch events {kern * 1e3:.1f} us)")
    # the same product with F16 weights (converted, not dequantized, to bf16)
    wf = Q.f16_weight(WL.weights_device(WL.seed(5, 0), M, K, dev).to(torch.float16))
    gf = Graph(lambda: [Q.gemm(wf, x, out=y) for _ in range(reps)])
    ms_f, _ = timed(gf, max(2, args.steps // 2), 2)
    tf_f = flops / (ms_f / reps * 1e-3) / 1e12
    log(f"prefill GEMM, F16 weights {ms_f / reps * 1e3:.1f} us  {tf_f:.0f} TFLOP/s")
    # and with 64-weight blocks
    w64 = Q.quantize(WL.weights_device(WL.seed(5, 0), M, K, dev), Q.Q4_B64)
    g64 = Graph(lambda: [Q.gemm(w64, x, out=y) for _ in range(reps)])
    ms_b, _ = timed(g64, max(2, args.steps // 2), 2)
    tf_b = flops / (ms_b / reps * 1e-3) / 1e12
    log(f"prefill GEMM, Q4_B64 weights {ms_b / reps * 1e3:.1f} us  {tf_b:.0f} TFLOP/s")
    # and with Q8_0 weights (twice the code bytes per step)
    w8 = Q.quantize(WL.weights_device(WL.seed(5, 0), M, K, dev), Q.Q8_0)
    g8 = Graph(lambda: [Q.gemm(w8, x, out=y) for _ in range(reps)])
    ms_8, _ = timed(g8, max(2, args.steps // 2), 2)
    tf_8 = flops / (ms_8 / reps * 1e-3) / 1e12
    log(f"prefill GEMM, Q8_0 weights {ms_8 / reps * 1e3:.1f} us  {tf_8:.0f} TFLOP/s")
    # the layer's other prefill shapes, which leave compute units idle at 128 x 128
    # tiles: K split over a workspace (two launches) against one launch without
    shapes = {}
    for name, Ms, Ks in (("wdown", WL.HIDDEN, WL.FFN), ("wq", WL.HIDDEN, WL.HIDDEN), ("wk", 256, WL.HIDDEN)):
        ws_w = Q.quantize(WL.weights_device(WL.seed(5, 4), Ms, Ks, dev), Q.Q4_0)
        ws_x = WL.activations_device(WL.seed(5, 5), N, Ks, dev).to(torch.bfloat16)
        ws_y = torch.empty((N, Ms), device=dev)
        nbytes = Q.gemm_workspace_size(ws_w, ws_x)
        buf = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)[:nbytes]
        row = {"workspace_bytes": nbytes}
        for mode, wsarg in (("split", buf), ("unsplit", None)):
            gs = Graph(lambda: [Q.gemm(ws_w, ws_x, out=ws_y, workspace=wsarg) for _ in range(reps)])
            ms_s, _ = timed(gs, max(2, args.steps // 2), 2)
            us = ms_s / reps * 1e3
            row[mode] = {"us": round(us, 2), "tflops": round(2.0 * Ms * Ks * N / (us * 1e-6) / 1e12, 1)}
        log(f"prefill {name} {Ms}x{Ks}x{N}: split {row['split']['us']:.1f} us, unsplit {row['unsplit']['us']:.1f} us")
        shapes[f"{name}_{Ms}x{Ks}x{N}"] = row
        del ws_w, ws_x, ws_y, buf
    # one decoder layer's seven projections at 512 tokens: one launch each
    # (K split where it pays), against [Wq Wk Wv] and [Wgate Wup] as one
    # batched launch each (Wo and Wdown alone)
    lw = {name: Q.quantize(WL.weights_device(WL.seed(5, 6 + t), Ml, Kl, dev), Q.Q4_0)
          for t, (name, Ml, Kl, _) in enumerate(WL.LAYER)}
    lx = {Kl: WL.activations_device(WL.seed(5, 20 + Kl), N, Kl, dev).to(torch.bfloat16)
          for Kl in {Kl for _, _, Kl, _ in WL.LAYER}}
    ly = {name: torch.empty((N, Ml), device=dev) for name, Ml, _, _ in WL.LAYER}
    lws = {name: torch.empty(max(1, Q.gemm_workspace_size(lw[name], lx[Kl])), dtype=torch.uint8, device=dev)
           [:Q.gemm_workspace_size(lw[name], lx[Kl])] for name, _, Kl, _ in WL.LAYER}

    def layer_separate():
        for name, _, Kl, _ in WL.LAYER:
            Q.gemm(lw[name], lx[Kl], out=ly[name], workspace=lws[name])

    def layer_batched():
        Q.gemm_batch([(lw[n], lx[WL.HIDDEN], ly[n]) for n in ("wq", "wk", "wv")])
        Q.gemm(lw["wo"], lx[WL.HIDDEN], out=ly["wo"], workspace=lws["wo"])
        Q.gemm_batch([(lw[n], lx[WL.HIDDEN], ly[n]) for n in ("wgate", "wup")])
        Q.gemm(lw["wdown"], lx[WL.FFN], out=ly["wdown"], workspace=lws["wdown"])

    lh = torch.empty((N, WL.FFN), device=dev)

    def layer_fused():          # gate/up as one fused SwiGLU launch writing h only
        Q.gemm_batch([(lw[n], lx[WL.HIDDEN], ly[n]) for n in ("wq", "wk", "wv")])
        Q.gemm(lw["wo"], lx[WL.HIDDEN], out=ly["wo"], workspace=lws["wo"])
        Q.gemm_swiglu(lw["wgate"], lw["wup"], lx[WL.HIDDEN], out=lh)
        Q.gemm(lw["wdown"], lx[WL.FFN], out=ly["wdown"], workspace=lws["wdown"])

    layer_flops = sum(2.0 * Ml * Kl * N for _, Ml, Kl, _ in WL.LAYER)
    layer = {"flops": layer_flops}
    for mode, fn in (("separate", layer_separate), ("batched", layer_batched),
                     ("batched_swiglu_fused", layer_fused)):
        gl = Graph(lambda: [fn() for _ in range(reps)])
        ms_l, _ = timed(gl, max(2, args.steps // 2), 2)
        us = ms_l / reps * 1e3
        layer[mode] = {"us": round(us, 2), "tflops": round(layer_flops / (us * 1e-6) / 1e12, 1)}
        log(f"prefill layer (7 projections, 512 tokens) {mode}: {us:.1f} us  {layer[mode]['tflops']:.0f} TFLOP/s")
    del lw, lx, ly, lws, lh
    return {"workload": "Q4_0 5632 x 2048 x bf16 2048 x 512 -> f32", "us": round(per * 1e3, 2),
            "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
            "avg_launch_us": round(kern * 1e3, 2), "flops": flops,
            "f16_weights": {"us": round(ms_f / reps * 1e3, 2), "tflops": round(tf_f, 1),
                            "frac_of_bf16_peak": round(tf_f / BF16_PEAK_TFLOPS, 4)},
            "q4_b64_weights": {"us": round(ms_b / reps * 1e3, 2), "tflops": round(tf_b, 1),
                               "frac_of_bf16_peak": round(tf_b / BF16_PEAK_TFLOPS, 4)},
            "q8_0_weights": {"us": round(ms_8 / reps * 1e3, 2), "tflops": round(tf_8, 1),
                             "frac_of_bf16_peak": round(tf_8 / BF16_PEAK_TFLOPS, 4)},
            "split_k_shapes": shapes,
            "layer_512_tokens": layer}


def breakdown_leg(Q, WL, dev, args, gemv_bytes, ceiling):
    import ctypes
    import torch
    from quantized_matmul_ggml_amd import binding as B
    out = {}

    def stream_ptr():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def rotate(ws, x, y, n_per_graph):
        calls = [ws[i % len(ws)] for i in range(n_per_graph)]
        g = Graph(lambda: [Q.gemv(w, x, out=y) for w in calls])
        ms, _ = timed(g, max(2, args.steps // 2), 2)
        return ms / n_per_graph

    # 512 x 512 Q8_0, one token (latency bound: 0.28 MB per call)
    w1 = [Q.quantize(WL.weights_device(WL.seed(1, 0, r), 512, 512, dev), Q.Q8_0) for r in range(64)]
    x1 = WL.activations_device(WL.seed(1, 1), 1, 512, dev)
    y1 = torch.empty((1, 512), device=dev)
    per = rotate(w1, x1, y1, 256)
    b = gemv_bytes(w1[0], 1)
    out["q8_0_gemv_512x512_n1"] = {"us": round(per * 1e3, 3), "gbs": round(b / per / 1e6, 1), "bytes": b}
    del w1

    # Q4_0 5632 x 2048 (the FFN gate / up shape), one token: fp32 activations
    # against Q8_0 activations (the integer path), 48 copies (311 MB)
    w3 = [Q.quantize(WL.weights_device(WL.seed(3, 4, r), WL.FFN, WL.HIDDEN, dev), Q.Q4_0) for r in range(48)]
    x3 = WL.activations_device(WL.seed(3, 9), 1, WL.HIDDEN, dev)
    xq3 = Q.quantize(x3, Q.Q8_0)
    y3 = torch.empty((1, WL.FFN), device=dev)
    for name, xx, xbytes in (("q4_0_gemv_5632x2048_n1", x3, 4 * WL.HIDDEN),
                             ("q4_0_gemv_5632x2048_n1_int8_activations", xq3, xq3.data.numel())):
        per = rotate(w3, xx, y3, 96)
        b = WL.FFN * Q.row_size(Q.Q4_0, WL.HIDDEN) + xbytes + 4 * WL.FFN
        out[name] = {"us": round(per * 1e3, 3), "gbs": round(b / per / 1e6, 1), "bytes": b,
                     "frac_of_hbm_peak": round(b / per / 1e6 / HBM_PEAK_GBS, 4)}
    del w3

    # the same shape with 64-weight blocks (one fp16 scale per 64 weights)
    w5 = [Q.quantize(WL.weights_device(WL.seed(3, 4, r), WL.FFN, WL.HIDDEN, dev), Q.Q4_B64) for r in range(48)]
    per = rotate(w5, x3, y3, 96)
    b = WL.FFN * Q.row_size(Q.Q4_B64, WL.HIDDEN) + 4 * WL.HIDDEN + 4 * WL.FFN
    out["q4_b64_gemv_5632x2048_n1"] = {"us": round(per * 1e3, 3), "gbs": round(b / per / 1e6, 1), "bytes": b,
                                       "frac_of_hbm_peak": round(b / per / 1e6 / HBM_PEAK_GBS, 4)}
    del w5

    # Q4_0 2048 x 5632 (the FFN down projection) at 4 and 8 tokens: rows of
    # 176 blocks in one matrix-core launch; 48 copies (311 MB)
    w6 = [Q.quantize(WL.weights_device(WL.seed(3, 6, r), WL.HIDDEN, WL.FFN, dev), Q.Q4_0) for r in range(48)]
    for n in (4, 8):
        x6 = WL.activations_device(WL.seed(3, 10), n, WL.FFN, dev)
        y6 = torch.empty((n, WL.HIDDEN), device=dev)
        per = rotate(w6, x6, y6, 96)
        b = gemv_bytes(w6[0], n)
        out[f"q4_0_wdown_2048x5632_n{n}"] = {"us": round(per * 1e3, 3), "gbs": round(b / per / 1e6, 1), "bytes": b,
                                             "frac_of_hbm_peak": round(b / per / 1e6 / HBM_PEAK_GBS, 4)}
    del w6

    # fp16 5632 x 2048, one token: 48 copies (1.1 GB) so HBM is read
    w2 = []
    for r in range(48):
        h = WL.weights_device(WL.seed(2, 0, r), WL.FFN, WL.HIDDEN, dev).to(torch.float16)
        w2.append(Q.f16_weight(h))
    # (and with 8 tokens, on the matrix cores)
    for n in (1, 8):
        x2 = WL.activations_device(WL.seed(2, 1), n, WL.HIDDEN, dev)
        y2 = torch.empty((n, WL.FFN), device=dev)
        per = rotate(w2, x2, y2, 96)
        b = gemv_bytes(w2[0], n)
        out[f"f16_gemv_5632x2048_n{n}"] = {"us": round(per * 1e3, 3), "gbs": round(b / per / 1e6, 1), "bytes": b,
                                           "frac_of_hbm_peak": round(b / per / 1e6 / HBM_PEAK_GBS, 4)}
    del w2

    # Q8_0 LM head, 16 copies (1.1 GB), N = 1, 2, 4, 8
    w4 = [Q.quantize(WL.weights_device(WL.seed(4, 0, r), WL.VOCAB, WL.HIDDEN, dev), Q.Q8_0)
          for r in range(16)]
    for n in (1, 2, 4, 8):
        x4 = WL.activations_device(WL.seed(4, 1), n, WL.HIDDEN, dev)
        y4 = torch.empty((n, WL.VOCAB), device=dev)
        per = rotate(w4, x4, y4, 32)
        b = gemv_bytes(w4[0], n)
        out[f"q8_0_lm_head_32000x2048_n{n}"] = {
            "us": round(per * 1e3, 3), "gbs": round(b / per / 1e6, 1), "bytes": b,
            "frac_of_hbm_peak": round(b / per / 1e6 / HBM_PEAK_GBS, 4)}
    # the integer-activation path: activations quantized to Q8_0 blocks, block
    # dot products in int8 (bytes: weights + Q8_0 activations + fp32 outputs)
    for n in (1, 8):
        xq4 = Q.quantize(WL.activations_device(WL.seed(4, 1), n, WL.HIDDEN, dev), Q.Q8_0)
        y4 = torch.empty((n, WL.VOCAB), device=dev)
        per = rotate(w4, xq4, y4, 32)
        b = w4[0].M * Q.row_size(Q.Q8_0, WL.HIDDEN) + xq4.data.numel() + 4 * n * WL.VOCAB
        out[f"q8_0_lm_head_32000x2048_n{n}_int8_activations"] = {
            "us": round(per * 1e3, 3), "gbs": round(b / per / 1e6, 1), "bytes": b,
            "frac_of_hbm_peak": round(b / per / 1e6 / HBM_PEAK_GBS, 4)}
    # block-record interchange of the LM head (GGUF-style records <-> rows),
    # 4 copies so the 139 MB each call moves is not cache-resident
    recs = [Q.rows_to_records(w) for w in w4[:4]]
    rows = [Q.Weight(torch.empty_like(w.data), w.type, w.K, w.M) for w in w4[:4]]
    for name, fn in (("q8_0_records_to_rows_32000x2048",
                      lambda i: B.lib().qmm_records_to_rows(ctypes.c_void_p(recs[i].data_ptr()),
                                                            ctypes.byref(descs[i]), stream_ptr())),
                     ("q8_0_rows_to_records_32000x2048",
                      lambda i: B.lib().qmm_rows_to_records(ctypes.byref(srcs[i]),
                                                            ctypes.c_void_p(recs[i].data_ptr()), stream_ptr()))):
        descs = [r.desc() for r in rows]
        srcs = [w.desc() for w in w4[:4]]
        g = Graph(lambda: [fn(i) for i in range(4)])
        ms, _ = timed(g, max(2, args.steps // 2), 2)
        per = ms / 4
        b = 2 * recs[0].numel()                 # record bytes read + row bytes written (equal)
        out[name] = {"us": round(per * 1e3, 3), "gbs": round(b / per / 1e6, 1), "bytes": b,
                     "frac_of_hbm_peak": round(b / per / 1e6 / HBM_PEAK_GBS, 4)}
    assert torch.equal(rows[0].data, w4[0].data), "records -> rows must restore the packed rows"
    del w4, recs, rows
    for k, v in out.items():
        if "records" not in k:                  # a copy, not a read: no read ceiling
            ceiling.attach(v, v["bytes"], v["gbs"])
        log(f"{k}: {v}")
    return out


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_leg(WL):
    """The oracle (plain C, binary64; oracle/oracle_timing.c splits the rows
    over POSIX threads) timed on the host: each workload once on 1 thread
    and once on the host's threads (capped at 16, the CPU share of one GPU
    here), median of 3 runs each.  The large workloads are bounded samples of
    their rows (all of K and of the tokens).  `value` is the decode layer's
    rate on the host's threads, in the step's unit (algorithmic GB/s)."""
    import numpy as np
    import oracle as orc
    hw = orc.online_cpus()
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = hw
    threads = max(1, min(16, avail))
    rs = orc.row_size

    def entry(name, parts, sample):
        """parts: [(type, packed, K, x, x_bf16)]; times the sum over parts."""
        nbytes = flops = 0
        for t, packed, K, x, bf in parts:
            M = packed.shape[0]
            N = x.shape[0]
            nbytes += M * (rs(t, K) if t != orc.F16 else 2 * K) + (2 if bf else 4) * N * K + 4 * N * M
            flops += 2 * M * K * N
        r = {"sample": sample, "bytes": nbytes, "flops": flops}
        for label, th in (("1_thread", 1), (f"{threads}_threads", threads)):
            sec = sum(orc.time_mul_mat(t, packed, K, x, threads=th, reps=3, x_bf16_bits=bf)
                      for t, packed, K, x, bf in parts)
            r[label] = {"s": round(sec, 5), "gbs": round(nbytes / sec / 1e9, 4),
                        "gflops": round(flops / sec / 1e9, 4)}
        log(f"cpu oracle {name}: 1 thread {r['1_thread']['gbs']} GB/s, {threads} threads "
            f"{r[f'{threads}_threads']['gbs']} GB/s ({sample})")
        return r

    per = {}
    w = WL.weights(WL.seed(1, 0), 512, 512)
    per["q8_0_gemv_512x512_n1"] = entry("C1", [(orc.Q8_0, orc.quantize(orc.Q8_0, w), 512,
                                               WL.activations(WL.seed(1, 1), 1, 512), False)], "whole")
    w = WL.round_f16(WL.weights(WL.seed(2, 0), WL.FFN, WL.HIDDEN))
    per["f16_gemv_5632x2048_n1"] = entry("C2", [(orc.F16, w.view(np.uint8).reshape(WL.FFN, -1), WL.HIDDEN,
                                                WL.activations(WL.seed(2, 1), 1, WL.HIDDEN), False)], "whole")
    xs = [WL.activations(WL.seed(3, 7 + s), 1, k) for s, k in enumerate(WL.LAYER_X_K)]
    layer = [(orc.Q4_0, orc.quantize(orc.Q4_0, WL.weights(WL.seed(3, t), M, K)), K, xs[slot], False)
             for t, (_, M, K, slot) in enumerate(WL.LAYER)]
    per["q4_0_decode_layer"] = entry("C3", layer, "one whole layer (7 GEMVs)")
    rows = 2048
    wl = orc.quantize(orc.Q8_0, WL.weights(WL.seed(4, 0), rows, WL.HIDDEN))
    for n in (1, 2, 4, 8):
        per[f"q8_0_lm_head_32000x2048_n{n}"] = entry(
            f"C4 N={n}", [(orc.Q8_0, wl, WL.HIDDEN, WL.activations(WL.seed(4, 1), n, WL.HIDDEN), False)],
            f"{rows} of 32000 rows")
    rows5 = 64
    w5 = orc.quantize(orc.Q4_0, WL.weights(WL.seed(5, 0), rows5, WL.HIDDEN))
    x5 = WL.round_bf16_bits(WL.activations(WL.seed(5, 1), 512, WL.HIDDEN))
    per["q4_0_prefill_gemm_5632x2048x512"] = entry("C5", [(orc.Q4_0, w5, WL.HIDDEN, x5, True)],
                                                   f"{rows5} of 5632 rows, all 512 tokens")
    head = per["q4_0_decode_layer"][f"{threads}_threads"]
    return {"value": head["gbs"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "one Q4_0 decoder layer (the decode step's unit of work: 7 GEMVs, batch 1), "
                      f"binary64 oracle, rows split over {threads} POSIX threads, median of 3",
            "nproc": hw, "affinity_cpus": avail, "cpu_model": cpu_model(), "per_config": per}


if __name__ == "__main__":
    main()

#!/usr/bin/env python
"""Benchmark: the full NVFP4 verify pass on one MI355X.

Workload: a 64-layer dense stack with, per layer, q/k/v/o [5120x5120],
gate/up [17408x5120] and down [5120x17408] in NVFP4 (13,400,801,280 bytes of
codes + scales per pass), applied to M draft-tree rows (bf16) and chained layer
to layer. One step = one pass, replayed from a HIP graph; weights and inputs are
resident in HBM before the timed region.

Prints one JSON line: value = achieved HBM GB/s of the pass at M = --m
(weight + scale bytes / pass time), plus the per-M staircase of the pass
(M = 1..32), a roofline entry for the dominant kernel (the verify GEMM) from
HIP events on its own stream, the HBM read ceiling measured by a plain
streaming kernel, and the CPU oracle timed on the host's cores over a bounded
sample of the same GEMMs.
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

H, I, LAYERS = 5120, 17408, 64
BYTES_PER_WEIGHT = 0.5625  # 4-bit code + one E4M3 byte per 16 weights
PEAK_HBM_GBS = 8000.0
METRIC = "verify-pass µs and achieved HBM GB/s vs M (1..32), full 27B layer stack"
PAGES_CONTEXT = {"hardware": "DGX Spark GB10 (other machine; whole forward pass incl. attention)",
                 "verify_pass_ms": {"8": 75.5, "16": 74.4, "24": 83.1, "32": 87.8}}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def layer_weight_bytes():
    return int((4 * H * H + 2 * I * H + H * I) * BYTES_PER_WEIGHT)


def interleave_tiles(torch, w):
    """[gate; up] (rows) -> 16-row tiles alternating gate, up."""
    n, k = w.shape
    half = n // 2
    return torch.stack([w[:half].reshape(half // 16, 16, k), w[half:].reshape(half // 16, 16, k)],
                       dim=1).reshape(n, k)


def build_stack(torch, nv, synth, ctx, layers):
    """Quantise and pack `layers` layers of synthetic N(0,1) weights on the GPU."""
    scratch = torch.empty((2 * I, H), dtype=torch.float32, device="cuda")
    packed = []
    t0 = time.time()
    for l in range(layers):
        mats = {}
        for name, parts, n, k in (("qkv", ("q", "k", "v"), 3 * H, H), ("o", ("o",), H, H),
                                  ("gate_up", ("gate", "up"), 2 * I, H), ("down", ("down",), H, I)):
            rows = n // len(parts)
            w = scratch.view(-1)[: n * k].view(n, k)
            for i, part in enumerate(parts):
                synth.weights_f32_cuda(rows, k, seed=0, stream="L%d/%s" % (l, part),
                                       out=w[i * rows:(i + 1) * rows])
            if name == "gate_up":  # the pass takes gate and up interleaved in 16-row tiles
                w = interleave_tiles(torch, w)
            codes, scales = ctx.quantize(w)
            mats[name] = ctx.pack(codes, scales, n, k)
            del codes, scales
        packed.append(mats)
        if (l + 1) % 16 == 0:
            torch.cuda.synchronize()
            log("packed %d/%d layers (%.1f s)" % (l + 1, layers, time.time() - t0))
    del scratch
    torch.cuda.synchronize()
    return packed


def time_graph(torch, graph, warmup, steps):
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


class DirectPass:
    """Enqueues the pass directly (same interface as a captured graph)."""

    def __init__(self, torch, ctx, layer_arr, h0, ws, h_out, m):
        self.args = (layer_arr, H, I, h0[:m], ws, h_out[:m])
        self.ctx = ctx
        ctx.verify_pass(*self.args)
        torch.cuda.synchronize()

    def replay(self):
        self.ctx.verify_pass(*self.args)


def capture_pass(torch, ctx, layer_arr, h0, ws, h_out, m):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ctx.verify_pass(layer_arr, H, I, h0[:m], ws, h_out[:m])  # eager warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx.verify_pass(layer_arr, H, I, h0[:m], ws, h_out[:m])
    torch.cuda.synchronize()
    return g


def gemm_event_timing(torch, ctx, packed, h0, m, passes=2):
    """Run the pass eagerly, op by op, with HIP events around every GEMM launch on
    the stream the GEMMs run on. Returns (sum of GEMM bytes, sum of GEMM ms, launches)."""
    stream = torch.cuda.current_stream()
    c_h = float((1.0 / (H ** 0.5)))
    c_i = float((1.0 / (I ** 0.5)))
    c_2 = float((1.0 / ((2 * H) ** 0.5)))
    qkv = torch.empty((m, 3 * H), dtype=torch.float32, device="cuda")
    o = torch.empty((m, H), dtype=torch.float32, device="cuda")
    gu = torch.empty((m, 2 * I), dtype=torch.float32, device="cuda")
    d = torch.empty((m, H), dtype=torch.float32, device="cuda")
    events = []
    total_bytes = 0
    for _ in range(passes):
        h = h0[:m]
        for mats in packed:
            for (a, name, n, k, out) in (("h", "qkv", 3 * H, H, qkv), ("o_in", "o", H, H, o),
                                         ("g_in", "gate_up", 2 * I, H, gu), ("d_in", "down", H, I, d)):
                if name == "o":
                    a_t = ctx.glue_scale(qkv[:, 2 * H:], c_h)
                elif name == "gate_up":
                    a_t = ctx.glue_scale(o, c_h)
                elif name == "down":
                    t = gu.view(m, I // 16, 2, 16)
                    a_t = ctx.glue_sum(t[:, :, 0].reshape(m, I), t[:, :, 1].reshape(m, I), c_2)
                else:
                    a_t = h
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                ctx.verify_gemm(a_t, mats[name], n, k, out=out)
                e1.record(stream)
                events.append((e0, e1))
                total_bytes += int(n * k * BYTES_PER_WEIGHT)
            h = ctx.glue_scale(d, c_i)
    torch.cuda.synchronize()
    total_ms = sum(e0.elapsed_time(e1) for e0, e1 in events)
    return total_bytes, total_ms, len(events)


def read_ceiling(torch, ctx, gib=4, reps=5):
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(ctx.read_probe_sink_words(), dtype=torch.int32, device="cuda")
    ctx.read_probe(buf, sink)
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        ctx.read_probe(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1))
    del buf
    t.sort()
    return (gib << 30) / (t[len(t) // 2] * 1e-3) / 1e9


def cpu_baseline(target_s=12.0, m=16):
    """The oracle (as it stands) on the host cores: decode + fp64 GEMM over a
    bounded sample of the pass's weight rows (all four projection shapes)."""
    import numpy as np

    import oracle
    import synth

    oracle.build()
    threads = oracle.thread_count()
    a_h = synth.activations_bf16(m, H, seed=0, stream="cpu/h")
    a_i = synth.activations_bf16(m, I, seed=0, stream="cpu/i")
    shapes = [("qkv", 3 * H, H, a_h), ("o", H, H, a_h), ("gate_up", 2 * I, H, a_h), ("down", H, I, a_i)]
    # calibrate on a small sample, then size the real one to about target_s seconds
    w = synth.weights_f32(256, H, seed=0, stream="cpu/cal")
    codes, scales = oracle.quantize(w)
    t0 = time.perf_counter()
    oracle.gemm(a_h, codes, scales)
    rate = 256 * H / max(time.perf_counter() - t0, 1e-6)  # weights per second
    per_shape_weights = rate * target_s / len(shapes)
    total_w, total_t = 0, 0.0
    desc = []
    for name, n, k, a in shapes:
        rows = int(max(1, min(n, per_shape_weights / k)))
        w = synth.weights_f32(n, k, seed=0, stream="cpu/" + name, rows=np.arange(rows))
        codes, scales = oracle.quantize(w)
        t0 = time.perf_counter()
        oracle.gemm(a, codes, scales, threads=threads)
        total_t += time.perf_counter() - t0
        total_w += rows * k
        desc.append("%s %dx%d" % (name, rows, k))
    gbs = total_w * BYTES_PER_WEIGHT / total_t / 1e9
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "oracle decode + fp64 GEMM at M=%d over the first rows of each projection "
                      "shape (%s), %.1f s" % (m, ", ".join(desc), total_t)}


def traffic_from_profile(gemm_src_hash):
    """HBM bytes per GEMM launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "verify_gemm_pmc_fullpass_m16.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != gemm_src_hash:
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse_sweep(s):
    out = []
    for part in s.split(","):
        if not part:
            continue
        if "-" in part:
            a, b = part.split("-")
            out.extend(range(int(a), int(b) + 1))
        else:
            out.append(int(part))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--m", type=int, default=16)
    ap.add_argument("--sweep", default="1-32", help="M values for the per-M pass staircase ('' = none)")
    ap.add_argument("--sweep-steps", type=int, default=5)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (sharding is "
              "described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import nvfp4_skinny_gemm_amd as nv
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ctx = nv.Context(0)
    layers = args.layers
    log("device: %s, %d layers" % (torch.cuda.get_device_name(0), layers))
    packed = build_stack(torch, nv, synth, ctx, layers)
    layer_arr = (nv.Layer * layers)()
    for l, mats in enumerate(packed):
        layer_arr[l] = nv.Layer(mats["qkv"].data_ptr(), mats["o"].data_ptr(),
                                mats["gate_up"].data_ptr(), mats["down"].data_ptr(), 1.0, 1.0, 1.0, 1.0)
    h0 = torch.from_numpy(synth.activations_bf16(64, H, seed=0, stream="pass/h0").view("int16")).cuda()
    h0 = h0.view(torch.bfloat16)
    ws = torch.empty(nv.pass_workspace_bytes(64, H, I, layers), dtype=torch.uint8, device="cuda")
    h_out = torch.empty((64, H), dtype=torch.bfloat16, device="cuda")
    pass_bytes = layer_weight_bytes() * layers

    # ---- headline: the pass at M = args.m --------------------------------------
    # A pass is one packing kernel plus the layers' GEMM launches (or one
    # persistent kernel per 32 layers); it is replayed from a HIP graph when the
    # runtime can capture it, else enqueued directly.
    mode = "graph"
    try:
        runner = capture_pass(torch, ctx, layer_arr, h0, ws, h_out, args.m)
    except Exception as exc:  # capture of cooperative launches unsupported
        log("graph capture unavailable (%s); timing direct launches" % type(exc).__name__)
        mode = "direct"
        runner = DirectPass(torch, ctx, layer_arr, h0, ws, h_out, args.m)
    sec = time_graph(torch, runner, args.warmup, args.steps)
    assert ctx.pass_status() == nv.OK, "persistent pass timed out"
    assert torch.isfinite(h_out[: args.m].float()).all(), "non-finite pass output"
    gbs = pass_bytes / sec / 1e9
    log("M=%d: %.1f us per pass, %.1f GB/s (%s, grid %d)" % (args.m, sec * 1e6, gbs, mode,
                                                             ctx.last_pass_grid()))
    del runner

    # ---- per-M staircase of the pass ------------------------------------------
    per_m = {}
    for m in parse_sweep(args.sweep):
        gm = (capture_pass(torch, ctx, layer_arr, h0, ws, h_out, m) if mode == "graph"
              else DirectPass(torch, ctx, layer_arr, h0, ws, h_out, m))
        s = time_graph(torch, gm, 2, args.sweep_steps)
        per_m[str(m)] = {"us": round(s * 1e6, 1), "GBps": round(pass_bytes / s / 1e9, 1),
                         "TFLOPs": round(2.0 * m * pass_bytes / BYTES_PER_WEIGHT / s / 1e12, 2)}
        del gm
    if per_m:
        log("staircase: " + " ".join("%s:%.0f" % (k, v["us"]) for k, v in per_m.items()))

    # ---- roofline of the dominant kernel (verify GEMM), HIP events -------------
    gbytes, gms, launches = gemm_event_timing(torch, ctx, packed, h0, args.m)
    achieved = gbytes / (gms * 1e-3) / 1e9
    src_hash = hashlib.sha256(open(os.path.join(ROOT, "nvfp4_skinny_gemm_amd", "csrc", "gemm.hip"),
                                   "rb").read()).hexdigest()
    traffic = traffic_from_profile(src_hash)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": "k_gemm_mfma (verify GEMM), M=%d" % args.m,
                "avg_launch_us": round(gms * 1e3 / launches, 2),
                "algorithmic_bytes_per_launch": round(gbytes / launches)}
    ceiling = read_ceiling(torch, ctx)
    log("GEMM kernels alone: %.1f GB/s (%.1f%% of peak); read ceiling %.1f GB/s" % (
        achieved, 100 * achieved / PEAK_HBM_GBS, ceiling))

    result = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "full verify pass: %d layers x (q,k,v,o 5120x5120; gate,up 17408x5120; "
                               "down 5120x17408) NVFP4, M=%d bf16 rows" % (layers, args.m),
                   "m": args.m, "layers": layers, "weight_bytes_per_pass": pass_bytes,
                   "launch": "%s, %s" % ("4 GEMM launches per layer" if ctx.get_pass_mode() == nv.PASS_CHAIN
                                         else "persistent kernel per 32 layers", mode),
                   "grid": ctx.last_pass_grid()},
        "pass_us": round(sec * 1e6, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "per_m": per_m,
        "roofline": roofline,
        "read_ceiling_GBps": round(ceiling, 1),
        "pages_context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(m=args.m)
    print(json.dumps(result), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()

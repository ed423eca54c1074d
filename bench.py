#!/usr/bin/env python
"""Benchmark: the full NVFP4 verify pass on one MI355X.

Workload: a 64-layer dense stack with, per layer, q/k/v/o [5120x5120],
gate/up [17408x5120] and down [5120x17408] in NVFP4 (13,400,801,280 bytes of
codes + scales per pass), applied to M draft-tree rows (bf16) and chained layer
to layer. One step = one pass, replayed from a HIP graph; weights and inputs are
resident in HBM before the timed region.

Prints one JSON line: value = achieved HBM GB/s of the pass at M = --m
(weight + scale bytes / pass time) in the chosen schedule (the other schedule's
time beside it), the per-M staircase of the pass (M = 1..32), a roofline entry
for the dominant kernel (the verify GEMM, timed alone with HIP events on its
own stream), the HBM read ceiling measured by a plain streaming kernel, the
per-shape GEMM staircase M = 1..64 with its step positions (LM head and the
layer shapes), and the CPU oracle timed on the host's cores over a bounded
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


def gemm_event_timing(torch, ctx, packed, m, reps=2):
    """The verify GEMM kernel alone, as the pass launches it at M = m: activations
    packed once per shape (pack_activations), then one verify_gemm_pa launch per
    layer and projection, timed with HIP events on the stream the kernel runs on
    (one pair around each shape's 64 back-to-back launches). Returns (algorithmic
    weight+scale bytes, summed ms, launches, per-shape {us, GBps, plan})."""
    import synth

    stream = torch.cuda.current_stream()  # the stream verify_gemm_pa launches on
    shapes = (("qkv", 3 * H, H), ("o", H, H), ("gate_up", 2 * I, H), ("down", H, I))
    acts = {}
    for name, n, k in shapes:
        a = torch.from_numpy(synth.activations_bf16(64, k, seed=0, stream="roofline/%d" % k)[:m].view("int16"))
        acts[k] = ctx.pack_activations(a.cuda().view(torch.bfloat16))
    outs = {name: torch.empty((m, n), dtype=torch.float32, device="cuda") for name, n, k in shapes}
    for name, n, k in shapes:  # warm-up
        ctx.verify_gemm_pa(acts[k], m, k, packed[0][name], n, out=outs[name])
    torch.cuda.synchronize()
    # One event pair around each shape's back-to-back launches (all layers):
    # per-launch pairs would add the dispatch latency of every launch.
    events = {name: [] for name, _, _ in shapes}
    for _ in range(reps):
        for name, n, k in shapes:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for mats in packed:
                ctx.verify_gemm_pa(acts[k], m, k, mats[name], n, out=outs[name])
            e1.record(stream)
            events[name].append((e0, e1, len(packed)))
    torch.cuda.synchronize()
    total_bytes, total_ms, launches, per_shape = 0, 0.0, 0, {}
    for name, n, k in shapes:
        ms = sum(e0.elapsed_time(e1) for e0, e1, _ in events[name])
        cnt = sum(c for _, _, c in events[name])
        b = int(n * k * BYTES_PER_WEIGHT)
        per_shape[name] = {"us": round(1e3 * ms / cnt, 2), "GBps": round(b * cnt / (ms * 1e-3) / 1e9, 1),
                           "plan": ctx.describe_plan(n, k, m)}
        total_bytes += b * cnt
        total_ms += ms
        launches += cnt
    return total_bytes, total_ms, launches, per_shape


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


def cpu_baseline(target_s=12.0, m=16, rows=512):
    """The oracle (as it stands) on the host's cores: decode + fp64 GEMM of an
    M = m activation block against the first `rows` weight rows of each of the
    pass's four projection shapes, repeated until about target_s seconds of
    GEMM time (input generation and quantisation are not timed)."""
    import numpy as np

    import oracle
    import synth

    oracle.build()
    threads = oracle.thread_count()
    a_h = synth.activations_bf16(m, H, seed=0, stream="cpu/h")
    a_i = synth.activations_bf16(m, I, seed=0, stream="cpu/i")
    work = []
    for name, n, k, a in (("qkv", 3 * H, H, a_h), ("o", H, H, a_h), ("gate_up", 2 * I, H, a_h),
                          ("down", H, I, a_i)):
        w = synth.weights_f32(n, k, seed=0, stream="cpu/" + name, rows=np.arange(rows))
        codes, scales = oracle.quantize(w)
        work.append((a, codes, scales, rows * k))
    total_w, total_t, reps = 0, 0.0, 0
    while total_t < target_s:
        for a, codes, scales, nw in work:
            t0 = time.perf_counter()
            oracle.gemm(a, codes, scales, threads=threads)
            total_t += time.perf_counter() - t0
            total_w += nw
        reps += 1
    gbs = total_w * BYTES_PER_WEIGHT / total_t / 1e9
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "oracle decode + fp64 GEMM at M=%d of the first %d weight rows of each projection "
                      "(q|k|v 15360x5120, o 5120x5120, gate|up 34816x5120, down 5120x17408), %d "
                      "repetitions, %.1f s; weight+scale bytes per second" % (m, rows, reps, total_t)}


def kernel_source_hash():
    """sha256 over the verify GEMM's device sources (the traffic figure in
    profiles/ is valid only for the kernel it was taken on)."""
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm_device.h"):
        h.update(open(os.path.join(ROOT, "nvfp4_skinny_gemm_amd", "csrc", f), "rb").read())
    return h.hexdigest()


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


def find_steps(us, m0=1):
    """Staircase steps: M where the time exceeds 1.03x the median of the plateau
    of preceding M values by more than 3 MADs of that plateau's noise."""
    import numpy as np

    steps, start = [], 0
    for i in range(1, len(us)):
        plateau = np.asarray(us[start:i])
        med = float(np.median(plateau))
        mad = float(np.median(np.abs(plateau - med))) if len(plateau) > 1 else 0.0
        if us[i] > 1.03 * med and us[i] - med > 3 * mad:
            steps.append(m0 + i)
            start = i
    return steps


def staircase_report(ctx, m_hi=64, reps=7):
    """A10: microseconds per M (1..m_hi) of the verify GEMM on the LM head and
    the layer shapes (rotating >= 2 GiB of weight copies), with step positions."""
    shapes = (("head", 151936, 5120), ("qkvo", 5120, 5120), ("gate_up", 17408, 5120), ("down", 5120, 17408))
    out = {}
    for name, n, k in shapes:
        us = [round(float(x), 2) for x in ctx.staircase(n, k, 1, m_hi, warmup=2, reps=reps, rotate_bytes=2 << 30)]
        out[name] = {"shape": [n, k], "us": us, "steps": find_steps(us),
                     "GBps_m16": round(n * k * BYTES_PER_WEIGHT / (us[15] * 1e-6) / 1e9, 1)}
        log("staircase %s [%dx%d]: M1 %.1f us, M16 %.1f, M32 %.1f, M64 %.1f; steps at %s" % (
            name, n, k, us[0], us[15], us[31], us[63], out[name]["steps"]))
    return out


def fp8_head_report(torch, nv, synth, ctx, ms=(1, 8, 16, 24, 32), warmup=3, reps=20):
    """The FP8 output head (151936 x 5120 E4M3 codes + fp32 row scales, the
    step after the last layer): microseconds per launch and weight GB/s at the
    tree sizes. Random finite codes; the 778 MB of weights exceed every cache,
    so back-to-back launches stream them from HBM."""
    n, k = 151936, 5120
    packed = torch.from_numpy(nv.fp8_pack_host(synth.fp8_codes(n, k, seed=1),
                                               synth.fp8_row_scales(n, seed=1))).cuda()
    wbytes = n * k + n * 4
    out = {"shape": [n, k], "weight_bytes": wbytes, "us": {}, "GBps": {}}
    for m in ms:
        a = torch.from_numpy(synth.activations_bf16(m, k, seed=m, stream="headbench").view("int16")).cuda().view(torch.bfloat16)
        c = torch.empty((m, n), dtype=torch.float32, device="cuda")
        for _ in range(warmup):
            ctx.fp8_head_gemm(a, packed, n, k, out=c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            ctx.fp8_head_gemm(a, packed, n, k, out=c)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out["us"][str(m)] = round(us, 2)
        out["GBps"][str(m)] = round(wbytes / (us * 1e-6) / 1e9, 1)
    log("fp8 head [%dx%d]: %s us; %s GB/s" % (n, k, out["us"], out["GBps"]))
    del packed
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--m", type=int, default=16)
    ap.add_argument("--mode", choices=("chain", "persistent"), default="chain",
                    help="pass schedule of the headline number (the other is reported beside it)")
    ap.add_argument("--sweep", default="1-32", help="M values for the per-M pass staircase ('' = none)")
    ap.add_argument("--sweep-steps", type=int, default=5)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-staircase", action="store_true")
    ap.add_argument("--no-head", action="store_true", help="skip the FP8 output head timing")
    ap.add_argument("--head-only", action="store_true", help="time only the FP8 output head")
    ap.add_argument("--gemm-only", action="store_true",
                    help="only the verify-GEMM roofline leg and a 256 MiB copy (for hardware-counter runs)")
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
    if args.head_only:
        print(json.dumps({"fp8_head": fp8_head_report(torch, nv, synth, ctx)}), flush=True)
        ctx.close()
        return
    packed = build_stack(torch, nv, synth, ctx, layers)

    if args.gemm_only:
        gbytes, gms, launches, per_shape = gemm_event_timing(torch, ctx, packed, args.m)
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        src.fill_(3)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        ctx.copy_probe(src, dst)
        torch.cuda.synchronize()
        print(json.dumps({"gemm_launches": launches, "algorithmic_bytes_per_launch": gbytes / launches,
                          "avg_launch_us": gms * 1e3 / launches, "copy_probe_bytes": 256 << 20,
                          "per_shape": per_shape}), flush=True)
        ctx.close()
        return

    layer_arr = (nv.Layer * layers)()
    for l, mats in enumerate(packed):
        layer_arr[l] = nv.Layer(mats["qkv"].data_ptr(), mats["o"].data_ptr(),
                                mats["gate_up"].data_ptr(), mats["down"].data_ptr(), 1.0, 1.0, 1.0, 1.0)
    h0 = torch.from_numpy(synth.activations_bf16(64, H, seed=0, stream="pass/h0").view("int16")).cuda()
    h0 = h0.view(torch.bfloat16)
    ws = torch.empty(nv.pass_workspace_bytes(64, H, I, layers), dtype=torch.uint8, device="cuda")
    h_out = torch.empty((64, H), dtype=torch.bfloat16, device="cuda")
    pass_bytes = layer_weight_bytes() * layers
    modes = {"chain": nv.PASS_CHAIN, "persistent": nv.PASS_PERSISTENT}
    other = "persistent" if args.mode == "chain" else "chain"

    def timed_pass(m, warmup, steps):
        launch = "graph"
        try:
            runner = capture_pass(torch, ctx, layer_arr, h0, ws, h_out, m)
        except Exception as exc:  # the runtime cannot capture this schedule
            log("graph capture unavailable (%s); timing direct launches" % type(exc).__name__)
            launch = "direct"
            runner = DirectPass(torch, ctx, layer_arr, h0, ws, h_out, m)
        sec = time_graph(torch, runner, warmup, steps)
        assert ctx.pass_status() == nv.OK, "persistent pass timed out"
        del runner
        return sec, launch

    # ---- headline: the pass at M = args.m --------------------------------------
    # One step is one pass over all layers: a packing kernel plus the layers'
    # GEMMs (four launches per layer, or one persistent kernel per 32 layers),
    # replayed from a HIP graph; weights and input are resident in HBM.
    ctx.set_pass_mode(modes[other])
    sec_other, _ = timed_pass(args.m, 2, max(3, args.steps // 4))
    ctx.set_pass_mode(modes[args.mode])
    sec, launch = timed_pass(args.m, args.warmup, args.steps)
    assert torch.isfinite(h_out[: args.m].float()).all(), "non-finite pass output"
    gbs = pass_bytes / sec / 1e9
    log("M=%d: %.1f us per pass, %.1f GB/s (%s, %s); %s schedule %.1f us" % (
        args.m, sec * 1e6, gbs, args.mode, launch, other, sec_other * 1e6))

    # ---- per-M staircase of the pass ------------------------------------------
    per_m = {}
    for m in parse_sweep(args.sweep):
        s_m, _ = timed_pass(m, 2, args.sweep_steps)
        per_m[str(m)] = {"us": round(s_m * 1e6, 1), "GBps": round(pass_bytes / s_m / 1e9, 1),
                         "TFLOPs": round(2.0 * m * pass_bytes / BYTES_PER_WEIGHT / s_m / 1e12, 2)}
    if per_m:
        log("pass staircase: " + " ".join("%s:%.0f" % (k, v["us"]) for k, v in per_m.items()))

    # ---- roofline of the dominant kernel (the verify GEMM), HIP events ----------
    gbytes, gms, launches, per_shape = gemm_event_timing(torch, ctx, packed, args.m)
    achieved = gbytes / (gms * 1e-3) / 1e9
    traffic = traffic_from_profile(kernel_source_hash())
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": "verify GEMM (k_gemm / k_gemm_lds as the tile table picks) at M=%d over the pass's four projection shapes" % args.m,
                "avg_launch_us": round(gms * 1e3 / launches, 2),
                "algorithmic_bytes_per_launch": round(gbytes / launches), "launches": launches,
                "per_shape": per_shape}
    ceiling = read_ceiling(torch, ctx)
    log("GEMM kernel alone: %.1f GB/s (%.1f%% of peak); read ceiling %.1f GB/s" % (
        achieved, 100 * achieved / PEAK_HBM_GBS, ceiling))

    stair = None if args.no_staircase else staircase_report(ctx)
    head = None if args.no_head else fp8_head_report(torch, nv, synth, ctx)

    result = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "full verify pass: %d layers x (q,k,v,o 5120x5120; gate,up 17408x5120; "
                               "down 5120x17408) NVFP4, M=%d bf16 rows" % (layers, args.m),
                   "m": args.m, "layers": layers, "weight_bytes_per_pass": pass_bytes,
                   "schedule": args.mode, "launch": launch},
        "pass_us": round(sec * 1e6, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "pass_us_%s" % other: round(sec_other * 1e6, 1),
        "per_m": per_m,
        "roofline": roofline,
        "read_ceiling_GBps": round(ceiling, 1),
        "staircase": stair,
        "fp8_head": head,
        "pages_context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(m=args.m)
    print(json.dumps(result), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()

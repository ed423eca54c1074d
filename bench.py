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
PROFILED_M = 16  # M of the committed rocprofv3 counter summaries
BYTES_PER_WEIGHT = 0.5625  # 4-bit code + one E4M3 byte per 16 weights
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense fp16 and bf16 MFMA (the same peak)
CLOCK_GHZ, SIMDS = 2.4, 1024  # 256 CUs x 4 SIMDs
VALU_CYCLES = 4  # a wave64 VALU instruction occupies a 16-lane SIMD for 4 cycles
METRIC = "verify-pass µs and achieved HBM GB/s vs M (1..32), full 27B layer stack"
# Pass schedules (nvfp4v_set_pass_mode) by name.
SCHEDULES = {"chain": "PASS_CHAIN", "persistent": "PASS_PERSISTENT"}
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
        flops = 2.0 * 16 * ((m + 15) // 16) * n * k  # the MFMAs run on M padded to 16-row blocks
        per_shape[name] = {"us": round(1e3 * ms / cnt, 2), "GBps": round(b * cnt / (ms * 1e-3) / 1e9, 1),
                           "mfma_TFLOPs": round(flops * cnt / (ms * 1e-3) / 1e12, 1),
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


def check_device(ctx, nv, what):
    """A timed leg counts only if every split-K row block of it completed (its
    pieces met on one XCD); the library reports anything else here."""
    st = ctx.device_status()
    assert st == nv.OK, "%s: device status %d (%s)" % (what, st, nv.strerror(st))


def teardown(torch, ctx, *holders):
    """Synchronise, drop the caller's device tensors, return the caching
    allocator's memory, then destroy the context, in that order."""
    import gc

    torch.cuda.synchronize()
    for h in holders:
        h.clear()
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    ctx.close()
    torch.cuda.synchronize()


def kernel_source_hash():
    """sha256 over the verify GEMM's device sources (the traffic figure in
    profiles/ is valid only for the kernel it was taken on)."""
    h = hashlib.sha256()
    for f in ("csrc/gemm.hip", "csrc/gemm_device.h", "csrc/internal.h", "tables/gfx950.txt"):
        h.update(open(os.path.join(ROOT, "nvfp4_skinny_gemm_amd", f), "rb").read())
    return h.hexdigest()


def profile_keys(name, gemm_src_hash):
    """The `key: value` lines of a committed rocprofv3 summary under profiles/,
    if it was taken on the current kernel source (same hash); else {}."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return {}
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != gemm_src_hash:
        return {}
    return vals


def traffic_from_profile(gemm_src_hash):
    """HBM bytes per GEMM launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source; else None."""
    try:
        return float(profile_keys("verify_gemm_pmc_fullpass_m16.txt", gemm_src_hash)["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def utilisation(gemm_src_hash, avg_launch_us):
    """MFMA and VALU utilisation of the verify GEMM launches: the committed
    rocprofv3 counters per launch (MFMA busy cycles, VALU instructions), if they
    were taken on the current kernel source, over the SIMD cycles of this run's
    average launch (1024 SIMDs at 2.4 GHz); None otherwise."""
    vals = profile_keys("verify_gemm_pmc_util_m16.txt", gemm_src_hash)
    simd_cycles = avg_launch_us * 1e-6 * CLOCK_GHZ * 1e9 * SIMDS
    try:
        return (float(vals["mfma_busy_cycles_per_launch"]) / simd_cycles,
                float(vals["valu_insts_per_launch"]) * VALU_CYCLES / simd_cycles)
    except (KeyError, ValueError):
        return None, None


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


def find_steps(us, m0=1, persist=2):
    """Staircase steps: M where the time exceeds 1.03x the median of the plateau
    of preceding M values by more than 3 MADs of that plateau's noise, and the
    next `persist` M values (where measured) stay above that threshold too, so
    a single noisy point is not a step."""
    import numpy as np

    steps, start = [], 0
    for i in range(1, len(us)):
        plateau = np.asarray(us[start:i])
        med = float(np.median(plateau))
        mad = float(np.median(np.abs(plateau - med))) if len(plateau) > 1 else 0.0
        thr = max(1.03 * med, med + 3 * mad)
        if us[i] > thr and all(u > thr for u in us[i + 1:i + 1 + persist]):
            steps.append(m0 + i)
            start = i
    return steps


STAIR_SHAPES = (("head", 151936, 5120), ("qkvo", 5120, 5120), ("gate_up", 17408, 5120), ("down", 5120, 17408))
STAIR_WARMUP, STAIR_ROUNDS = 2, 5  # the library times STAIR_ROUNDS batches of reps launches per M


def staircase_report(ctx, m_hi=64, reps=7):
    """A10: microseconds per M (1..m_hi) of the verify GEMM on the LM head and
    the layer shapes (rotating >= 2 GiB of weight copies), with step positions."""
    out = {}
    for name, n, k in STAIR_SHAPES:
        us = [round(float(x), 2) for x in ctx.staircase(n, k, 1, m_hi, warmup=STAIR_WARMUP, reps=reps,
                                                         rotate_bytes=2 << 30)]
        out[name] = {"shape": [n, k], "us": us, "steps": find_steps(us),
                     "GBps_m16": round(n * k * BYTES_PER_WEIGHT / (us[15] * 1e-6) / 1e9, 1) if m_hi >= 16 else None}
        at = lambda m: us[m - 1] if m <= m_hi else float("nan")
        log("staircase %s [%dx%d]: M1 %.1f us, M16 %.1f, M32 %.1f, M64 %.1f, M128 %.1f; steps at %s" % (
            name, n, k, at(1), at(16), at(32), at(64), at(128), out[name]["steps"]))
    return out


def summarize_staircase_trace(csv_path, m_hi=64, reps=7):
    """Per-M kernel durations of a `--staircase-only` run from its rocprofv3
    kernel trace (CSV): dispatches in start order; each shape's sweep begins
    with its fill kernel and one activation-packing kernel followed by an
    untimed launch per weight copy, then each M with its activation-packing
    kernel, followed by STAIR_WARMUP + STAIR_ROUNDS * reps GEMM launches, of
    which the timed ones are kept. Returns {shape: {"us": [median per M],
    "steps": [...]}}."""
    import csv
    import re
    import statistics

    rows = list(csv.DictReader(open(csv_path)))
    col = lambda key: next(c for c in rows[0] if key in c)
    kn, ks, ke = col("Kernel_Name"), col("Start_Timestamp"), col("End_Timestamp")
    rows.sort(key=lambda r: int(r[ks]))
    sections, cur, group = [], None, None
    for r in rows:
        found = re.search(r"\b(k_\w+)", r[kn])  # "void (anonymous namespace)::k_gemm<1, 2, 2>(...)"
        name = found.group(1) if found else r[kn]
        if name.startswith("k_fill_packed"):
            cur = []
            sections.append(cur)
        elif cur is not None and name.startswith("k_pack_act"):
            group = []
            cur.append(group)
        elif group is not None and name.startswith("k_gemm"):
            group.append((int(r[ke]) - int(r[ks])) * 1e-3)
    assert len(sections) == len(STAIR_SHAPES), "expected %d sweeps, found %d" % (len(STAIR_SHAPES), len(sections))
    out = {}
    timed = STAIR_ROUNDS * reps
    for (name, n, k), groups in zip(STAIR_SHAPES, sections):
        groups = groups[1:]  # the untimed rotation over the weight copies
        assert len(groups) == m_hi, "%s: %d row counts in the trace" % (name, len(groups))
        us = []
        for g in groups:
            assert len(g) == STAIR_WARMUP + timed, "%s: %d GEMM launches for one M" % (name, len(g))
            us.append(round(statistics.median(g[STAIR_WARMUP:]), 2))
        out[name] = {"shape": [n, k], "us": us, "steps": find_steps(us)}
    return out


def summarize_counters(csv_paths):
    """No GPU: per-kernel mean / min / max of every counter in rocprofv3
    counter-collection CSVs (one row per dispatch and counter), and the
    dispatch-weighted mean over all verify GEMM dispatches (k_gemm*)."""
    import csv
    import re
    from collections import defaultdict

    per = defaultdict(list)
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            found = re.search(r"\b(k_\w+(<[^>]*>)?)", r["Kernel_Name"])
            per[(found.group(1) if found else r["Kernel_Name"][:40], r["Counter_Name"])].append(float(r["Counter_Value"]))
    out = {}
    for (kernel, counter), v in sorted(per.items()):
        out.setdefault(kernel, {})[counter] = {"n": len(v), "mean": sum(v) / len(v), "min": min(v), "max": max(v)}
    gemm = defaultdict(list)
    for (kernel, counter), v in per.items():
        if kernel.startswith("k_gemm"):
            gemm[counter].extend(v)
    out["all verify GEMM dispatches"] = {c: {"n": len(v), "mean": sum(v) / len(v)} for c, v in sorted(gemm.items())}
    return out


ATTN_CTXS, ATTN_MS = (1024, 4096, 16384, 32768), (1, 8, 16, 17, 24, 32)


def attention_report(torch, nv, synth, ctx, ctxs=ATTN_CTXS, ms=ATTN_MS,
                     hq=40, hkv=40, warmup=3, reps=20):
    """Tree-verify attention of one layer (40 heads of 128, the stand-in layer's
    q, k and v) per context length and tree size: microseconds per call and the
    key/value bytes read per second. Random bf16 caches, rotated over enough
    copies (>= 512 MiB) that every call streams them from HBM. The `reps` calls
    are captured in a HIP graph and replayed, so the figure is the kernel's
    time, not the Python binding's per-call overhead."""
    d = 128
    out = {"heads": [hq, hkv], "head_dim": d, "us": {}, "GBps": {}, "plan": {}}
    for T in ctxs:
        cap = (T + max(ms) + 31) // 32 * 32
        nbytes = nv.kv_cache_bytes(cap, hkv, d)
        copies = max(1, min(24, -(-(512 << 20) // (2 * nbytes))))
        caches = []
        g = torch.Generator(device="cuda")
        g.manual_seed(T)
        for _ in range(copies):
            kc = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            vc = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            rows = torch.randn((cap, hkv, d), generator=g, device="cuda").to(torch.bfloat16)
            ctx.kv_write(rows, rows.roll(1, 0).contiguous(), 0, cap, kc, vc)
            caches.append((kc, vc))
            del rows
        for m in ms:
            q = torch.randn((m, hq, d), generator=g, device="cuda").to(torch.bfloat16)
            parent = synth.tree_parent_rows(m, seed=m)
            ws = torch.zeros(nv.tree_attention_workspace_bytes(T, m, hq, hkv, d), dtype=torch.uint8, device="cuda")
            o = torch.empty((m, hq, d), dtype=torch.float32, device="cuda")
            for i in range(warmup):
                kc, vc = caches[i % copies]
                ctx.tree_attention(q, kc, vc, cap, T, hkv, parent, out=o, ws=ws)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(reps):
                    kc, vc = caches[i % copies]
                    ctx.tree_attention(q, kc, vc, cap, T, hkv, parent, out=o, ws=ws)
            graph.replay()  # warm
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(2):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            del graph
            us = e0.elapsed_time(e1) * 1e3 / (2 * reps)
            key = "%d/%d" % (T, m)
            out["us"][key] = round(us, 2)
            out["GBps"][key] = round((T + m) * hkv * d * 4 / (us * 1e-6) / 1e9, 1)
            out["plan"][key] = list(ctx.tree_attention_plan(T, m, hq, hkv, d))
        log("tree attention, %d heads, context %d: %s us; %s GB/s" % (
            hq, T, [out["us"]["%d/%d" % (T, m)] for m in ms], [out["GBps"]["%d/%d" % (T, m)] for m in ms]))
        del caches
        torch.cuda.empty_cache()
    return out


def summarize_attention_trace(csv_path, counters=None):
    """No GPU: per (context, M) kernel durations of an `--attention-only` run
    from its rocprofv3 kernel trace. Per (context, M), in the order
    attention_report times them, the tree-attention dispatches come as a run of
    3 warm-up calls and a run of 60 graph-replayed ones (other kernels, the
    inputs' generation and the graph capture's own, separate the runs); the
    median of each 60-dispatch run. With `counters` (counter-collection CSVs of
    the same command), the per-dispatch means of each counter over those runs."""
    import csv
    import re
    import statistics

    rows = list(csv.DictReader(open(csv_path)))
    col = lambda key: next(c for c in rows[0] if key in c)
    kn, ks, ke = col("Kernel_Name"), col("Start_Timestamp"), col("End_Timestamp")
    rows.sort(key=lambda r: int(r[ks]))
    runs, cur = [], None
    for r in rows:
        if re.search(r"\bk_tree_attn<", r[kn]):
            if cur is None:
                cur = []
                runs.append(cur)
            cur.append((int(r[ke]) - int(r[ks])) * 1e-3)
        else:
            cur = None
    runs = [r for r in runs if len(r) > 3]
    keys = ["%d/%d" % (t, m) for t in ATTN_CTXS for m in ATTN_MS]
    assert len(runs) == len(keys), "expected %d runs of attention dispatches, found %d" % (len(keys), len(runs))
    out = {"us": {}, "GBps": {}}
    for key, run in zip(keys, runs):
        t, m = map(int, key.split("/"))
        us = statistics.median(run)
        out["us"][key] = round(us, 2)
        out["GBps"][key] = round((t + m) * 40 * 128 * 4 / (us * 1e-6) / 1e9, 1)
    if counters:
        per = {}
        for path in counters:
            cnt_rows = [r for r in csv.DictReader(open(path)) if re.search(r"\bk_tree_attn<", r["Kernel_Name"])]
            # rocprofv3 numbers dispatches in order; consecutive ids form the runs
            cnt_rows.sort(key=lambda r: int(r["Dispatch_Id"]))
            runs_c, prev = [], None
            for r in cnt_rows:
                d = int(r["Dispatch_Id"])
                if prev is None or d != prev + 1:
                    runs_c.append([])
                runs_c[-1].append(float(r["Counter_Value"]))
                prev = d
            runs_c = [r for r in runs_c if len(r) > 3]
            assert len(runs_c) == len(keys), "expected %d runs in %s, found %d" % (len(keys), path, len(runs_c))
            name = cnt_rows[0]["Counter_Name"]
            per[name] = {k: round(sum(v) / len(v), 1) for k, v in zip(keys, runs_c)}
        out["counters"] = per
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
    ap.add_argument("--mode", choices=tuple(SCHEDULES), default="chain",
                    help="pass schedule of the headline number")
    ap.add_argument("--compare", default="persistent",
                    help="comma-separated schedules timed beside the headline one ('' = none)")
    ap.add_argument("--sweep", default="1-32,40,48,64,65,96,128", help="M values for the per-M pass staircase ('' = none)")
    ap.add_argument("--sweep-steps", type=int, default=5)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-staircase", action="store_true")
    ap.add_argument("--no-head", action="store_true", help="skip the FP8 output head timing")
    ap.add_argument("--head-only", action="store_true", help="time only the FP8 output head")
    ap.add_argument("--no-attention", action="store_true", help="skip the tree-verify attention timing")
    ap.add_argument("--attention-only", action="store_true", help="time only the tree-verify attention")
    ap.add_argument("--staircase-only", action="store_true",
                    help="time only the per-shape staircase (M = 1..--stair-max) and print it as JSON")
    ap.add_argument("--stair-max", type=int, default=128)
    ap.add_argument("--summarize-staircase-trace", metavar="CSV",
                    help="no GPU: per-M kernel durations from the rocprofv3 kernel trace of a --staircase-only run")
    ap.add_argument("--summarize-attention-trace", metavar="CSV", nargs="+",
                    help="no GPU: per (context, M) kernel durations from the rocprofv3 kernel trace of an "
                         "--attention-only run, then optional counter-collection CSVs of the same command")
    ap.add_argument("--summarize-counters", metavar="CSV", nargs="+",
                    help="no GPU: per-kernel counter means from rocprofv3 counter-collection CSVs")
    ap.add_argument("--gemm-only", action="store_true",
                    help="only the verify-GEMM roofline leg and a 256 MiB copy (for hardware-counter runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the weight rows "
              "would shard by column, or by K with one all-reduce per row-parallel projection); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.summarize_attention_trace:
        paths = args.summarize_attention_trace
        print(json.dumps(summarize_attention_trace(paths[0], paths[1:])), flush=True)
        return
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters), indent=1), flush=True)
        return
    if args.summarize_staircase_trace:
        assert args.stair_max <= 64, "the trace summary reads one packing kernel per M (M <= 64)"
        print(json.dumps(summarize_staircase_trace(args.summarize_staircase_trace, args.stair_max)), flush=True)
        return

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
    if args.attention_only:
        print(json.dumps({"tree_attention": attention_report(torch, nv, synth, ctx)}), flush=True)
        ctx.close()
        return
    if args.staircase_only:
        print(json.dumps({"staircase": staircase_report(ctx, m_hi=args.stair_max)}), flush=True)
        check_device(ctx, nv, "staircase")
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
    rows = max([args.m] + parse_sweep(args.sweep))  # every timed pass reads its first M rows
    assert 1 <= rows <= nv.MAX_M, "M up to %d" % nv.MAX_M
    h0 = torch.from_numpy(synth.activations_bf16(rows, H, seed=0, stream="pass/h0").view("int16")).cuda()
    h0 = h0.view(torch.bfloat16)
    ws = torch.empty(nv.pass_workspace_bytes(rows, H, I, layers), dtype=torch.uint8, device="cuda")
    h_out = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    pass_bytes = layer_weight_bytes() * layers
    modes = {name: getattr(nv, const) for name, const in SCHEDULES.items()}
    others = [o for o in args.compare.split(",") if o and o != args.mode]
    for o in others:
        assert o in modes, "unknown schedule %r" % o

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
        check_device(ctx, nv, "pass M=%d" % m)
        del runner
        torch.cuda.synchronize()
        return sec, launch

    # ---- headline: the pass at M = args.m --------------------------------------
    # One step is one pass over all layers: a packing kernel plus the layers'
    # GEMMs (four launches per layer, or one persistent kernel per 32 layers),
    # replayed from a HIP graph; weights and input are resident in HBM.
    sec_others = {}
    for o in others:
        ctx.set_pass_mode(modes[o])
        sec_others[o], _ = timed_pass(args.m, 2, max(3, args.steps // 4))
    ctx.set_pass_mode(modes[args.mode])
    sec, launch = timed_pass(args.m, args.warmup, args.steps)
    assert torch.isfinite(h_out[: args.m].float()).all(), "non-finite pass output"
    gbs = pass_bytes / sec / 1e9
    log("M=%d: %.1f us per pass, %.1f GB/s (%s, %s); %s" % (
        args.m, sec * 1e6, gbs, args.mode, launch,
        ", ".join("%s %.1f us" % (o, t * 1e6) for o, t in sec_others.items())))

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
    check_device(ctx, nv, "roofline GEMMs")
    achieved = gbytes / (gms * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    avg_us = gms * 1e3 / launches
    # The committed counter summaries were taken at M = 16: other M report none.
    traffic = traffic_from_profile(src_hash) if args.m == PROFILED_M else None
    mfma_util, valu_util = utilisation(src_hash, avg_us) if args.m == PROFILED_M else (None, None)
    mfma_tflops = sum(v["mfma_TFLOPs"] * v["us"] for v in per_shape.values()) / sum(v["us"] for v in per_shape.values())
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "mfma_util": None if mfma_util is None else round(mfma_util, 4),
                "valu_util": None if valu_util is None else round(valu_util, 4),
                "mfma_flops_frac": round(mfma_tflops / PEAK_BF16_TFLOPS, 4),
                "kernel": "verify GEMM (k_gemm / k_gemm_lds as the tile table picks) at M=%d over the pass's four projection shapes" % args.m,
                "avg_launch_us": round(avg_us, 2),
                "algorithmic_bytes_per_launch": round(gbytes / launches), "launches": launches,
                "per_shape": per_shape}
    ceiling = read_ceiling(torch, ctx)
    log("GEMM kernel alone: %.1f GB/s (%.1f%% of peak); read ceiling %.1f GB/s" % (
        achieved, 100 * achieved / PEAK_HBM_GBS, ceiling))

    stair = None if args.no_staircase else staircase_report(ctx, m_hi=args.stair_max)
    check_device(ctx, nv, "staircase")
    head = None if args.no_head else fp8_head_report(torch, nv, synth, ctx)
    check_device(ctx, nv, "fp8 head")
    attn = None if args.no_attention else attention_report(torch, nv, synth, ctx)

    result = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "full verify pass: %d layers x (q,k,v,o 5120x5120; gate,up 17408x5120; "
                               "down 5120x17408) NVFP4, M=%d bf16 rows" % (layers, args.m),
                   "m": args.m, "layers": layers, "weight_bytes_per_pass": pass_bytes,
                   "schedule": args.mode, "launch": launch,
                   "arithmetic": "weights dequantised to fp16 and bf16 activations held exactly as fp16 "
                                 "x 2^8 in the MFMA operands, fp32 sums (C bitwise equal to the bf16 "
                                 "computation)"},
        "pass_us": round(sec * 1e6, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "pass_us_other_schedules": {o: round(t * 1e6, 1) for o, t in sec_others.items()},
        "per_m": per_m,
        "roofline": roofline,
        "read_ceiling_GBps": round(ceiling, 1),
        "staircase": stair,
        "fp8_head": head,
        "tree_attention": attn,
        "pages_context": PAGES_CONTEXT,
    }
    # Release every device object (weights, workspace, the context) before the
    # interpreter exits, so nothing of the run is torn down by late destructors.
    del layer_arr, h0, ws, h_out
    teardown(torch, ctx, packed)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(m=args.m)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

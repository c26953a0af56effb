#!/usr/bin/env python3
"""Benchmark of the CSA/HCA attention hot path on one MI355X.

A step is one layer's pass over one batch of new tokens: compress the entries the
tokens complete, write the tokens into the sliding-window cache, score and select
entries with the lightning indexer (CSA), attend.  The headline workload is
DeepSeek-V4-Pro CSA decode at 65,536 tokens of context: batch 32, 128 query heads
of dim 512 on one shared KV head, 64 x 128 indexer with fp8 keys, top-1,024,
128-token window, per-head sink.  Synthetic seeded inputs; distinct per-layer caches
are rotated so that the 256 MB last-level cache cannot serve repeated reads.

Prints one JSON line.  Extra measurements (HCA decode at 1M context, the Flash fp8
decode at 1M, per-call times) ride in the same line under "extra".

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
METRIC = "CSA/HCA decode tokens/s + indexer HBM GB/s at 65K/1M ctx; % of roofline"


def kv_row_bytes(wl):
    """Bytes of one stored compressed-KV row: bf16 values, fp8 codes + fp32 scale per block, or
    fp4 codes (two per byte) + fp32 scale per 32 channels."""
    if wl.kv_dtype == "fp8":
        return wl.D + 4 * wl.D // wl.kv_scale_block
    if wl.kv_dtype == "fp4":
        return wl.D // 2 + 4 * wl.D // wl.kv_scale_block
    return 2 * wl.D


def algorithmic_costs(wl):
    """Bytes / flops each C-ABI call of one step must move / do at minimum.

    indexer: each visible key once per sequence (Di bytes fp8 + 4-byte scale, or 2*Di bf16;
             a sequence's query tokens all score the same keys), the indexer queries and
             weights, the selected indices.
    attend:  each attended row once per query token (1 KB bf16, 512 B + 32 B scales fp8,
             256 B + 64 B scales fp4; window rows bf16), q in (bf16) and out (bf16); flops
             4 * H * rows * 512 per token.
    compress: raw kv + logits of the new tokens (2 KB per token) and the new rows.
    """
    rows = wl.B * wl.Tq
    E = wl.E
    key_b = (wl.Di + 4) if wl.idx_dtype == "fp8" else 2 * wl.Di
    kv_row_b = kv_row_bytes(wl)
    c = {}
    if wl.mode == "csa":
        c["index_bytes"] = wl.B * E * key_b + rows * (wl.Hi * wl.Di * 2 + wl.Hi * 4 + wl.topk * 4)
        c["index_flops"] = rows * E * wl.Hi * wl.Di * 2
        ent_rows = wl.topk
    else:
        ent_rows = E
    att_rows = ent_rows + wl.W
    c["attend_bytes"] = rows * (ent_rows * kv_row_b + wl.W * 2 * wl.D + 2 * wl.H * wl.D * 2)
    c["attend_flops"] = rows * 4 * wl.H * att_rows * wl.D
    new_entries = wl.E - wl.n_entries(wl.N - wl.Tq)
    raw = (new_entries - 1) * wl.stride + wl.window if new_entries else 0
    c["compress_bytes"] = wl.B * (raw * 2 * wl.D * 2 + new_entries * kv_row_b + wl.Tq * wl.D * 4)
    return c


def stats(samples):
    """Median, 10th and 90th percentiles (nearest rank) and count of timing samples (ms)."""
    xs = sorted(samples)
    n = len(xs)
    pick = lambda q: xs[min(n - 1, max(0, int(math.ceil(q * n)) - 1))]
    return {"median_ms": pick(0.5), "p10_ms": pick(0.1), "p90_ms": pick(0.9), "n": n}


def build_layers(wl, n_layers, device, torch, out_dtype):
    import csa_inputs as ci
    from compressed_attention_long_amd.step import LayerStep
    steps = []
    for i in range(n_layers):
        t, meta = ci.step_tensors(wl, device, seed=ci.seed_for(wl.name) + 7919 * i)
        steps.append(LayerStep(wl, t, meta, out_dtype=out_dtype))
    torch.cuda.synchronize()
    return steps


def layer_bytes(wl):
    kv_row_b = kv_row_bytes(wl)
    key_b = ((wl.Di + 4) if wl.idx_dtype == "fp8" else 2 * wl.Di) if wl.mode == "csa" else 0
    return wl.B * wl.E * (kv_row_b + key_b + (4 if wl.mode == "csa" else 0))


def capture_graphs(layers, torch):
    """One HIP graph per layer holding that layer's whole step (all buffers preallocated)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for L in layers:
            L.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for L in layers:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            L.run()
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def capture_chain(layers, torch):
    """One HIP graph holding the steps of all layers in order (as a decode step of a model
    replays all its layers from one graph)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for L in layers:
            L.run()
    torch.cuda.synchronize()
    return g


def time_workload(wl, steps_n, warmup, torch, min_cache_bytes=4 << 30, max_layers=30):
    if wl.Tq >= 64:
        max_layers = 2      # prefill: each step's own tensors (q, scores, output) exceed the 256 MB MALL
    """Time `steps_n` steps rotating over distinct layers; return timings (ms).

    Headline: layer steps replayed from one HIP graph that chains all rotated layers (as a
    serving loop replays a model's layers), K steps = K // L chain replays plus K % L
    single-layer graphs.  Also: one graph per layer step (includes a graph launch per step);
    per C-ABI call, a graph of that call over the rotated layers replayed between HIP events
    on the launch stream (the per-call times and the roofline); and an eager pass with events
    around each call (host launch gaps included, for reference).
    """
    n_layers = max(2, min(max_layers, math.ceil(min_cache_bytes / max(layer_bytes(wl), 1))))
    layers = build_layers(wl, n_layers, "cuda", torch, torch.bfloat16)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        layers[i % n_layers].run()
    torch.cuda.synchronize()
    # --- graph replay (headline)
    graphs = capture_graphs(layers, torch)
    for i in range(warmup):
        graphs[i % n_layers].replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_samp = max(steps_n, 50)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_samp + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_samp):
        step_ev[i].record(stream)
        graphs[i % n_layers].replay()
    step_ev[n_samp].record(stream)
    torch.cuda.synchronize()
    wall_per_layer_graph = (time.perf_counter() - t0) * 1e3 / n_samp
    step_samples = [step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(n_samp)]
    graph_gpu_per_layer_graph = sum(step_samples) / n_samp
    # --- chained graph (headline)
    chain = capture_chain(layers, torch)
    for i in range(max(1, warmup // n_layers)):
        chain.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record()
    for i in range(steps_n // n_layers):
        chain.replay()
    for i in range(steps_n % n_layers):
        graphs[i].replay()
    g1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps_n
    graph_gpu = g0.elapsed_time(g1) / steps_n
    # --- per-call graphs: one C-ABI call per layer, replayed between events (breakdown, roofline)
    call_fns = {"compress": lambda L: L.compress(), "attend": lambda L: L.attend()}
    if wl.mode == "csa":
        call_fns["index"] = lambda L: L.index()
        call_fns["index_compress"] = lambda L: L.index_compress()
    reps = max(50, steps_n // n_layers)
    calls_graph, calls_samples = {}, {}
    for name, fn in call_fns.items():
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for L in layers:
                fn(L)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            for L in layers:
                fn(L)
        cg.replay()
        torch.cuda.synchronize()
        cev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        for r in range(reps):
            cev[r].record(stream)
            cg.replay()
        cev[reps].record(stream)
        torch.cuda.synchronize()
        samples = [cev[r].elapsed_time(cev[r + 1]) / n_layers for r in range(reps)]
        calls_graph[name] = sum(samples) / reps
        calls_samples[name] = samples
        del cg
    # --- eager pass with per-call events (reference: includes host launch gaps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps_n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps_n):
        L = layers[i % n_layers]
        e = ev[i]
        e[0].record(stream)
        L.compress()
        e[1].record(stream)
        if wl.mode == "csa":
            L.index()
        e[2].record(stream)
        L.attend()
        e[3].record(stream)
    torch.cuda.synchronize()
    eager_wall = (time.perf_counter() - t0) * 1e3 / steps_n
    per = {"compress": [], "index": [], "attend": [], "step_gpu": []}
    for e in ev:
        per["compress"].append(e[0].elapsed_time(e[1]))
        per["index"].append(e[1].elapsed_time(e[2]))
        per["attend"].append(e[2].elapsed_time(e[3]))
        per["step_gpu"].append(e[0].elapsed_time(e[3]))
    med = lambda xs: sorted(xs)[len(xs) // 2]
    out = {k: sum(v) / len(v) for k, v in per.items()}
    out["calls_graph"] = calls_graph
    out["calls_stats"] = {k: stats(v) for k, v in calls_samples.items()}
    out["step_stats"] = stats(step_samples)
    out["step_gpu_median"] = med(per["step_gpu"])
    out["wall_ms_per_step"] = wall
    out["graph_gpu_ms_per_step"] = graph_gpu
    out["per_layer_graph_wall_ms_per_step"] = wall_per_layer_graph
    out["per_layer_graph_gpu_ms_per_step"] = graph_gpu_per_layer_graph
    out["eager_wall_ms_per_step"] = eager_wall
    out["layers"] = n_layers
    del graphs, chain, layers
    torch.cuda.empty_cache()
    return out


def time_reuse(wl, steps_n, warmup, torch, min_cache_bytes=4 << 30):
    """Reuse layers (CSA2: KV and top-k selection computed in one layer and reused by others):
    one csa_attend per layer with the layer's own queries and sink over a computed layer's
    caches and selection.  Replayed from one HIP graph chaining the reuse layers of the rotated
    computed layers; returns ms per reuse-layer step."""
    import csa_inputs as ci
    from compressed_attention_long_amd.step import ReuseStep
    n_layers = max(2, min(30, math.ceil(min_cache_bytes / max(layer_bytes(wl), 1))))
    layers = build_layers(wl, n_layers, "cuda", torch, torch.bfloat16)
    for L in layers:
        L.run()                       # the computed layers' caches and selections
    reuse = []
    for i, L in enumerate(layers):
        r = ci.reuse_tensors(wl, "cuda", seed=ci.seed_for(wl.name) + 31337 * (i + 1))
        reuse.append(ReuseStep(L, r["q"], r["sink"]))
    for i in range(warmup):
        reuse[i % n_layers].run()
    torch.cuda.synchronize()
    chain = capture_chain(reuse, torch)
    chain.replay()
    torch.cuda.synchronize()
    reps = max(1, steps_n // n_layers)
    t0 = time.perf_counter()
    for _ in range(reps):
        chain.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / (reps * n_layers)
    del chain, reuse, layers
    torch.cuda.empty_cache()
    return ms


def out_projection_bench(torch, T=32, reps=50):
    """csa_out_proj at the 65K decode batch (32 tokens; 128 heads x 512 -> 16 groups x rank 1,024 ->
    hidden 7,168, atlas Raw config fields o_groups, o_lora_rank, hidden_size), synthetic bf16
    factors, the bf16 attention output the decode step writes.  Not part of the timed step (the
    pages' attention path ends at the attention output); reported as its own HBM-bound call: the
    factors (2 B per element) are read once per call, the tokens' activations are small."""
    from compressed_attention_long_amd import _lib as ops
    dev = "cuda"
    H, D, G, R, hidden = 128, 512, 16, 1024, 7168
    g = torch.Generator(device=dev)
    g.manual_seed(777)
    o = torch.randn((T, H, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    wa = (torch.randn((G, R, (H // G) * D), generator=g, device=dev, dtype=torch.float32) / 64.0).to(torch.bfloat16)
    wb = (torch.randn((hidden, G * R), generator=g, device=dev, dtype=torch.float32) / 128.0).to(torch.bfloat16)
    y = torch.empty((T, hidden), dtype=torch.bfloat16, device=dev)
    ws = ops.workspace(ops.csa_out_proj_workspace_bytes(T, G, R, hidden), dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ops.csa_out_proj(o, wa, wb, y, ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        ops.csa_out_proj(o, wa, wb, y, ws)
    samples = []
    with torch.cuda.stream(s):
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            graph.replay()
            e1.record(s)
            e1.synchronize()
            samples.append(e0.elapsed_time(e1))
    ms = sum(samples) / len(samples)
    nbytes = (wa.numel() + wb.numel()) * 2 + o.numel() * 2 + y.numel() * 2 + 2 * T * G * R * 4
    flops = 2 * T * (H * D * R + G * R * hidden)
    return {"tokens": T, "ms": ms, "stats": stats(samples), "bytes": nbytes, "GB_per_s": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "TFLOP_per_s": flops / (ms * 1e-3) / 1e12,
            "shape": "o [32, 128, 512] bf16; wa [16, 1024, 4096] bf16; wb [7168, 16384] bf16; y bf16"}


def compressor_bulk(torch, reps=3):
    """csa_compress over whole raw streams (the compressor's HBM benchmark): kv and pooling
    logits read once, entries written once.  Inputs tile one seeded 64K-token random block
    (the kernel has no data-dependent control flow).  Shapes: the 65K CSA decode batch
    (32 x 65,536 tokens), the Flash 1M batch with fp8 entries (4 x 1,048,576) and HCA at 1M
    (4 of the 16 sequences of the HCA decode batch; the per-sequence work is identical)."""
    import math as _m
    from compressed_attention_long_amd import _lib as ops
    from compressed_attention_long_amd.rope import yarn_inv_freq
    dev = "cuda"
    inv = yarn_inv_freq(160000.0, 64, 16.0, 65536, dev)   # the model's table
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    blk = 65536
    base_kv = torch.randn((1, blk, 512), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    base_z = torch.randn((1, blk, 512), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    out = {}
    for name, B, T, window, stride, fp8 in [("csa_65k_b32", 32, 65536, 8, 4, False),
                                            ("csa_1m_b4_fp8", 4, 1 << 20, 8, 4, True),
                                            ("hca_1m_b4", 4, 1 << 20, 128, 128, False)]:
        kv = torch.empty((B, T, 512), dtype=torch.bfloat16, device=dev)
        z = torch.empty_like(kv)
        kv.view(B, T // blk, blk, 512).copy_(base_kv.expand(B, T // blk, blk, 512).reshape(B, T // blk, blk, 512))
        z.view(B, T // blk, blk, 512).copy_(base_z.expand(B, T // blk, blk, 512).reshape(B, T // blk, blk, 512))
        E = (T - window) // stride + 1
        nv = torch.full((B,), E, dtype=torch.int32, device=dev)
        p0 = torch.ones((B,), dtype=torch.int64, device=dev)
        if fp8:
            cache = ops.Cache(torch.empty((B, E, 512), dtype=torch.uint8, device=dev), nv, p0, window, stride,
                              scales=torch.empty((B, E, 8), dtype=torch.float32, device=dev), scale_block=64)
            out_bytes = B * E * (512 + 32)
        else:
            cache = ops.Cache(torch.empty((B, E, 512), dtype=torch.bfloat16, device=dev), nv, p0, window, stride)
            out_bytes = B * E * 1024
        in_bytes = 2 * B * T * 1024
        ops.compress(kv, z, cache, 0, E, inv, 64)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ops.compress(kv, z, cache, 0, E, inv, 64)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        t = sorted(ts)[len(ts) // 2]
        gbs = (in_bytes + out_bytes) / (t * 1e-3) / 1e9
        out[name] = {"ms": t, "bytes": in_bytes + out_bytes, "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                     "entries": B * E}
        del kv, z, cache
        torch.cuda.empty_cache()
    return out


PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_bytes_csa_decode_65k.md")


CALL_SOURCES = {"attend": ("attend.hip", "attend_dev.hpp", "workspace.hpp"),
                "index": ("indexer.hip", "compress_dev.hpp", "workspace.hpp"),
                "compress": ("compress.hip", "compress_dev.hpp")}


def code_only(text):
    """C++ source without its comments and blank space: what the compiler sees, so that an edit to
    a comment does not count as a change of the kernels."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":                       # string or character literal, escapes kept
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(" ".join(line.split()) for line in "".join(out).splitlines() if line.strip())


def source_digest(call):
    """sha256 over the code (comments and blank space dropped) of one C-ABI call's kernel sources:
    counter-derived traffic is only reported for the code it was measured on."""
    import hashlib
    h = hashlib.sha256()
    for f in (*CALL_SOURCES[call], "api.hip", "common.hpp", "internal.hpp"):
        with open(os.path.join(ROOT, "compressed_attention_long_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()


def measured_traffic(workload, call):
    """HBM bytes per call from the committed counter summary (FETCH_SIZE x calibration + WRITE_SIZE),
    or None when the summary is missing, covers another workload/call, or the kernels changed since."""
    try:
        with open(PMC_SUMMARY) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    d = json.loads(line[len("traffic-json: "):])
                    if d.get("workload") == workload and d.get("call") == call and d.get("sources") == source_digest(call):
                        return d["bytes_per_call"]
    except OSError:
        pass
    return None


def pmc_probe(wl, torch, layers_n=4, reps=2):
    """Workload for hardware-counter passes: a plain 256 MiB device copy three times (calibrates
    FETCH_SIZE / WRITE_SIZE against a known byte count), then `reps` eager steps over `layers_n`
    distinct layers, every C-ABI call launched on its own (compress, index, attend as three
    calls, so that the counters split by call)."""
    src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    layers = build_layers(wl, layers_n, "cuda", torch, torch.bfloat16)
    for _ in range(reps):
        for L in layers:
            L.run(combined=False)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_probe": wl.name, "copy_bytes_each_way": 256 << 20, "layers": layers_n, "reps": reps,
                      "sources": {c: source_digest(c) for c in CALL_SOURCES}}), flush=True)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(wl, budget_s=12.0, threads=None, max_rows=None):
    """The fp64 oracle on a bounded sample of the same workload, in tokens/s.

    Inputs are one sequence's share of the workload (B = 1, same shapes and distributions).
    A decode step per query row: compress the step's new entries and window rows, then (CSA)
    index, select and attend, or (HCA) attend to every visible entry.  A prefill chunk: its
    new entries are compressed once (charged pro rata to the sampled rows), then sampled query
    rows (first, last, the rest spread uniformly) each run the indexer, top-k and attention.
    Rows are taken until about `budget_s` seconds have passed (at most `max_rows`).  `threads`
    limits the BLAS pool (None: all the host's cores)."""
    import contextlib
    import dataclasses
    import numpy as np
    import csa_inputs as ci
    from oracle import csa_oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=threads) if threads else contextlib.nullcontext()
    except Exception:
        limit = contextlib.nullcontext()
    one = dataclasses.replace(wl, B=1)
    t, meta = ci.step_tensors(one, "cpu", seed=ci.seed_for(wl.name))
    with limit:
        cores = _blas_threads()
        if wl.yarn_factor > 1.0:
            f = O.yarn_inv_freq(160000.0, wl.R, wl.yarn_factor, wl.yarn_base_len)
            scale = O.yarn_logit_scale(wl.yarn_factor) / math.sqrt(wl.D)
        else:
            f = O.rope_inv_freq(160000.0, wl.R)
            scale = 1 / math.sqrt(wl.D)
        ent_pos = O.entry_positions(wl.pos0, wl.E, wl.window, wl.stride)
        win_pos = int(t["win_pos0"][0]) + np.arange(meta["win_cap"])
        sink = t["sink"].double().numpy()
        if wl.kv_dtype == "fp4":
            kv = O.mxfp4_block_dequantize(O.fp4_unpack(t["kv_cache"][0].numpy()), t["kv_cache_scale"][0].numpy(),
                                          wl.kv_scale_block)
        elif wl.kv_dtype == "fp8":
            kv = O.fp8_block_dequantize(t["kv_cache"][0].numpy(), t["kv_cache_scale"][0].numpy(), wl.kv_scale_block)
        else:
            kv = t["kv_cache"][0].double().numpy()
        keys = None
        if wl.mode == "csa":
            keys = t["k_idx"][0].double().numpy() if wl.idx_dtype == "bf16" else O.fp8_block_dequantize(
                t["k_idx"][0].numpy(), t["k_idx_scale"][0].numpy(), wl.Di)
        win = t["win_cache"][0].double().numpy()
        kv_raw, z_raw = t["kv_raw"][0].double().numpy(), t["z_raw"][0].double().numpy()
        Tq = wl.Tq
        if Tq > 1:
            order = [0, Tq - 1] + [int(round(x)) for x in np.linspace(0, Tq - 1, 64)[1:-1]]
        else:
            order = [0]

        def compress_step():
            new, _ = O.compress(kv_raw, z_raw, wl.window, wl.stride, wl.pos0 + meta["E_pre"] * wl.stride, f)
            kv[meta["E_pre"]:] = new[:meta["n_new_entries"]]
            win[meta["win_first_new"]:] = O.rope(kv_raw[-meta["new_tok"]:], win_pos[meta["win_first_new"]:], f)

        def query(tq):
            qp = int(t["q_pos"][0, tq])
            q = t["q"][0, tq].double().numpy()
            if wl.mode == "csa":
                O.csa_query(q, qp, t["q_idx"][0, tq].double().numpy(), t["w"][0, tq].double().numpy(), kv, ent_pos,
                            keys, win, win_pos, sink, wl.topk, scale, f, wl.W)
            else:
                O.hca_query(q, qp, kv, ent_pos, win, win_pos, sink, scale, f, wl.W)

        n_rows, t_rows, t_comp, n_comp = 0, 0.0, 0.0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s and (max_rows is None or n_rows < max_rows):
            if Tq == 1 or n_comp == 0:
                c0 = time.perf_counter()
                compress_step()
                t_comp += time.perf_counter() - c0
                n_comp += 1
            r0 = time.perf_counter()
            query(order[n_rows % len(order)])
            t_rows += time.perf_counter() - r0
            n_rows += 1
        if Tq == 1:
            total = t_comp + t_rows
            what = f"{n_rows} single-sequence decode steps"
        else:
            total = t_comp * n_rows / Tq + t_rows         # the chunk's compression, pro rata
            what = (f"{n_rows} sampled query rows of the {Tq}-row chunk (first, last, uniform), the chunk's "
                    f"compression charged pro rata")
    return {"value": n_rows / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{what} of {wl.name} (one sequence's inputs of the same shapes; fp64 NumPy oracle, "
                      f"{cores} BLAS thread{'s' if cores > 1 else ''}; {time.perf_counter() - t0:.1f} s of host time)"}


def achievable_peaks(torch):
    """Measured ceilings on this GPU, beside the datasheet peaks: HBM bandwidth of a plain
    device copy of 2 GiB (torch's copy kernel; bytes read + written) and dense bf16 GEMM
    throughput at 8192^3 (torch.matmul, the vendor BLAS).  Context for the roofline fractions,
    which stay against the datasheet peaks."""
    out = {}
    src = torch.empty(1 << 29, dtype=torch.float32, device="cuda").fill_(1.0)   # 2 GiB
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 1e9
    for _ in range(5):
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    out["hbm_copy_GB_per_s"] = 2 * src.numel() * 4 / (best * 1e-3) / 1e9
    del src, dst
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    best = 1e9
    for _ in range(5):
        e0.record()
        a @ b
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    out["bf16_gemm_TFLOP_per_s"] = 2 * n ** 3 / (best * 1e-3) / 1e12
    out["how"] = "best of 5: torch copy of a 2 GiB buffer (read + write bytes); torch.matmul bf16 8192^3"
    del a, b
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v4pro_csa_decode_65k")
    ap.add_argument("--extra", default="v4pro_hca_decode_1m,v4flash_csa_decode_1m_fp8,v4pro_csa_prefill_4k_on_131k,"
                                       "v41flash_csa2_decode_1m_fp4,v4pro_csa_decode_65k_mtp4",
                    help="comma-separated extra workloads measured into 'extra' ('none' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compressor-bulk", action="store_true")
    ap.add_argument("--no-out-proj", action="store_true", help="skip the output projection's own timing")
    ap.add_argument("--no-achievable", action="store_true", help="skip the measured HBM / GEMM ceilings")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run only the hardware-counter workload (calibration copy + eager steps) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the library runs the path on one GPU only; --gpus must be 1 "
                                   "(sharding across GPUs is not implemented)"}))
        sys.exit(2)

    import torch
    import csa_inputs as ci
    from compressed_attention_long_amd import _lib
    _lib.load()                       # fails loudly when the HIP library is missing
    assert torch.cuda.is_available(), "no GPU visible"

    wl = ci.WORKLOADS[args.workload]
    if args.pmc_probe:
        pmc_probe(wl, torch)
        return
    print(f"[bench] workload {wl.name}: timing {args.steps} steps after {args.warmup} warmup", file=sys.stderr,
          flush=True)
    tm = time_workload(wl, args.steps, args.warmup, torch)
    costs = algorithmic_costs(wl)
    ms = tm["wall_ms_per_step"]
    tokens = wl.B * wl.Tq
    value = tokens / (ms / 1e3)
    calls = {}
    for name in ("compress", "index", "index_compress", "attend"):
        if name not in tm["calls_graph"]:
            continue
        t_ms = tm["calls_graph"][name]
        d = {"ms": t_ms, "eager_event_ms": tm.get(name)}
        if name == "index_compress":
            d["GB_per_s"] = (costs["index_bytes"] + costs["compress_bytes"]) / (t_ms * 1e-3) / 1e9
            d["hbm_frac"] = d["GB_per_s"] / HBM_PEAK_GBS
            calls[name] = d
            continue
        if f"{name}_bytes" in costs:
            d["GB_per_s"] = costs[f"{name}_bytes"] / (t_ms * 1e-3) / 1e9
            d["hbm_frac"] = d["GB_per_s"] / HBM_PEAK_GBS
        if f"{name}_flops" in costs:
            d["TFLOP_per_s"] = costs[f"{name}_flops"] / (t_ms * 1e-3) / 1e12
            d["mfma_frac"] = d["TFLOP_per_s"] / BF16_PEAK_TFLOPS
        calls[name] = d
    # dominant call of the step.  Attention (and the indexer of several query tokens per sequence,
    # whose keys cross HBM once per sequence) is a dense contraction: its roofline is bf16 MFMA;
    # the one-token decode indexer and the compressor stream HBM.
    dom = max((k for k in calls if k != "index_compress"), key=lambda k: calls[k]["ms"])
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if dom == "attend" or (dom == "index" and wl.Tq > 1):
        att_k = "k_attend_grp" if wl.kv_dtype == "bf16" else "k_attend"
        kern = (f"{'csa_attend' if wl.mode == 'csa' else 'hca_attend'} ({att_k} + k_attend_combine)" if dom == "attend"
                else f"csa_index_topk ({'k_index_scores_mq' if wl.Tq >= 16 else 'k_index_scores'} + top-k)")
        intensity = costs[f"{dom}_flops"] / costs[f"{dom}_bytes"]
        roof = {"bound": "mfma", "achieved": calls[dom]["TFLOP_per_s"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": calls[dom]["mfma_frac"], "traffic": measured_traffic(wl.name, dom), "kernel": kern,
                "hbm_GB_per_s": calls[dom]["GB_per_s"], "hbm_frac": calls[dom]["hbm_frac"],
                "intensity_flop_per_byte": intensity, "ridge_flop_per_byte": ridge}
    else:
        roof = {"bound": "hbm", "achieved": calls[dom]["GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": calls[dom]["hbm_frac"], "traffic": measured_traffic(wl.name, dom),
                "kernel": "csa_index_topk (k_index_scores + k_topk)" if dom == "index" else "csa_compress"}
    for name in calls:
        if name in tm["calls_stats"]:
            calls[name]["stats"] = tm["calls_stats"][name]
    extra = {"calls": calls, "timing": "value = tokens / wall time of layer steps replayed from one HIP graph "
                                       "chaining the rotated layers; per_layer_graph = one graph launch per step; "
                                       "calls[*].ms = per C-ABI call, a HIP graph of that call over the rotated "
                                       "layers replayed between HIP events on the launch stream (average per call); "
                                       "calls[*].eager_event_ms = events around each call in an eager pass (host "
                                       "launch gaps included)",
             "graph_gpu_ms_per_step": tm["graph_gpu_ms_per_step"], "eager_wall_ms_per_step": tm["eager_wall_ms_per_step"],
             "per_layer_graph_ms_per_step": tm["per_layer_graph_wall_ms_per_step"],
             "step_gpu_ms": tm["step_gpu"], "step_gpu_median_ms": tm["step_gpu_median"],
             "step_stats": tm["step_stats"],
             "layers_rotated": tm["layers"], "pages_config_context": {
                 "layers": 61, "csa_layers": 30, "hca_layers": 31, "heads": 128, "head_dim": 512,
                 "index_topk": 1024, "sliding_window": 128}}
    for name in [x for x in args.extra.split(",") if x and x != "none"]:
        w2 = ci.WORKLOADS[name]
        print(f"[bench] extra workload {name}", file=sys.stderr, flush=True)
        t2 = time_workload(w2, max(10, args.steps // 2), args.warmup, torch)
        c2 = algorithmic_costs(w2)
        cg2 = t2["calls_graph"]
        e2 = {"ms_per_step": t2["wall_ms_per_step"], "tokens_per_s": w2.B * w2.Tq / (t2["wall_ms_per_step"] / 1e3),
              "attend_ms": cg2["attend"], "attend_TFLOP_per_s": c2["attend_flops"] / (cg2["attend"] * 1e-3) / 1e12,
              "attend_GB_per_s": c2["attend_bytes"] / (cg2["attend"] * 1e-3) / 1e9, "compress_ms": cg2["compress"]}
        e2["attend_mfma_frac"] = e2["attend_TFLOP_per_s"] / BF16_PEAK_TFLOPS
        e2["step_stats"] = t2["step_stats"]
        e2["attend_stats"] = t2["calls_stats"]["attend"]
        if w2.mode == "csa":
            e2["index_ms"] = cg2["index"]
            e2["index_stats"] = t2["calls_stats"]["index"]
            if w2.Tq > 1:
                # several query tokens per sequence score the same keys, which cross HBM once per
                # sequence (prefill: once per chunk): a contraction, reported against bf16 MFMA with
                # its HBM rate beside
                e2["index_TFLOP_per_s"] = c2["index_flops"] / (cg2["index"] * 1e-3) / 1e12
                e2["index_mfma_frac"] = e2["index_TFLOP_per_s"] / BF16_PEAK_TFLOPS
            e2["index_GB_per_s"] = c2["index_bytes"] / (cg2["index"] * 1e-3) / 1e9
            e2["index_hbm_frac"] = e2["index_GB_per_s"] / HBM_PEAK_GBS
            e2["index_compress_ms"] = cg2["index_compress"]
        if w2.reuse > 0:
            tr = time_reuse(w2, max(10, args.steps // 2), args.warmup, torch)
            avg = (t2["wall_ms_per_step"] + w2.reuse * tr) / (1 + w2.reuse)
            e2.update({"reuse_ms_per_step": tr, "reuse_layers_per_computed": w2.reuse, "layer_avg_ms": avg,
                       "tokens_per_s_layer_avg": w2.B * w2.Tq / (avg / 1e3)})
        extra[name] = e2
    if not args.no_out_proj:
        print("[bench] output projection (decode batch)", file=sys.stderr, flush=True)
        extra["out_projection"] = out_projection_bench(torch)
    if not args.no_compressor_bulk:
        print("[bench] compressor over whole raw streams", file=sys.stderr, flush=True)
        extra["compressor_bulk"] = compressor_bulk(torch)
    if not args.no_achievable:
        print("[bench] measured ceilings", file=sys.stderr, flush=True)
        extra["achievable_peaks"] = achievable_peaks(torch)
    base = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        base = cpu_baseline(wl, args.cpu_budget)
        # the oracle on the other workloads, each on a bounded sample (tokens/s, cores stated)
        others = {}
        for name, budget, threads, max_rows in [("tiny_csa_decode", 3.0, None, None), ("tiny_csa_decode", 3.0, 1, None),
                                                ("v4pro_hca_decode_1m", 4.0, None, None),
                                                ("v4flash_csa_decode_1m_fp8", 6.0, None, None),
                                                ("v4pro_csa_prefill_4k_on_131k", 6.0, None, 64)]:
            if name == wl.name and threads is None:
                continue
            print(f"[bench] cpu oracle {name} threads={threads or 'all'}", file=sys.stderr, flush=True)
            key = name + ("_single_thread" if threads == 1 else "")
            others[key] = cpu_baseline(ci.WORKLOADS[name], budget, threads=threads, max_rows=max_rows)
        extra["cpu_oracle"] = others
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; fp8 indexer keys; caches rotated over distinct layers)",
        "config": {"workload": wl.name, "batch": wl.B, "context": wl.N, "query_heads": wl.H, "head_dim": wl.D,
                   "index_heads": wl.Hi, "index_dim": wl.Di, "topk": wl.topk, "window": wl.W,
                   "kv_dtype": wl.kv_dtype, "index_key_dtype": wl.idx_dtype, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": base,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

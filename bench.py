#!/usr/bin/env python3
"""Benchmark of the TurboQuant hot path on one MI355X.

Default workload: the Llama-70B-shaped cache (80 layers, 8 KV heads, 64 query heads, head_dim 128, batch 4,
131072 cached tokens per sequence; layers 0, 1, 78 and 79 with K and V at 8 bits, the others K 4-bit / V 2-bit,
MSE; 16-token pages with a shuffled page table; bf16 inputs). Every layer has its own page pool (36 GB in all),
filled by a 131072-token prefill quantize-on-write per sequence; one step is one decode step of the whole model:
for every layer, the new token of every sequence is quantized into its slot and the new queries attend over every
cached token (tq_decode_step: the split-K launch with the append fused, plus the merge; 8-bit layers:
tq_quantize_kv + tq_decode_attention). The timed region replays the K steps as one HIP graph.

Prints one JSON line. ``value`` is the step's algorithmic bytes (the compressed records of every cached token of
every layer and KV head, the new tokens' K/V input, page ids) divided by the wall time of the K steps, in GB/s;
``roofline`` is the split-K launch of the K4/V2 layers (algorithmic bytes per launch / its average duration from
HIP events around a graph of those launches alone), with its HBM traffic from committed rocprofv3 counter runs
while the kernel source is unchanged; ``quantize`` reports the prefill's quantize-on-write (a K4/V2 layer and an
8-bit layer: vectors/s and bytes in + out against the HBM peak); ``stream_read`` is a plain streaming read of a
large buffer, the practical ceiling; ``step_breakdown`` sums the launches of one step timed by kind;
``cpu_baseline`` times the CPU oracle on a bounded sample of the same cache. ``secondary`` holds the Llama-3.1-8B
single-layer line (``--workload 1`` prints it as the main line): one layer, batch 1, 32768 tokens, cycled through
16 cache copies so that every step's bytes come from HBM, with the uncompressed comparators and the chunked
prefill leg.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
QREPS = 4                  # prefill quantize launches timed back to back per format
WORKLOAD_INDEX = 4         # the headline workload: the largest one that fits one GPU (Llama-70B shape)
SINGLE_LAYER_INDEX = 1     # the Llama-3.1-8B single layer (secondary line)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the decode kernel's sources and of the build recipe (its compile flags)."""
    h = hashlib.sha256()
    for f in ("tq_decode.hip", "tq_common.h", "tq_quant_common.h", "tq_lanes.h", "tq_operands.h"):
        with open(os.path.join(ROOT, "kv_cache_quantization_wht_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "kv_cache_quantization_wht_amd", "build.py"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def prefill_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("tq_prefill.hip", "tq_common.h", "tq_lanes.h", "tq_operands.h"):
        with open(os.path.join(ROOT, "kv_cache_quantization_wht_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def quantize_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("tq_quantize.hip", "tq_common.h", "tq_quant_common.h"):
        with open(os.path.join(ROOT, "kv_cache_quantization_wht_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(name, source_hash, key="hbm_bytes_per_launch"):
    """HBM traffic of a kernel from committed rocprofv3 counter runs (``profiles/<name>``), if they were taken on
    the current source of that kernel; else None."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != source_hash:
        return None
    return t.get(key)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: the workload's own, 64 for the 70B shape, 128 for the 8B layer)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (default 2; 8B layer: 16)")
    ap.add_argument("--copies", type=int, default=16, help="8B single layer: independent layer caches cycled per step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the uncompressed bf16 and FP8 comparators")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill leg")
    ap.add_argument("--no-secondary", action="store_true", help="skip the 8B single-layer line after the headline")
    ap.add_argument("--eager", action="store_true", help="8B layer: launch steps from Python instead of a graph")
    ap.add_argument("--workload", default=None,
                    help="workload by name or index (default: the Llama-70B shape, index 4); index 1, the 8B "
                         "single layer, prints that line as the main one")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="only run a plain device-to-device copy of MB megabytes (5 times), to scale the HBM "
                         "byte counters of rocprofv3")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch

        n = args.calibrate_copy * 1000 * 1000
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "copies": 5}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this hot path is measured on one GPU only; multi-GPU runs are not part of it "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import torch

    import kvsynth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    wi = WORKLOAD_INDEX
    if args.workload is not None:
        names = [w.name for w in kvsynth.workloads()]
        wi = int(args.workload) if args.workload.isdigit() else names.index(args.workload)
    if wi == SINGLE_LAYER_INDEX:
        result = single_layer(args, args.steps if args.steps is not None else 128,
                              args.warmup if args.warmup is not None else 16, cpu=not args.no_cpu_baseline)
    else:
        result = run_workload(args, wi)
        torch.cuda.empty_cache()
        if not args.no_secondary:
            sec = single_layer(args, 128, 16, cpu=False)
            result["secondary"] = {sec["config"]["workload"]: sec}
    print(json.dumps(result), flush=True)


def single_layer(args, K, W, cpu=True):
    """The Llama-3.1-8B single-layer line: one decode step = tq_decode_step of the new token over 32768 cached
    tokens of one layer (batch 1), the layer cycled through ``--copies`` independent caches."""
    import torch

    import kvsynth
    import kv_cache_quantization_wht_amd as tq

    dev = "cuda"
    wl = kvsynth.workloads()[SINGLE_LAYER_INDEX]
    H, Hq, d, T = wl.kv_heads, wl.q_heads, wl.head_dim, wl.seq_len
    bits = wl.bits[0]
    layout = tq.Layout(d, H, bits.k_bits, bits.k_mode, bits.v_bits, bits.v_mode)
    offs = tq.page_layout(layout)
    page_bytes = offs["page_bytes"]
    C = args.copies
    total_steps = W + K
    max_len = T + (total_steps + C - 1) // C + 1
    pages_per_copy = (max_len + 15) // 16
    num_pages = C * pages_per_copy
    log(f"workload {wl.name}: page {page_bytes} B, {C} copies x {pages_per_copy} pages = "
        f"{num_pages * page_bytes / 1e6:.1f} MB")

    sw = kvsynth.rotation_signs(kvsynth.rotation_seed(0), d)
    kcb = torch.from_numpy(tq.build_codebook(d, bits.k_bits, bits.k_mode, sw)).to(dev)
    vcb = torch.from_numpy(tq.build_codebook(d, bits.v_bits, bits.v_mode, sw)).to(dev)
    pages = torch.zeros(num_pages * page_bytes, dtype=torch.uint8, device=dev)
    page_tables = [torch.arange(c * pages_per_copy, (c + 1) * pages_per_copy, dtype=torch.int32, device=dev)[None]
                   for c in range(C)]

    # ---- prefill: quantize T tokens into every copy (timed on copy 0 for the quantize rate)
    k_pre, v_pre = kvsynth.make_kv(wl, SINGLE_LAYER_INDEX, 0, T, device=dev)
    slots0 = torch.arange(T, dtype=torch.int64, device=dev)
    # one launch, then 8 more back to back with an event between each two: the median launch interval
    tq.quantize_kv(layout, pages, k_pre, v_pre, slots0, kcb, vcb)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(9)]
    ev[0].record()
    for rep in range(8):
        tq.quantize_kv(layout, pages, k_pre, v_pre, slots0, kcb, vcb)
        ev[rep + 1].record()
    torch.cuda.synchronize()
    q_time = float(np.median([ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(8)]))
    n_vec = T * H * 2
    quant_vps = n_vec / q_time
    for c in range(1, C):
        tq.quantize_kv(layout, pages, k_pre, v_pre, slots0 + c * pages_per_copy * 16, kcb, vcb)
    torch.cuda.synchronize()
    log(f"prefill quantize: {n_vec} vectors in {q_time * 1e6:.1f} us -> {quant_vps / 1e9:.2f} G vectors/s")

    # ---- per-step inputs: new token K/V, query, slot, sequence length (all resident before timing)
    k_new, v_new = kvsynth.make_kv(wl, SINGLE_LAYER_INDEX, 0, total_steps, device=dev, token_offset_seed=1)
    g = torch.Generator(device=dev).manual_seed(kvsynth.data_seed(SINGLE_LAYER_INDEX, 0, "q"))
    qs = torch.randn(total_steps, 1, Hq, d, generator=g, device=dev).to(torch.bfloat16)
    lens = [T] * C
    step_slots, step_lens, step_copy, step_bytes = [], [], [], []
    rec_bytes = offs["k_norms"] // (H * 16) + 2 + (offs["v_norms"] - offs["v_codes"]) // (H * 16) + 2
    for i in range(total_steps):
        c = i % C
        t = lens[c]
        step_slots.append(torch.tensor([(c * pages_per_copy + t // 16) * 16 + t % 16], dtype=torch.int64, device=dev))
        lens[c] = t + 1
        step_lens.append(torch.tensor([t + 1], dtype=torch.int32, device=dev))
        step_copy.append(c)
        # records of every cached token (t read, the new one written), the new token's K/V input, page ids
        step_bytes.append(H * (t + 1) * rec_bytes + H * 2 * d * 2 + 4 * ((t + 1 + 15) // 16))
    ws_bytes = tq.decode_workspace_bytes(layout, 1, Hq, pages_per_copy)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty(1, Hq, d, dtype=torch.float32, device=dev)
    scale = wl.softmax_scale

    def step(i):
        # one decode step: the new token's K and V are quantized into their slot and the new query attends
        # over every cached token, in one split-K launch (tq_decode_step_partial) plus the merge
        # (tq_decode_combine); tq_decode_step is exactly that pair
        tq.decode_step(layout, pages, k_new[i:i + 1], v_new[i:i + 1], qs[i], page_tables[step_copy[i]], step_lens[i],
                       scale, kcb, vcb, workspace=ws, out=out)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    mode = "eager" if args.eager else "graph"
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(W, total_steps):
                step(i)
        torch.cuda.synchronize()

    # ---- timed region: exactly K steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(W, total_steps):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / K
    bytes_timed = float(np.sum(step_bytes[W:]))
    value = bytes_timed / elapsed / 1e9

    # ---- split-K kernel and merge durations: HIP events on the launch stream around a graph of the K launches
    def partial_only(i):
        tq.decode_step(layout, pages, k_new[i:i + 1], v_new[i:i + 1], qs[i], page_tables[step_copy[i]], step_lens[i],
                       scale, kcb, vcb, workspace=ws, out=out, first_pass_only=True)

    def combine_only(i):
        tq.decode_combine(layout, pages, qs[i], page_tables[step_copy[i]], step_lens[i], scale, kcb, vcb, ws, out=out)

    kmode = "graph of the K launches, one event pair"
    kern_s = graph_avg(lambda: [partial_only(i) for i in range(W, total_steps)], K)
    comb_s = graph_avg(lambda: [combine_only(i) for i in range(W, total_steps)], K)
    alg_per_launch = float(np.mean(step_bytes[W:]))
    achieved = alg_per_launch / kern_s / 1e9
    traffic = load_traffic("decode_traffic.json", kernel_source_hash())
    log(f"step {ms_per_step * 1e3:.2f} us ({mode}); split-K decode kernel {kern_s * 1e6:.2f} us, combine "
        f"{comb_s * 1e6:.2f} us ({kmode}); {alg_per_launch / 1e6:.2f} MB/launch -> {achieved:.0f} GB/s")

    result = {
        "metric": "decode-attn compressed-KV GB/s (% of HBM peak); KV quantize vectors/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16-mfma+fp32",
        "data": "synthetic",
        "config": {"workload": wl.name, "kv_heads": H, "q_heads": Hq, "head_dim": d, "batch": 1,
                   "seq_len": T, "k_bits": bits.k_bits, "v_bits": bits.v_bits, "mode": "mse",
                   "page_tokens": 16, "cache_copies": C, "launch": mode},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "quantize_vectors_per_s": round(quant_vps, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_kernel<128,4,false,2,true,true> (tq_decode_step_partial)",
                     "bytes_per_launch": round(alg_per_launch), "avg_launch_us": round(kern_s * 1e6, 3),
                     "combine_avg_us": round(comb_s * 1e6, 3), "timing": kmode},
        "cpu_baseline": None,
    }

    if not args.no_dense:
        result["dense_bf16"] = dense_comparator(wl, k_pre, v_pre, k_new, v_new, qs, W, K, ms_per_step, step_bytes)
        result["dense_fp8"] = dense_comparator(wl, k_pre, v_pre, k_new, v_new, qs, W, K, ms_per_step, step_bytes,
                                               fmt="fp8")
    if not args.no_prefill:
        result["prefill"] = prefill_leg(wl, layout, pages, page_tables[0], k_pre, v_pre, kcb, vcb)
        result["prefill_k2qjl"] = prefill_sketched(wl, k_pre, v_pre, sw)
    if cpu:
        first = int(page_tables[0][0, 0].item())
        npg = (T + 15) // 16
        pool = pages[first * page_bytes:(first + npg) * page_bytes].cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(H, d, bits, pool, T, qs.double().cpu().numpy(), scale, sw, None,
                                              args.cpu_seconds, rec_bytes, "copy 0")
    return result


def graph_avg(launch_all, n):
    """Average duration of ``n`` launches: they are captured into one graph (no other kernel between them),
    replayed once to warm up, then once between two HIP events on the launch stream (events recorded inside a
    captured graph are not timed on this platform)."""
    import torch

    gph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gph):
        launch_all()
    gph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    gph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / n


def prefill_leg(wl, layout, pages, page_table, k_pre, v_pre, kcb, vcb, chunk=2048, reps=8):
    """The last ``chunk`` tokens of the layer's prompt as one prefill chunk over the packed cache of copy 0
    (prefix T - chunk cached tokens): tq_prefill_attention alone (its kernel, from HIP events around a graph of
    ``reps`` launches) and tq_prefill_chunk (quantize of the chunk's K/V into their slots, which rewrites the
    same bytes, plus the attention). Algorithmic work: 4 * d flops per (query head, visible key) pair - the
    q.k and p.v products - over the causal pairs; the kernel runs each product as fp16 hi + lo MFMA pairs,
    so the matrix cores issue twice these flops."""
    import torch

    import kv_cache_quantization_wht_amd as tq

    dev = "cuda"
    H, Hq, d, T = wl.kv_heads, wl.q_heads, wl.head_dim, wl.seq_len
    P = T - chunk
    g = torch.Generator(device=dev).manual_seed(kvsynth_seed_q())
    q = torch.randn(1, chunk, Hq, d, generator=g, device=dev).to(torch.bfloat16)
    prefix = torch.tensor([P], dtype=torch.int32, device=dev)
    first = int(page_table[0, 0].item())
    slots = (first * 16 + torch.arange(P, T, dtype=torch.int64, device=dev))
    kc, vc = k_pre[P:T].unsqueeze(0).contiguous(), v_pre[P:T].unsqueeze(0).contiguous()
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)

    def attn():
        tq.prefill_attention(layout, pages, q, page_table, prefix, wl.softmax_scale, kcb, vcb, out=out)

    def fused():
        tq.prefill_chunk(layout, pages, kc, vc, slots, q, page_table, prefix, wl.softmax_scale, kcb, vcb, out=out)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            for _ in range(reps):
                fn()
        gph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_attn = timed(attn)
    t_fused = timed(fused)
    pairs = chunk * P + chunk * (chunk + 1) // 2  # (query token, visible key) pairs per query head
    flops = 4.0 * d * Hq * pairs
    tflops = flops / t_attn / 1e12
    peak = 2500.0
    log(f"prefill: chunk {chunk} after {P} cached tokens: attention kernel {t_attn * 1e6:.1f} us "
        f"({tflops:.0f} TFLOP/s algorithmic, {100 * tflops / peak:.1f}% of fp16 MFMA peak); with the chunk's "
        f"quantize {t_fused * 1e6:.1f} us -> {chunk / t_fused:.0f} tokens/s")
    return {"chunk": chunk, "prefix": P, "attn_us": round(t_attn * 1e6, 2), "chunk_us": round(t_fused * 1e6, 2),
            "tokens_per_s": round(chunk / t_fused, 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(tflops / peak, 4), "traffic": load_traffic("prefill_traffic.json", prefill_source_hash()),
                         "flops_per_launch": flops,
                         "kernel": "prefill_kernel<128,4,false,2> (tq_prefill_attention)", "mfma_issue_factor": 2},
            "what": "tq_prefill_attention / tq_prefill_chunk of the last 2048 prompt tokens of the 8B layer, "
                    "HIP events around a graph of 8 launches"}


def prefill_sketched(wl, k_pre, v_pre, sw, chunk=2048, reps=8):
    """The same chunk over a cache of the layer's K/V with a sketched K (K2 + QJL / V2, prod mode: 1-bit levels and
    the 1-bit residual sketch): one cache, prefilled by tq_quantize_kv, tq_prefill_attention timed as in
    prefill_leg. Algorithmic flops: 6 d per (query head, visible key) pair (q.k, the sketch term q_s.z, p.v)."""
    import torch

    import kvsynth
    import kv_cache_quantization_wht_amd as tq

    dev = "cuda"
    H, Hq, d, T = wl.kv_heads, wl.q_heads, wl.head_dim, wl.seq_len
    P = T - chunk
    layout = tq.Layout(d, H, 2, 1, 2, 0)
    S = kvsynth.qjl_projection(kvsynth.rotation_seed(0), d)
    kcb = torch.from_numpy(tq.build_codebook(d, 2, 1, sw, S)).to(dev)
    vcb = torch.from_numpy(tq.build_codebook(d, 2, 0, sw)).to(dev)
    pages = torch.zeros((T // 16) * tq.page_layout(layout)["page_bytes"], dtype=torch.uint8, device=dev)
    tq.quantize_kv(layout, pages, k_pre, v_pre, torch.arange(T, dtype=torch.int64, device=dev), kcb, vcb)
    pt = torch.arange(T // 16, dtype=torch.int32, device=dev)[None]
    g = torch.Generator(device=dev).manual_seed(kvsynth_seed_q())
    q = torch.randn(1, chunk, Hq, d, generator=g, device=dev).to(torch.bfloat16)
    prefix = torch.tensor([P], dtype=torch.int32, device=dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)

    def attn():
        tq.prefill_attention(layout, pages, q, pt, prefix, wl.softmax_scale, kcb, vcb, out=out)

    attn()
    torch.cuda.synchronize()
    gph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gph):
        for _ in range(reps):
            attn()
    gph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    gph.replay()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    pairs = chunk * P + chunk * (chunk + 1) // 2
    flops = 6.0 * d * Hq * pairs
    log(f"prefill, sketched K (K2+QJL/V2): attention kernel {t * 1e6:.1f} us ({flops / t / 1e12:.0f} TFLOP/s "
        f"algorithmic)")
    return {"chunk": chunk, "prefix": P, "attn_us": round(t * 1e6, 2), "tflops": round(flops / t / 1e12, 1),
            "kernel": "prefill_kernel<128,1,true,2> (tq_prefill_attention)",
            "what": "tq_prefill_attention of the last 2048 prompt tokens over a K2+QJL/V2 cache of the 8B layer, "
                    "HIP events around a graph of 8 launches"}


def kvsynth_seed_q():
    import kvsynth

    return kvsynth.data_seed(SINGLE_LAYER_INDEX, 0, "q") + 17


def dense_comparator(wl, k_pre, v_pre, k_new, v_new, qs, W, K, ms_compressed, step_bytes, fmt="bf16"):
    """The same decode steps over an uncompressed cache of the layer, bf16 or FP8 E4M3 (one scale per tensor,
    amax / 448 of the prefilled K and V): per step, the new token's K/V is written into its slot
    (tq_dense_write_kv / tq_dense_fp8_write_kv) and the new query attends over every cached token
    (tq_dense_decode_attention / tq_dense_fp8_decode_attention: split-K launch + merge). 4 copies of the
    layer cache (4 x 134 MB in bf16, more than the Infinity Cache) are cycled as for the compressed cache;
    the K steps replay as one HIP graph."""
    import torch

    import kv_cache_quantization_wht_amd as tq

    dev = "cuda"
    H, Hq, d, T = wl.kv_heads, wl.q_heads, wl.head_dim, wl.seq_len
    C = 4
    total = W + K
    ppc = (T + (total + C - 1) // C + 1 + 15) // 16
    fp8 = fmt == "fp8"
    elem = 1 if fp8 else 2
    ks, vs = (k_pre.abs().max().item() / 448.0, v_pre.abs().max().item() / 448.0) if fp8 else (1.0, 1.0)
    pb = tq.dense_fp8_page_bytes(d, H) if fp8 else tq.dense_page_bytes(d, H)
    pages = torch.zeros(C * ppc * pb, dtype=torch.uint8, device=dev)
    slots0 = torch.arange(T, dtype=torch.int64, device=dev)

    def write(k, v, slots):
        if fp8:
            tq.dense_fp8_write_kv(d, H, pages, k, v, slots, ks, vs)
        else:
            tq.dense_write_kv(d, H, pages, k, v, slots)

    for c in range(C):
        write(k_pre, v_pre, slots0 + c * ppc * 16)
    pts = [torch.arange(c * ppc, (c + 1) * ppc, dtype=torch.int32, device=dev)[None] for c in range(C)]
    lens = [T] * C
    st_slots, st_lens, st_copy, st_bytes = [], [], [], []
    for i in range(total):
        c = i % C
        t = lens[c]
        st_slots.append(torch.tensor([(c * ppc + t // 16) * 16 + t % 16], dtype=torch.int64, device=dev))
        lens[c] = t + 1
        st_lens.append(torch.tensor([t + 1], dtype=torch.int32, device=dev))
        st_copy.append(c)
        st_bytes.append(H * (t + 1) * d * elem * 2 + H * 2 * d * elem + 4 * ((t + 1 + 15) // 16))
    ws = torch.zeros(tq.dense_decode_workspace_bytes(d, H, 1, Hq, ppc), dtype=torch.uint8, device=dev)
    out = torch.empty(1, Hq, d, dtype=torch.float32, device=dev)

    def step(i):
        write(k_new[i:i + 1], v_new[i:i + 1], st_slots[i])
        if fp8:
            tq.dense_fp8_decode_attention(d, H, pages, qs[i], pts[st_copy[i]], st_lens[i], wl.softmax_scale, ks, vs,
                                          workspace=ws, out=out)
        else:
            tq.dense_decode_attention(d, H, pages, qs[i], pts[st_copy[i]], st_lens[i], wl.softmax_scale,
                                      workspace=ws, out=out)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(W, total):
            step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / K
    dense_bytes = float(np.mean(st_bytes[W:]))
    comp_bytes = float(np.mean(step_bytes[W:]))
    log(f"dense {fmt} comparator: step {ms * 1e3:.2f} us, {dense_bytes / 1e6:.1f} MB/step -> "
        f"{dense_bytes / (ms * 1e-3) / 1e9:.0f} GB/s; compressed step is {ms / ms_compressed:.2f}x faster "
        f"on {dense_bytes / comp_bytes:.2f}x fewer bytes")
    return {"ms_per_step": round(ms, 6), "bytes_per_step": round(dense_bytes),
            "gbs": round(dense_bytes / (ms * 1e-3) / 1e9, 1), "compressed_speedup": round(ms / ms_compressed, 3),
            "bytes_ratio": round(dense_bytes / comp_bytes, 3),
            "what": (f"tq_dense{'_fp8' if fp8 else ''}_write_kv + tq_dense{'_fp8' if fp8 else ''}_decode_attention "
                     f"per step over a{'n FP8 E4M3 (per-tensor scales)' if fp8 else ' bf16'} cache of the same layer "
                     "(4 cycled copies), one HIP graph of the K steps")}


def cpu_baseline(H, d, bits, pool, T, qall, scale, sw, S, budget_s, rec_bytes, what):
    """Time the CPU oracle's decode attention over one sequence's T cached tokens (``pool`` holds its pages in
    order): one KV head (its query heads) at a time, over successive decode queries, until the time budget is
    spent. ``qall`` is [queries, batch, Hq, d]; batch row 0 is used."""
    from oracle import attention, codec

    Lo = codec.page_layout(H, d, bits.k_bits, bits.k_mode, bits.v_bits, bits.v_mode)
    cbk = codec.make_codebook(d, bits.k_bits, bits.k_mode, sw, S)
    cbv = codec.make_codebook(d, bits.v_bits, bits.v_mode, sw, S if bits.v_mode else None)
    npg = (T + 15) // 16
    pt = np.arange(npg, dtype=np.int64)[None]
    G = qall.shape[2] // H
    done, t_used, step = 0, 0.0, 0
    t0 = time.perf_counter()
    while t_used < budget_s and step < qall.shape[0]:
        for g in range(H):
            heads = [(0, h) for h in range(g * G, (g + 1) * G)]
            attention.decode_attention(pool, Lo, cbk, cbv, qall[step][:1], pt, [T], scale, heads=heads)
            done += 1
            t_used = time.perf_counter() - t0
            if t_used > budget_s:
                break
        step += 1
    bytes_done = done * T * rec_bytes
    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = 1
    return {"value": round(bytes_done / t_used / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 oracle decode attention of {what} (T={T}, {H} KV heads x {G} query heads each): {done} "
                      f"(KV head, query) units over {step} decode queries in {t_used:.1f} s; same unit as value",
            "host_cpus": os.cpu_count()}


def record_bytes(offs, H):
    """Stored bytes of one token of one KV head (K and V records: codes, norms, sketch, gamma)."""
    return offs["page_bytes"] // (H * 16)


def run_workload(args, wi):
    """A multi-layer or batched workload: every layer has its own cache (no copies needed: the layers
    together exceed the Infinity Cache), prefilled through tq_quantize_kv; one step is one decode step of
    the whole model: for every layer, the new token of every sequence is quantized into its slot and the
    new queries attend (tq_decode_step where the format allows, tq_quantize_kv + tq_decode_attention for
    prod K or 8-bit codes). The timed region replays the K steps as one HIP graph."""
    import torch

    import kvsynth
    import kv_cache_quantization_wht_amd as tq

    dev = "cuda"
    wl = kvsynth.workloads()[wi]
    L, H, Hq, d, B, T = wl.layers, wl.kv_heads, wl.q_heads, wl.head_dim, wl.batch, wl.seq_len
    K = args.steps if args.steps is not None else wl.decode_steps
    W = args.warmup if args.warmup is not None else 2
    total = W + K
    pps = (T + total + 15) // 16
    layers = []
    for l in range(L):
        bits = wl.bits[l]
        layout = tq.Layout(d, H, bits.k_bits, bits.k_mode, bits.v_bits, bits.v_mode)
        offs = tq.page_layout(layout)
        pt, npages = kvsynth.page_table(B, pps, wl.shuffled_pages, seed=4242 + l)
        sw = kvsynth.rotation_signs(kvsynth.rotation_seed(l), d)
        S = kvsynth.qjl_projection(kvsynth.rotation_seed(l), d) if bits.k_mode or bits.v_mode else None
        layers.append(dict(bits=bits, layout=layout, offs=offs, pt=pt, ptd=torch.from_numpy(pt).to(dev), sw=sw, S=S,
                           kcb=torch.from_numpy(tq.build_codebook(d, bits.k_bits, bits.k_mode, sw, S)).to(dev),
                           vcb=torch.from_numpy(tq.build_codebook(d, bits.v_bits, bits.v_mode, sw, S)).to(dev),
                           pages=torch.zeros(npages * offs["page_bytes"], dtype=torch.uint8, device=dev),
                           fused=not bits.k_mode and not bits.v_mode and bits.k_bits <= 4 and bits.v_bits <= 4))
    total_mb = sum(x["pages"].numel() for x in layers) / 1e6
    log(f"workload {wl.name}: {L} layers, batch {B}, {T} cached tokens, {total_mb:.0f} MB of pages")

    def fmt_of(x):
        b0 = x["bits"]
        return f"K{b0.k_bits}{'qjl' if b0.k_mode else ''}/V{b0.v_bits}{'qjl' if b0.v_mode else ''}"

    # ---- prefill every layer (all sequences of a layer in one launch). The first layer of each format is timed
    #      (4 more launches back to back, HIP events between them on the launch stream, the median launch): the
    #      quantize-on-write rate and its bytes
    prefill_t = {}
    for l, x in enumerate(layers):
        k, v = kvsynth.make_kv(wl, wi, l, B * T, device=dev)
        sl_all = torch.from_numpy(np.concatenate([kvsynth.slots_for(x["pt"], b, 0, T) for b in range(B)])).to(dev)
        f = fmt_of(x)
        tq.quantize_kv(x["layout"], x["pages"], k, v, sl_all, x["kcb"], x["vcb"])
        if f not in prefill_t:
            # the same launch QREPS more times back to back (it writes the same bytes again), an event between each
            # two: the median of the launch intervals
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(QREPS + 1)]
            ev[0].record()
            for i in range(QREPS):
                tq.quantize_kv(x["layout"], x["pages"], k, v, sl_all, x["kcb"], x["vcb"])
                ev[i + 1].record()
            torch.cuda.synchronize()
            prefill_t[f] = (l, float(np.median([ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(QREPS)])))
        del k, v, sl_all
        if l % 16 == 15:
            log(f"  prefilled {l + 1} layers")
    torch.cuda.synchronize()
    quantize = {}
    n_vec = B * T * H * 2
    for f, (l, t) in prefill_t.items():
        x = layers[l]
        rec = record_bytes(x["offs"], H)  # K + V record bytes of one token of one KV head
        bytes_io = B * T * H * (2 * d * 2 + rec)
        gbs = bytes_io / t / 1e9
        quantize[f] = {"layer": l, "vectors": n_vec, "avg_launch_us": round(t * 1e6, 2),
                       "vectors_per_s": round(n_vec / t, 1),
                       "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": bytes_io,
                                    "traffic": load_traffic("quantize_traffic.json", quantize_source_hash(),
                                                            key=f"hbm_bytes_per_launch_{f.replace('/', '')}"),
                                    "kernel": ("quantize_wide_kernel" if x["bits"].k_bits == 8 else "quantize_kernel")
                                              + " (tq_quantize_kv)",
                                    "bytes": "bf16 K and V in (2 x 256 B per token and KV head) + their records out"}}
        log(f"prefill quantize {f} (layer {l}, {n_vec} vectors): {t * 1e6:.0f} us -> {n_vec / t / 1e9:.2f} G vectors/s, "
            f"{gbs:.0f} GB/s in + out ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak)")

    # ---- per-step inputs, resident before timing
    news = [kvsynth.make_kv(wl, wi, l, total * B, device=dev, token_offset_seed=1) for l in range(L)]
    qs = [kvsynth.make_q(wl, wi, l, total * B, device=dev).view(total, B, Hq, d) for l in range(L)]
    lens = [torch.full((B,), T + i + 1, dtype=torch.int32, device=dev) for i in range(total)]
    step_slots = [[torch.from_numpy(x["pt"][:, (T + i) // 16].astype(np.int64) * 16 + (T + i) % 16).to(dev)
                   for i in range(total)] for x in layers]
    wss = {}
    for x in layers:
        key = (x["bits"].k_bits, x["bits"].k_mode, x["bits"].v_bits, x["bits"].v_mode)
        if key not in wss:
            wss[key] = torch.zeros(tq.decode_workspace_bytes(x["layout"], B, Hq, pps), dtype=torch.uint8, device=dev)
        x["ws"] = wss[key]
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    scale = wl.softmax_scale

    def layer_bytes(x, i):
        """Algorithmic bytes of layer x at step i: records of the T + i + 1 cached tokens (the new one written),
        the new tokens' K/V input, page ids."""
        return B * H * (T + i + 1) * record_bytes(x["offs"], H) + B * H * 2 * d * 2 + 4 * B * ((T + i + 1 + 15) // 16)

    step_bytes = [sum(layer_bytes(x, i) for x in layers) for i in range(total)]

    def layer_step(l, i, part="all"):
        """part: all (the layer's whole step), scan (its split-K launch alone), combine (its merge launch alone),
        append (the separate quantize launch of a layer outside the fused step)."""
        x = layers[l]
        kn, vn = news[l][0][i * B:(i + 1) * B], news[l][1][i * B:(i + 1) * B]
        if part == "combine":
            tq.decode_combine(x["layout"], x["pages"], qs[l][i], x["ptd"], lens[i], scale, x["kcb"], x["vcb"],
                              x["ws"], out=out)
        elif x["fused"]:
            if part in ("all", "scan"):
                tq.decode_step(x["layout"], x["pages"], kn, vn, qs[l][i], x["ptd"], lens[i], scale, x["kcb"],
                               x["vcb"], workspace=x["ws"], out=out, first_pass_only=part == "scan")
        else:
            if part in ("all", "append"):
                tq.quantize_kv(x["layout"], x["pages"], kn, vn, step_slots[l][i], x["kcb"], x["vcb"])
            if part == "all":
                tq.decode_attention(x["layout"], x["pages"], qs[l][i], x["ptd"], lens[i], scale, x["kcb"], x["vcb"],
                                    workspace=x["ws"], out=out)
            elif part == "scan":
                tq.decode_partial(x["layout"], x["pages"], qs[l][i], x["ptd"], lens[i], scale, x["kcb"], x["vcb"],
                                  x["ws"], out=out)

    def step(i):
        for l in range(L):
            layer_step(l, i)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(W, total):
            step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / K
    value = float(np.sum(step_bytes[W:])) / elapsed / 1e9
    del graph

    # ---- the launches of one step timed by kind (graphs of that kind alone, every layer of the kind in step order,
    #      HIP events around one replay): the split-K launch of each format, the merges, the 8-bit layers' appends.
    #      The K4/V2 split-K launch is the roofline kernel.
    fmts = sorted(set(fmt_of(x) for x in layers), key=lambda f: -sum(fmt_of(x) == f for x in layers))
    breakdown = {}
    for f in fmts:
        ls = [l for l, x in enumerate(layers) if fmt_of(x) == f]
        n = len(ls) * K
        t_scan = graph_avg(lambda: [layer_step(l, i, "scan") for i in range(W, total) for l in ls], n)
        t_comb = graph_avg(lambda: [layer_step(l, i, "combine") for i in range(W, total) for l in ls], n)
        ent = {"layers": len(ls), "scan_avg_us": round(t_scan * 1e6, 3), "combine_avg_us": round(t_comb * 1e6, 3),
               "scan_bytes_avg": round(float(np.mean([layer_bytes(layers[l], i) if layers[l]["fused"] else
                                                      layer_bytes(layers[l], i) - B * H * 2 * d * 2
                                                      for i in range(W, total) for l in ls])))}
        if not layers[ls[0]]["fused"]:
            ent["append_avg_us"] = round(graph_avg(lambda: [layer_step(l, i, "append") for i in range(W, total)
                                                          for l in ls], n) * 1e6, 3)
        ent["scan_gbs"] = round(ent["scan_bytes_avg"] / t_scan / 1e9, 1)
        breakdown[f] = ent
        log(f"  {f}: {len(ls)} layers, split-K launch {t_scan * 1e6:.2f} us ({ent['scan_gbs']:.0f} GB/s), merge "
            f"{t_comb * 1e6:.2f} us" + (f", append {ent['append_avg_us']:.2f} us" if "append_avg_us" in ent else ""))
    parts_us = sum(e["layers"] * (e["scan_avg_us"] + e["combine_avg_us"] + e.get("append_avg_us", 0.0))
                   for e in breakdown.values())
    step_breakdown = {"by_format": breakdown, "sum_of_launches_us": round(parts_us, 1),
                      "step_us": round(ms_per_step * 1e3, 1),
                      "what": "per format: the average of its launches, each kind timed as a graph of that kind "
                              "alone over every layer of the format and every timed step; the sum is the "
                              "step's launches end to end"}

    main_f = fmts[0]
    xr = layers[next(l for l, x in enumerate(layers) if fmt_of(x) == main_f)]
    lr = next(l for l, x in enumerate(layers) if fmt_of(x) == main_f)
    kern_s = breakdown[main_f]["scan_avg_us"] * 1e-6
    alg = breakdown[main_f]["scan_bytes_avg"]
    achieved = alg / kern_s / 1e9
    b0 = xr["bits"]
    kname = (f"decode_kernel<{d},{b0.k_bits - b0.k_mode},{'true' if b0.k_mode else 'false'},{b0.v_bits},"
             f"{'true' if xr['fused'] else 'false'},{'true' if Hq // H <= 8 else 'false'}> "
             f"({'tq_decode_step_partial' if xr['fused'] else 'tq_decode_partial'})")
    log(f"step {ms_per_step * 1e3:.1f} us -> {value:.0f} GB/s; {main_f} split-K kernel {kern_s * 1e6:.2f} us, "
        f"{alg / 1e6:.1f} MB/launch -> {achieved:.0f} GB/s; launches of a step end to end {parts_us:.0f} us")

    # ---- the practical ceiling: a plain streaming read of a buffer the size of a few layers
    ceiling = stream_ceiling()

    main_q = quantize.get(main_f)
    result = {
        "metric": "decode-attn compressed-KV GB/s (% of HBM peak); KV quantize vectors/s",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16-mfma+fp32", "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "kv_heads": H, "q_heads": Hq, "head_dim": d, "batch": B,
                   "seq_len": T, "bits": {f: sum(fmt_of(x) == f for x in layers) for f in fmts},
                   "page_tokens": 16, "shuffled_pages": wl.shuffled_pages, "launch": "graph"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "quantize_vectors_per_s": main_q["vectors_per_s"] if main_q else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(f"decode_traffic_{wl.name}.json", kernel_source_hash()),
                     "kernel": kname, "bytes_per_launch": round(alg), "avg_launch_us": round(kern_s * 1e6, 3),
                     "frac_of_stream_read": round(achieved / ceiling["gbs"], 4) if ceiling else None,
                     "timing": f"graph of the {main_f} layers' split-K launches of the timed steps "
                               f"({breakdown[main_f]['layers']} x {K}), one event pair"},
        "quantize": quantize,
        "stream_read": ceiling,
        "step_breakdown": step_breakdown,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        pool = _seq_pages(xr["pages"], xr["offs"]["page_bytes"], xr["pt"][0, :(T + 15) // 16])
        result["cpu_baseline"] = cpu_baseline(H, d, b0, pool, T, qs[lr].double().cpu().numpy(), scale, xr["sw"],
                                              xr["S"], args.cpu_seconds, record_bytes(xr["offs"], H),
                                              f"layer {lr} ({main_f}), sequence 0")
    del layers, news, qs, wss
    return result


def stream_ceiling(mb=2048, reps=5):
    """A plain streaming read (tq_stream_read) of an ``mb`` MB buffer, larger than the Infinity Cache: the best of
    a few launch sizes, each timed by HIP events around ``reps`` launches; GB/s."""
    import torch

    import kv_cache_quantization_wht_amd as tq

    buf = torch.ones(mb * 1000 * 1000 // 16 * 16, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    best = None
    for per_cu in (1, 2, 4, 8, 16):
        blocks = cus * per_cu
        tq.stream_read(buf, blocks, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            tq.stream_read(buf, blocks, sink)
        e1.record()
        torch.cuda.synchronize()
        gbs = buf.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes": buf.numel(),
                    "blocks": blocks, "kernel": "stream_read_kernel (tq_stream_read)",
                    "what": f"plain streaming read of {mb} MB, 16-byte loads, best of 1-16 work-groups per CU"}
    log(f"streaming-read ceiling: {best['gbs']:.0f} GB/s ({100 * best['frac_of_peak']:.1f}% of 8 TB/s)")
    del buf
    return best


def _seq_pages(pages, page_bytes, ids):
    """Host copy of the listed pages, in order."""
    import torch

    idx = torch.as_tensor(np.asarray(ids, dtype=np.int64), device=pages.device)
    return pages.view(-1, page_bytes).index_select(0, idx).cpu().numpy().reshape(-1)


if __name__ == "__main__":
    main()

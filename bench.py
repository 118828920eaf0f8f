#!/usr/bin/env python3
"""Benchmark of the TurboQuant hot path on one MI355X.

Workload: the Llama-3.1-8B single-layer cache (8 KV heads, 32 query heads, head_dim 128, batch 1,
32768 cached tokens, K 4-bit / V 2-bit MSE, bf16 inputs). One step is one decode step of that workload:
quantize-on-write of the new token's K and V (8 heads each) into its page slot and decode attention of the
new query over all cached tokens (rotation of q, split-K scores/softmax/value sums on the packed pages,
merge and inverse rotation), as tq_decode_step: the work-group owning the new token's page quantizes it,
so the step is one split-K launch plus the merge launch.

The cache of one layer is 26 MB, which would stay in the 256 MB Infinity Cache if the same layer were
read step after step. A real model reads every other layer's cache before it comes back to this one, so
the benchmark cycles through ``--copies`` independent copies of the layer cache (16 x 26 MB by default,
more than the Infinity Cache) and each step works on the next copy: every step's bytes come from HBM.

Prints one JSON line. ``value`` is the step's algorithmic bytes (compressed-KV records of every cached token,
the new token's K/V input, page ids) divided by the wall time of the whole step (both launches), in GB/s;
``roofline`` reports the split-K launch alone (algorithmic bytes per launch / its average launch duration
from HIP events); ``quantize_vectors_per_s`` is the quantize kernel's rate on the 32768-token prefill of the
layer (524288 vectors); ``cpu_baseline`` times the CPU oracle on a bounded sample of the same cache.
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
WORKLOAD_INDEX = 1


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("tq_decode.hip", "tq_common.h", "tq_quant_common.h"):
        with open(os.path.join(ROOT, "kv_cache_quantization_wht_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(bytes_per_launch_alg):
    """HBM traffic of the decode kernel from committed rocprofv3 counter runs, if taken on this source."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--copies", type=int, default=16, help="independent layer caches cycled per step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch steps from Python instead of a captured graph")
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
    import kv_cache_quantization_wht_amd as tq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda"
    wl = kvsynth.workloads()[WORKLOAD_INDEX]
    H, Hq, d, T = wl.kv_heads, wl.q_heads, wl.head_dim, wl.seq_len
    bits = wl.bits[0]
    layout = tq.Layout(d, H, bits.k_bits, bits.k_mode, bits.v_bits, bits.v_mode)
    offs = tq.page_layout(layout)
    page_bytes = offs["page_bytes"]
    K, W, C = args.steps, args.warmup, args.copies
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
    k_pre, v_pre = kvsynth.make_kv(wl, WORKLOAD_INDEX, 0, T, device=dev)
    slots0 = torch.arange(T, dtype=torch.int64, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    qtimes = []
    for rep in range(6):
        ev[0].record()
        tq.quantize_kv(layout, pages, k_pre, v_pre, slots0, kcb, vcb)
        ev[1].record()
        torch.cuda.synchronize()
        if rep:
            qtimes.append(ev[0].elapsed_time(ev[1]) * 1e-3)
    q_time = float(np.median(qtimes))
    n_vec = T * H * 2
    quant_vps = n_vec / q_time
    for c in range(1, C):
        tq.quantize_kv(layout, pages, k_pre, v_pre, slots0 + c * pages_per_copy * 16, kcb, vcb)
    torch.cuda.synchronize()
    log(f"prefill quantize: {n_vec} vectors in {q_time * 1e6:.1f} us -> {quant_vps / 1e9:.2f} G vectors/s")

    # ---- per-step inputs: new token K/V, query, slot, sequence length (all resident before timing)
    k_new, v_new = kvsynth.make_kv(wl, WORKLOAD_INDEX, 0, total_steps, device=dev, token_offset_seed=1)
    g = torch.Generator(device=dev).manual_seed(kvsynth.data_seed(WORKLOAD_INDEX, 0, "q"))
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
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(W, total_steps):
                    step(i)
            torch.cuda.synchronize()
        except Exception as e:  # noqa: BLE001
            log(f"graph capture unavailable ({e!r}); timing eagerly")
            graph, mode = None, "eager"

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

    # ---- split-K kernel duration from HIP events on the launch stream. Events recorded inside a captured
    #      graph are not timed on this platform, so the K tq_decode_partial launches of the timed steps are
    #      captured on their own (no other kernel between them) and one event pair brackets the replay:
    #      average duration = elapsed / K. The same is done for the K tq_decode_combine launches.
    def replay_avg(fn):
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            for i in range(W, total_steps):
                fn(i)
        gph.replay()  # warm
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / K

    def partial_only(i):
        tq.decode_step(layout, pages, k_new[i:i + 1], v_new[i:i + 1], qs[i], page_tables[step_copy[i]], step_lens[i],
                       scale, kcb, vcb, workspace=ws, out=out, first_pass_only=True)

    def combine_only(i):
        tq.decode_combine(layout, pages, qs[i], page_tables[step_copy[i]], step_lens[i], scale, kcb, vcb, ws, out=out)

    kmode = "graph of the K launches, one event pair"
    try:
        durs = np.array([replay_avg(partial_only)])
        comb = np.array([replay_avg(combine_only)])
    except Exception as e:  # noqa: BLE001
        log(f"graph timing unavailable ({e!r}); events around eager launches")
        kmode = "eager+sleep"
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(K)]
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(50_000_000)  # keep the GPU busy while every launch is queued
        for j, i in enumerate(range(W, total_steps)):
            evs[j][0].record()
            partial_only(i)
            evs[j][1].record()
            combine_only(i)
            evs[j][2].record()
        torch.cuda.synchronize()
        durs = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
        comb = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    kern_s = float(np.mean(durs))
    alg_per_launch = float(np.mean(step_bytes[W:]))
    achieved = alg_per_launch / kern_s / 1e9
    traffic = load_traffic(alg_per_launch)
    log(f"step {ms_per_step * 1e3:.2f} us ({mode}); split-K decode kernel {kern_s * 1e6:.2f} us, combine "
        f"{float(np.mean(comb)) * 1e6:.2f} us ({kmode}); {alg_per_launch / 1e6:.2f} MB/launch -> {achieved:.0f} GB/s")

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
                     "kernel": "decode_kernel<128,4,false,2,true> (tq_decode_step_partial)",
                     "bytes_per_launch": round(alg_per_launch), "avg_launch_us": round(kern_s * 1e6, 3),
                     "combine_avg_us": round(float(np.mean(comb)) * 1e6, 3), "timing": kmode},
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layout, offs, pages, page_tables[0], T, qs, scale, sw, args.cpu_seconds,
                                              bits)
    print(json.dumps(result), flush=True)


def cpu_baseline(layout, offs, pages, page_table, T, qs, scale, sw, budget_s, bits):
    """Time the CPU oracle's decode attention on copy 0 of the cache: one KV head (its query heads) at a time,
    over successive decode queries, until the time budget is spent."""
    from oracle import attention, codec

    H, d = layout.num_kv_heads, layout.head_dim
    pb = offs["page_bytes"]
    npg = (T + 15) // 16
    first = int(page_table[0, 0].item())
    pool = pages[first * pb:(first + npg) * pb].cpu().numpy()
    Lo = codec.page_layout(H, d, bits.k_bits, bits.k_mode, bits.v_bits, bits.v_mode)
    cbk = codec.make_codebook(d, bits.k_bits, bits.k_mode, sw)
    cbv = codec.make_codebook(d, bits.v_bits, bits.v_mode, sw)
    pt = np.arange(npg, dtype=np.int64)[None]
    qall = qs.double().cpu().numpy()  # [steps, 1, Hq, d]
    G = qall.shape[2] // H
    rec_bytes = offs["k_norms"] // (H * 16) + 2 + (offs["v_norms"] - offs["v_codes"]) // (H * 16) + 2
    done, t_used, step = 0, 0.0, 0
    t0 = time.perf_counter()
    while t_used < budget_s and step < qall.shape[0]:
        for g in range(H):
            heads = [(0, h) for h in range(g * G, (g + 1) * G)]
            attention.decode_attention(pool, Lo, cbk, cbv, qall[step], pt, [T], scale, heads=heads)
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
            "sample": f"fp64 oracle decode attention of copy 0 (T={T}, 8 KV heads x {G} query heads each): {done} "
                      f"(KV head, query) units over {step} decode queries in {t_used:.1f} s; same unit as value",
            "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()

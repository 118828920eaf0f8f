"""Parity at the workloads' full sizes, one layer at a time, in the launch configuration the benchmark
times (tq_decode_step with the automatic split plan; tq_quantize_kv then tq_decode_attention for the
formats the fused step does not take: prod K and 8-bit codes): every sequence of the layer is prefilled
through tq_quantize_kv, one decode step appends a token to each sequence and attends, and sampled outputs
are checked against the oracle one by one.

  records    sampled tokens of every sequence (first, last cached, the appended one and random ones),
             every KV head, K and V: the oracle's encoding of the same input vectors, under the code /
             norm / sketch rules of the other quantize tests
  attention  sampled (sequence, KV head) pairs: all G query heads against the oracle run on the GPU's
             own pages of that sequence, max relative error <= 2e-3; and, reported (not gated), the end-to-end
             figure of the first and last pair: against the oracle's attention over its own encoding of the raw
             K/V of the whole sequence
"""
import numpy as np
import pytest

import kvsynth
from oracle import attention, codec
from tests import parity

pytestmark = pytest.mark.gpu

# (id, workload index, layer)
LAYERS = [
    ("8b-1layer-T32768-k4v2", 1, 0),
    ("8b-32layer-B32-T8192-k3v3-layer0", 2, 0),
    ("prod-k2qjl-B16-T131072", 3, 0),
    ("70b-B4-T131072-k8v8-layer0", 4, 0),
    ("70b-B4-T131072-k4v2-layer2", 4, 2),
]


def _host_pages(pages, page_bytes, ids):
    """The listed pages copied to the host as a compact pool (page i of the result = page ids[i])."""
    import torch

    idx = torch.as_tensor(np.asarray(ids, dtype=np.int64), device=pages.device)
    return pages.view(-1, page_bytes).index_select(0, idx).cpu().numpy().reshape(-1)


@pytest.mark.parametrize("case", LAYERS, ids=[c[0] for c in LAYERS])
def test_full_size_layer(case):
    import torch
    import kv_cache_quantization_wht_amd as tq

    name, wi, layer = case
    wl = kvsynth.workloads()[wi]
    bits = wl.bits[layer]
    H, Hq, d, B, T = wl.kv_heads, wl.q_heads, wl.head_dim, wl.batch, wl.seq_len
    print(f"full-size layer {name}: B={B} T={T} H={H} Hq={Hq} d={d} bits={bits}", flush=True)
    layout, Lo = parity.make_layout(H, d, bits.k_bits, bits.k_mode, bits.v_bits, bits.v_mode)
    pb = Lo["page_bytes"]
    pps = (T + 1 + 15) // 16
    pt, npages = kvsynth.page_table(B, pps, wl.shuffled_pages, seed=4242 + layer)
    rseed = kvsynth.rotation_seed(layer)
    kcb, cbk = parity.device_codebook(d, bits.k_bits, bits.k_mode, seed=rseed)
    vcb, cbv = parity.device_codebook(d, bits.v_bits, bits.v_mode, seed=rseed)
    pages = torch.zeros(npages * pb, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(wi * 100 + layer)

    # prefill, sequence by sequence; keep the input vectors of the sampled tokens
    samples = []  # (b, token positions, k [n, H, d], v [n, H, d]) as fp64 host arrays
    raw = {}  # (b, KV head) -> raw K, V [T, d] of the end-to-end pairs
    for b in range(B):
        k, v = kvsynth.make_kv(wl, wi, layer, T, device="cuda", token_offset_seed=2 + b)
        for g in {0: [0], B - 1: [H - 1]}.get(b, []) if B > 1 else [0, H - 1]:
            raw[(b, g)] = (k[:, g].double().cpu().numpy(), v[:, g].double().cpu().numpy())
        slots = torch.from_numpy(kvsynth.slots_for(pt, b, 0, T)).cuda()
        tq.quantize_kv(layout, pages, k, v, slots, kcb, vcb)
        if b in (0, B - 1) or b % 7 == 3:
            t = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 30)]))
            ti = torch.from_numpy(t).cuda()
            samples.append((b, t, k.index_select(0, ti).double().cpu().numpy(), v.index_select(0, ti).double().cpu().numpy()))
        del k, v
    k_new, v_new = kvsynth.make_kv(wl, wi, layer, B, device="cuda", token_offset_seed=1)
    q = kvsynth.make_q(wl, wi, layer, B, device="cuda")
    sl = torch.full((B,), T + 1, dtype=torch.int32, device="cuda")
    ptd = torch.from_numpy(pt).cuda()
    if bits.k_mode == 0 and bits.v_mode == 0 and bits.k_bits <= 4 and bits.v_bits <= 4:
        out = tq.decode_step(layout, pages, k_new, v_new, q, ptd, sl, wl.softmax_scale, kcb, vcb)
    else:  # formats outside the fused step: append, then attend
        tq.quantize_kv(layout, pages, k_new, v_new, torch.from_numpy(pt[:, T // 16].astype(np.int64) * 16 + T % 16).cuda(),
                       kcb, vcb)
        out = tq.decode_attention(layout, pages, q, ptd, sl, wl.softmax_scale, kcb, vcb)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(out).all()

    # records of the sampled tokens and of every appended token
    rep = parity.Report()
    kn, vn = k_new.double().cpu().numpy(), v_new.double().cpu().numpy()
    samples.append((None, None, kn, vn))
    for b, t, kx, vx in samples:
        if b is None:  # the appended tokens: position T of every sequence
            bb, tt = np.arange(B), np.full(B, T)
        else:
            bb, tt = np.full(len(t), b), t
        gpage = pt[bb, tt // 16]
        uniq, inv = np.unique(gpage, return_inverse=True)
        pool = _host_pages(pages, pb, uniq)
        for h in range(H):
            for which, x, cb in (("k", kx, cbk), ("v", vx, cbv)):
                got = codec.read_records(pool, Lo, which, inv, tt % 16, h)
                one = parity.Report()
                parity.compare_records(got, codec.encode(x[:, h, :], cb), cb, one, which)
                for key, val in one.items():
                    rep[key] = rep.get(key, 0) + val
    print(f"  records {rep}", flush=True)

    # attention of sampled (sequence, KV head) pairs against the oracle on the GPU's own pages
    G = Hq // H
    picks = {(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))}
    qh = q.double().cpu().numpy()
    worst = 0.0
    for b, g in sorted(picks):
        pool = _host_pages(pages, pb, pt[b])
        heads = [(0, h) for h in range(g * G, (g + 1) * G)]
        ref = attention.decode_attention(pool, Lo, cbk, cbv, qh[b:b + 1], np.arange(pps, dtype=np.int64)[None],
                                         np.array([T + 1]), wl.softmax_scale, heads=heads)
        err = parity.attention_error(out[b:b + 1, g * G:(g + 1) * G], ref[:, g * G:(g + 1) * G])
        worst = max(worst, err)
        assert err <= parity.ATTN_TOL, (b, g, err)
    print(f"  attention: {len(picks)} (sequence, KV head) pairs, max relative error {worst:.2e}", flush=True)
    for (b, g), (kr, vr) in sorted(raw.items()):
        kr = np.concatenate([kr, kn[b:b + 1, g]])
        vr = np.concatenate([vr, vn[b:b + 1, g]])
        e2e = parity.end_to_end_reference(qh[b, g * G:(g + 1) * G], kr, vr, cbk, cbv, wl.softmax_scale)
        print(f"  end to end (the oracle's own codes of the raw K/V), sequence {b} KV head {g}: relative error "
              f"{parity.attention_error(out[b, g * G:(g + 1) * G], e2e):.2e}", flush=True)
    del pages
    torch.cuda.empty_cache()

"""GPU decode attention (tq_decode_attention through the C ABI) against the CPU oracle run on the
GPU's own packed pool."""
import math

import numpy as np
import pytest

import kvsynth
from oracle import attention
from tests import parity

pytestmark = pytest.mark.gpu


def build(H, d, Hq, B, lens, kb, km, vb, vm, seed=0, shuffled=True, dtype="bf16", q_scale=1.0,
          extra_pages=3, k_mult=1.0, min_pages=0, recipe="lognormal", v_mult=1.0):
    import torch
    import kv_cache_quantization_wht_amd as tq

    layout, Lo = parity.make_layout(H, d, kb, km, vb, vm)
    pps = max(1, min_pages, max((l + 15) // 16 for l in lens))
    pt, npages = kvsynth.page_table(B, pps, shuffled, seed=seed + 4, extra_pages=extra_pages)
    kcb, cbk = parity.device_codebook(d, kb, km, seed=seed + 1)
    vcb, cbv = parity.device_codebook(d, vb, vm, seed=seed + 2)
    pages = torch.full((npages * Lo["page_bytes"],), 0xA5, dtype=torch.uint8, device="cuda")
    for b in range(B):
        if lens[b] == 0:
            continue
        k, v = parity.seeded_kv(lens[b], H, d, seed=seed * 100 + b, recipe=recipe, dtype=dtype, v_mult=v_mult)
        slots = torch.from_numpy(kvsynth.slots_for(pt, b, 0, lens[b])).cuda()
        tq.quantize_kv(layout, pages, (k.float() * k_mult).to(k.dtype).cuda(), v.cuda(), slots, kcb, vcb)
    g = torch.Generator().manual_seed(seed + 77)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    q = (torch.randn(B, Hq, d, generator=g) * q_scale).to(tdt)
    torch.cuda.synchronize()
    return dict(layout=layout, Lo=Lo, pages=pages, pool=pages.cpu().numpy(), pt=pt,
                lens=np.array(lens, dtype=np.int32), q=q, kcb=kcb, vcb=vcb, cbk=cbk, cbv=cbv)


def run_gpu(c, scale, pps=0):
    import torch
    import kv_cache_quantization_wht_amd as tq

    out = tq.decode_attention(c["layout"], c["pages"], c["q"].cuda(), torch.from_numpy(c["pt"]).cuda(),
                              torch.from_numpy(c["lens"]).cuda(), scale, c["kcb"], c["vcb"], pages_per_split=pps)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def run_ref(c, scale):
    return attention.decode_attention(c["pool"], c["Lo"], c["cbk"], c["cbv"], c["q"].double().numpy(), c["pt"],
                                      c["lens"], scale)


CASES = [
    # name, H, d, Hq, B, lens, kb, km, vb, vm, dtype, q_scale
    ("gqa4-d64-f32", 1, 64, 4, 1, [1024], 4, 0, 2, 0, "f32", 1.0),
    ("ragged-d128", 2, 128, 8, 5, [0, 1, 17, 100, 333], 4, 0, 2, 0, "bf16", 1.0),
    ("mha", 4, 128, 4, 2, [65, 200], 4, 0, 2, 0, "bf16", 1.0),
    ("gqa2", 4, 128, 8, 1, [129], 3, 0, 3, 0, "bf16", 1.0),
    ("gqa8", 2, 128, 16, 2, [300, 47], 4, 0, 2, 0, "bf16", 1.0),
    ("gqa16", 1, 128, 16, 1, [250], 4, 0, 2, 0, "f16", 1.0),
    ("gqa3", 2, 128, 6, 2, [333, 31], 4, 0, 2, 0, "bf16", 1.0),
    ("gqa6-prod-k2v2", 2, 128, 12, 2, [210, 95], 2, 1, 2, 0, "bf16", 1.0),
    ("gqa5-k3v3", 1, 128, 5, 1, [477], 3, 0, 3, 0, "bf16", 2.0),
    ("k8v8", 2, 128, 8, 2, [90, 161], 8, 0, 8, 0, "bf16", 1.0),
    ("k1v4", 2, 128, 8, 1, [150], 1, 0, 4, 0, "bf16", 1.0),
    ("k3v3-d64", 2, 64, 8, 2, [77, 130], 3, 0, 3, 0, "bf16", 1.0),
    ("k8v1-d64", 1, 64, 4, 1, [99], 8, 0, 1, 0, "f32", 1.0),
    ("prod-k2v2", 2, 128, 8, 3, [40, 200, 1], 2, 1, 2, 0, "bf16", 1.0),
    ("prod-k3v3", 2, 128, 8, 1, [180], 3, 1, 3, 0, "bf16", 1.0),
    ("prod-k4v2-d64", 2, 64, 8, 2, [64, 95], 4, 1, 2, 0, "f32", 1.0),
    ("peaked", 2, 128, 8, 2, [257, 300], 4, 0, 2, 0, "bf16", 6.0),
    ("broad", 2, 128, 8, 2, [257, 300], 4, 0, 2, 0, "bf16", 0.05),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle(case):
    name, H, d, Hq, B, lens, kb, km, vb, vm, dt, qs = case
    print(f"decode case {name}", flush=True)
    c = build(H, d, Hq, B, lens, kb, km, vb, vm, seed=len(name), dtype=dt, q_scale=qs)
    scale = 1.0 / math.sqrt(d)
    out = run_gpu(c, scale)
    ref = run_ref(c, scale)
    err = parity.attention_error(out, ref)
    print(f"{name}: max rel err {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= parity.ATTN_TOL
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(out[b] == 0)


def test_split_count_invariance_and_determinism():
    c = build(2, 128, 8, 2, [500, 333], 4, 0, 2, 0, seed=3)
    scale = 1 / math.sqrt(128)
    ref = run_ref(c, scale)
    outs = {pps: run_gpu(c, scale, pps) for pps in (2, 4, 6, 32, 0)}
    for pps, o in outs.items():
        assert parity.attention_error(o, ref) <= parity.ATTN_TOL, pps
        assert np.allclose(o, outs[2], rtol=1e-5, atol=1e-6), pps
    again = run_gpu(c, scale, 4)
    assert np.array_equal(again, outs[4])


def test_page_table_shuffle_invariance():
    """The same tokens through an identity or a shuffled page table give the same output."""
    scale = 1 / math.sqrt(128)
    a = run_gpu(build(2, 128, 8, 2, [170, 64], 3, 0, 3, 0, seed=8, shuffled=False), scale, 4)
    b = run_gpu(build(2, 128, 8, 2, [170, 64], 3, 0, 3, 0, seed=8, shuffled=True), scale, 4)
    assert np.array_equal(a, b)


def test_large_key_norms():
    """K ~ N(0, 100^2) with V ~ N(0, 1) (norm ratio ~100): very peaked softmax stays within tolerance. (The zero
    vectors are planted, the 300x key is not: 300 times these keys would pass the fp16 range of the stored norm.)"""
    c = build(2, 128, 16, 1, [400], 4, 0, 2, 0, seed=21, k_mult=100.0, recipe="zeros")
    scale = 1 / math.sqrt(128)
    out = run_gpu(c, scale)
    assert parity.attention_error(out, run_ref(c, scale)) <= parity.ATTN_TOL


VALUE_CASES = [
    # name, H, d, Hq, B, lens, kb, km, vb, vm, q_scale, recipe, v_mult, pages_per_split
    ("v-tiny-k4v2", 2, 128, 8, 2, [300, 77], 4, 0, 2, 0, 1.0, "lognormal", 2.0 ** -16, 0),
    ("v-huge-k4v2", 2, 128, 8, 2, [300, 77], 4, 0, 2, 0, 1.0, "lognormal", 2.0 ** 8, 0),
    ("v-tiny-k3v3-splits", 2, 128, 8, 1, [700], 3, 0, 3, 0, 1.0, "lognormal", 2.0 ** -16, 4),
    ("v-tiny-gqa16", 1, 128, 16, 1, [260], 4, 0, 2, 0, 1.0, "lognormal", 2.0 ** -16, 0),
    ("v-tiny-prod-d64", 2, 64, 8, 2, [90, 200], 2, 1, 2, 0, 1.0, "lognormal", 2.0 ** -16, 0),
    ("v-range-k4v2", 2, 128, 8, 2, [600, 129], 4, 0, 2, 0, 1.0, "vrange", 1.0, 0),
    ("v-range-k8v8-peaked", 2, 128, 8, 1, [333], 8, 0, 8, 0, 4.0, "vrange", 1.0, 2),
    ("v-range-k4v4-gqa16", 1, 128, 16, 1, [400], 4, 0, 4, 0, 1.0, "vrange", 1.0, 0),
]


@pytest.mark.parametrize("case", VALUE_CASES, ids=[c[0] for c in VALUE_CASES])
def test_value_norm_range(case):
    """Values uniformly tiny (2^-16) or large (2^8), or of norms spread over 2^-14 .. 2^6 token by token: the value
    weights p * ||v|| enter the matrix cores as fp16, and each column's power-of-two shift keeps them in range, so
    every row is within the bar of the oracle and the output scales with V."""
    name, H, d, Hq, B, lens, kb, km, vb, vm, qs, recipe, vmul, pps = case
    print(f"value-range case {name}", flush=True)
    scale = 1.0 / math.sqrt(d)
    c = build(H, d, Hq, B, lens, kb, km, vb, vm, seed=len(name) + 5, q_scale=qs, recipe=recipe, v_mult=vmul)
    out = run_gpu(c, scale, pps)
    ref = run_ref(c, scale)
    err = parity.attention_error(out, ref)
    print(f"{name}: max rel err {err:.3e}", flush=True)
    assert np.all(np.isfinite(out))
    assert err <= parity.ATTN_TOL
    if vmul != 1.0:
        # the same keys and values at scale 1 (a power of two scales the fp16 norms exactly, the codes not at all)
        one = run_gpu(build(H, d, Hq, B, lens, kb, km, vb, vm, seed=len(name) + 5, q_scale=qs, recipe=recipe), scale,
                      pps)
        rel = parity.attention_error(out / vmul, one)
        print(f"{name}: output / {vmul:g} against the unscaled run {rel:.3e}", flush=True)
        assert rel <= 1e-5


def test_zero_value_winner():
    """A key far ahead of the others whose value is zero: the output is made of weights ~2^-30 .. 2^-50 of the winner's,
    which the value shift brings into the fp16 range of the value operand."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    H, d, Hq = 2, 128, 8
    scale = 1 / math.sqrt(d)
    for lead in (30.0, 50.0):
        c = build(H, d, Hq, 1, [400], 4, 0, 2, 0, seed=91, recipe="plain")
        # rewrite token 200 of both KV heads: a key along the mean query direction of its group whose logit is about
        # `lead` log2 units above the others' largest (~12), value zero; the oracle reads the GPU's own records of it
        q = c["q"].float()
        k = torch.zeros(1, H, d)
        for g in range(H):
            qm = q[0, g * (Hq // H):(g + 1) * (Hq // H)].mean(0)
            k[0, g] = qm / qm.norm() * ((lead + 12.0) * math.log(2) / (scale * qm.norm()))
        v = torch.zeros(1, H, d)
        slot = int(c["pt"][0, 200 // 16]) * 16 + 200 % 16
        tq.quantize_kv(c["layout"], c["pages"], k.to(torch.bfloat16).cuda(), v.to(torch.bfloat16).cuda(),
                       torch.tensor([slot], dtype=torch.int64, device="cuda"), c["kcb"], c["vcb"])
        torch.cuda.synchronize()
        c["pool"] = c["pages"].cpu().numpy()
        for pps in (0, 4):
            out = run_gpu(c, scale, pps)
            ref = run_ref(c, scale)
            err = parity.attention_error(out, ref)
            size = float(np.abs(ref).max(axis=-1).min())
            print(f"zero-value winner lead {lead}: smallest row max |o| {size:.2e}, max rel err {err:.3e} (pps {pps})",
                  flush=True)
            assert size < 1e-6  # the rows really are made of far-behind weights
            assert err <= parity.ATTN_TOL


def test_zero_softmax_scale_is_uniform_average():
    """scale 0: every cached token gets the same weight (mean of the dequantized values)."""
    c = build(2, 128, 8, 2, [130, 47], 4, 0, 2, 0, seed=31)
    out = run_gpu(c, 0.0)
    assert parity.attention_error(out, run_ref(c, 0.0)) <= parity.ATTN_TOL


def test_two_passes_equal_one_call():
    """tq_decode_partial then tq_decode_combine (same arguments) give the bytes of tq_decode_attention,
    with one run per sequence (combine launches nothing) and with several."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    c = build(2, 128, 8, 3, [700, 33, 290], 4, 0, 2, 0, seed=41)
    scale = 1 / math.sqrt(128)
    pt, sl = torch.from_numpy(c["pt"]).cuda(), torch.from_numpy(c["lens"]).cuda()
    q = c["q"].cuda()
    for pps in (0, 4, 64):
        need = tq.decode_workspace_bytes(c["layout"], 3, 8, pt.shape[1], pps)
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        one = tq.decode_attention(c["layout"], c["pages"], q, pt, sl, scale, c["kcb"], c["vcb"], pages_per_split=pps)
        two = torch.full_like(one, float("nan"))
        tq.decode_partial(c["layout"], c["pages"], q, pt, sl, scale, c["kcb"], c["vcb"], ws, out=two,
                          pages_per_split=pps)
        tq.decode_combine(c["layout"], c["pages"], q, pt, sl, scale, c["kcb"], c["vcb"], ws, out=two,
                          pages_per_split=pps)
        torch.cuda.synchronize()
        assert torch.equal(one, two), pps
        assert parity.attention_error(two.cpu().numpy().astype(np.float64), run_ref(c, scale)) <= parity.ATTN_TOL


STEP_CASES = [
    # name, H, d, Hq, lens (counting the new token), kb, vb, kv dtype, pages_per_split
    ("k4v2-ragged", 2, 128, 8, [700, 33, 1, 17], 4, 2, "bf16", 0),
    ("k3v3-gqa4-splits", 2, 128, 8, [290, 257], 3, 3, "bf16", 2),
    ("k2v2-gqa8", 2, 128, 16, [145, 64], 2, 2, "f16", 0),
    ("k1v4-d64", 2, 64, 8, [99, 16, 32], 1, 4, "f32", 4),
    ("k4v2-mha-d64", 4, 64, 4, [1, 200], 4, 2, "f32", 0),
    ("k4v4-gqa16", 1, 128, 16, [513], 4, 4, "bf16", 0),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_decode_step_equals_append_then_attention(case):
    """tq_decode_step writes the same page bytes as tq_quantize_kv of the new tokens and gives the output of
    tq_decode_attention over the result (and of the oracle on the written pool)."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    name, H, d, Hq, lens, kb, vb, dt, pps = case
    print(f"decode step case {name}", flush=True)
    prev = [max(L - 1, 0) for L in lens]
    c = build(H, d, Hq, len(lens), prev, kb, 0, vb, 0, seed=7 + len(name), dtype=dt,
              min_pages=max((L + 15) // 16 for L in lens))
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dt]
    g = torch.Generator().manual_seed(123 + len(name))
    k_new = (torch.randn(len(lens), H, d, generator=g) * 3).to(tdt).cuda()
    v_new = torch.randn(len(lens), H, d, generator=g).to(tdt).cuda()
    pt = torch.from_numpy(c["pt"]).cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    q = c["q"].cuda()
    scale = 1 / math.sqrt(d)
    # path A: append through tq_quantize_kv into the new tokens' slots, then decode attention
    pages_a = c["pages"].clone()
    slots = [int(c["pt"][b, (L - 1) // 16]) * 16 + (L - 1) % 16 if L > 0 else -1 for b, L in enumerate(lens)]
    for b, L in enumerate(lens):
        if L > 0:
            tq.quantize_kv(c["layout"], pages_a, k_new[b:b + 1].reshape(1, H, d), v_new[b:b + 1].reshape(1, H, d),
                           torch.tensor([slots[b]], dtype=torch.int64, device="cuda"), c["kcb"], c["vcb"])
    out_a = tq.decode_attention(c["layout"], pages_a, q, pt, sl, scale, c["kcb"], c["vcb"], pages_per_split=pps)
    # path B: one decode step
    pages_b = c["pages"].clone()
    out_b = tq.decode_step(c["layout"], pages_b, k_new, v_new, q, pt, sl, scale, c["kcb"], c["vcb"],
                           pages_per_split=pps)
    torch.cuda.synchronize()
    assert torch.equal(pages_a, pages_b)
    oa, ob = out_a.cpu().numpy().astype(np.float64), out_b.cpu().numpy().astype(np.float64)
    assert parity.attention_error(ob, oa) <= 1e-4
    ref = attention.decode_attention(pages_b.cpu().numpy(), c["Lo"], c["cbk"], c["cbv"], q.cpu().double().numpy(),
                                     c["pt"], np.array(lens, dtype=np.int32), scale)
    err = parity.attention_error(ob, ref)
    print(f"{name}: step vs oracle {err:.3e}")
    assert err <= parity.ATTN_TOL
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(ob[b] == 0)


@pytest.mark.parametrize("kb,vb", [(4, 2), (8, 8)], ids=["k4v2", "k8v8"])
def test_longest_single_run(kb, vb):
    """One sequence of 4095 pages read as a single run, the longest one work-group holds (a run is at most 4096
    pages): its page ids fill the work-group's id table, the run ends on a half pair, and the ring's loads past the
    end read the table's padding. Eight query heads per KV head (packed columns)."""
    H, d, Hq, T = 1, 128, 8, 4095 * 16
    print(f"longest single run K{kb}/V{vb}, {T} tokens", flush=True)
    c = build(H, d, Hq, 1, [T], kb, 0, vb, 0, seed=61 + kb)
    scale = 1 / math.sqrt(d)
    out = run_gpu(c, scale, pps=4096)
    ref = run_ref(c, scale)
    err = parity.attention_error(out, ref)
    print(f"longest single run K{kb}/V{vb}: max rel err {err:.3e}")
    assert err <= parity.ATTN_TOL

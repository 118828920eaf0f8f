"""Chunked prefill through the C ABI against the oracle's causal chunk attention.

  tq_prefill_chunk      the chunk's records byte-identical to tq_quantize_kv of the same tokens, and its
                        attention output against the oracle run on the GPU's own pool (max relative error
                        per row <= 2e-3, the decode bar), on inputs with a zero key, a zero value and a 300x key
                        planted, and values tiny, large or spread over 2^-14 .. 2^6 token by token
  tq_prefill_attention  the same attention over a cache written beforehand; ragged chunks (several
                        work-groups and a partial last one), prefixes that end inside a page or a page pair,
                        no prefix, GQA group sizes 1 to 16, d = 64 and 128, code widths 1 to 8, sketched (prod)
                        K, f32 / bf16 / f16 queries, a shuffled page table, and the 8B layer at full length
                        (sampled rows; K4 and K2 + sketch)
"""
import math

import numpy as np
import pytest

import kvsynth
from oracle import attention, codec
from tests import parity

pytestmark = pytest.mark.gpu


def _setup(H, d, Hq, B, prefix, C, fmt, seed, q_dtype="bf16", recipe="lognormal", v_mult=1.0):
    """A device pool holding each sequence's prefix, the chunk's K/V/q and the oracle's codebooks. The default
    recipe plants a zero key, a zero value and a 300x key among the first tokens."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    kb, km, vb, vm = fmt
    layout, Lo = parity.make_layout(H, d, kb, km, vb, vm)
    kcb, cbk = parity.device_codebook(d, kb, km, seed)
    vcb, cbv = parity.device_codebook(d, vb, vm, seed + 1)
    npp = max(1, max((p + C + 15) // 16 for p in prefix))
    pt, npages = kvsynth.page_table(B, npp, True, seed=seed + 4, extra_pages=1)
    pages = torch.full((npages * Lo["page_bytes"],), 0x5A, dtype=torch.uint8, device="cuda")
    for b in range(B):
        if prefix[b]:
            k, v = parity.seeded_kv(prefix[b], H, d, seed=seed * 10 + b, recipe=recipe, v_mult=v_mult)
            tq.quantize_kv(layout, pages, k.cuda(), v.cuda(), torch.from_numpy(kvsynth.slots_for(pt, b, 0, prefix[b])).cuda(),
                           kcb, vcb)
    kc, vc = parity.seeded_kv(B * C, H, d, seed=seed * 10 + 9, recipe=recipe, v_mult=v_mult)
    kc, vc = kc.reshape(B, C, H, d).contiguous(), vc.reshape(B, C, H, d).contiguous()
    slots = np.concatenate([kvsynth.slots_for(pt, b, prefix[b], prefix[b] + C) for b in range(B)])
    g = torch.Generator().manual_seed(seed + 5)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[q_dtype]
    q = torch.randn(B, C, Hq, d, generator=g).to(tdt)
    return dict(layout=layout, Lo=Lo, kcb=kcb, vcb=vcb, cbk=cbk, cbv=cbv, pt=pt, pages=pages, kc=kc, vc=vc,
                slots=slots, q=q, prefix=np.array(prefix, np.int32))


def _oracle_error(st, out, scale, rows=None):
    pool = st["pages"].cpu().numpy()
    ref = attention.prefill_attention(pool, st["Lo"], st["cbk"], st["cbv"], st["q"].double().numpy(), st["pt"],
                                      st["prefix"], scale, rows=rows)
    got = out.cpu().numpy().astype(np.float64)
    if rows is not None:
        sel = tuple(np.array(rows).T)
        got, ref = got[sel], ref[sel]
    return parity.attention_error(got, ref)


CASES = [  # name, H, d, Hq, B, prefix, C
    ("d128-gqa4", 2, 128, 8, 2, [0, 37], 150),
    ("d128-gqa8-long", 1, 128, 8, 1, [333], 40),
    ("d64-gqa4", 2, 64, 8, 2, [16, 31], 70),
    ("d128-mha", 3, 128, 3, 1, [50], 300),
    ("d64-gqa16", 1, 64, 16, 2, [5, 64], 21),
    ("d128-gqa2-onetoken", 2, 128, 4, 3, [0, 1, 90], 1),
]
FORMATS = [(4, 0, 2, 0), (3, 0, 3, 0), (8, 0, 8, 0), (1, 0, 4, 0), (2, 0, 1, 0), (2, 1, 2, 0), (4, 1, 3, 0)]


@pytest.mark.parametrize("fmt", FORMATS, ids=[f"k{f[0]}{'p' if f[1] else ''}v{f[2]}" for f in FORMATS])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_chunk_matches_oracle(case, fmt):
    import torch
    import kv_cache_quantization_wht_amd as tq

    name, H, d, Hq, B, prefix, C = case
    print(f"prefill {name} fmt {fmt}", flush=True)
    st = _setup(H, d, Hq, B, prefix, C, fmt, seed=len(name) + 3 * fmt[0] + fmt[2])
    scale = 1.0 / math.sqrt(d)
    two = st["pages"].clone()  # the same prefix; the chunk written by tq_quantize_kv alone
    out = tq.prefill_chunk(st["layout"], st["pages"], st["kc"].cuda(), st["vc"].cuda(),
                           torch.from_numpy(st["slots"]).cuda(), st["q"].cuda(), torch.from_numpy(st["pt"]).cuda(),
                           torch.from_numpy(st["prefix"]).cuda(), scale, st["kcb"], st["vcb"])
    tq.quantize_kv(st["layout"], two, st["kc"].reshape(B * C, H, d).cuda(), st["vc"].reshape(B * C, H, d).cuda(),
                   torch.from_numpy(st["slots"]).cuda(), st["kcb"], st["vcb"])
    torch.cuda.synchronize()
    assert torch.equal(st["pages"], two), "the chunk's records differ from tq_quantize_kv's"
    assert torch.isfinite(out).all()
    err = _oracle_error(st, out, scale)
    print(f"  max relative error {err:.2e}", flush=True)
    assert err <= parity.ATTN_TOL


@pytest.mark.parametrize("q_dtype", ["f32", "f16"])
def test_prefill_attention_query_dtypes(q_dtype):
    """tq_prefill_attention over a cache written beforehand, f32 and f16 queries, a softmax scale of 0
    (uniform weights over every visible token) and a large one, on the planted inputs: with the large scale some
    rows' winning key has the zero value, and their output (~1e-9 of the values' size) is made of weights far
    below the winner's, which the value shift keeps in the fp16 range of the value operand."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    st = _setup(2, 128, 8, 2, [20, 47], 97, (4, 0, 2, 0), seed=31, q_dtype=q_dtype)
    B, C, H, d = st["kc"].shape
    tq.quantize_kv(st["layout"], st["pages"], st["kc"].reshape(B * C, H, d).cuda(),
                   st["vc"].reshape(B * C, H, d).cuda(), torch.from_numpy(st["slots"]).cuda(), st["kcb"], st["vcb"])
    for scale in (0.0, 1.0 / math.sqrt(d), 0.5):
        print(f"prefill q {q_dtype} scale {scale}", flush=True)
        out = tq.prefill_attention(st["layout"], st["pages"], st["q"].cuda(), torch.from_numpy(st["pt"]).cuda(),
                                   torch.from_numpy(st["prefix"]).cuda(), scale, st["kcb"], st["vcb"])
        torch.cuda.synchronize()
        err = _oracle_error(st, out, scale)
        print(f"  max relative error {err:.2e}", flush=True)
        assert err <= parity.ATTN_TOL


VALUE_CASES = [  # name, fmt, recipe, v_mult
    ("v-tiny-k4v2", (4, 0, 2, 0), "lognormal", 2.0 ** -16),
    ("v-huge-k4v2", (4, 0, 2, 0), "lognormal", 2.0 ** 8),
    ("v-tiny-k2pv2", (2, 1, 2, 0), "lognormal", 2.0 ** -16),
    ("v-range-k4v2", (4, 0, 2, 0), "vrange", 1.0),
    ("v-range-k8v8", (8, 0, 8, 0), "vrange", 1.0),
    ("v-range-k4pv3", (4, 1, 3, 0), "vrange", 1.0),
]


@pytest.mark.parametrize("case", VALUE_CASES, ids=[c[0] for c in VALUE_CASES])
def test_prefill_value_norm_range(case):
    """Values uniformly tiny (2^-16) or large (2^8), or of norms spread over 2^-14 .. 2^6 token by token, through
    tq_prefill_chunk: every row within the bar of the oracle, and a uniform power-of-two scale of V scales the output."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    name, fmt, recipe, vmul = case
    print(f"prefill value-range case {name}", flush=True)

    def run(vm):
        st = _setup(2, 128, 8, 2, [45, 130], 70, fmt, seed=17, recipe=recipe, v_mult=vm)
        out = tq.prefill_chunk(st["layout"], st["pages"], st["kc"].cuda(), st["vc"].cuda(),
                               torch.from_numpy(st["slots"]).cuda(), st["q"].cuda(), torch.from_numpy(st["pt"]).cuda(),
                               torch.from_numpy(st["prefix"]).cuda(), 1.0 / math.sqrt(128), st["kcb"], st["vcb"])
        torch.cuda.synchronize()
        return st, out

    st, out = run(vmul)
    assert torch.isfinite(out).all()
    err = _oracle_error(st, out, 1.0 / math.sqrt(128))
    print(f"  max relative error {err:.2e}", flush=True)
    assert err <= parity.ATTN_TOL
    if vmul != 1.0:
        _, one = run(1.0)
        rel = parity.attention_error(out.cpu().numpy().astype(np.float64) / vmul,
                                     one.cpu().numpy().astype(np.float64))
        print(f"  output / {vmul:g} against the unscaled run {rel:.2e}", flush=True)
        assert rel <= 1e-5


def test_prefill_rows_match_decode():
    """Row i of a chunk against tq_decode_attention of the same query at length P + i + 1 (both from the same
    pool; the two kernels order their sums differently, so the bar is the oracle's)."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    st = _setup(2, 128, 8, 1, [61], 40, (4, 0, 2, 0), seed=41)
    B, C, H, d = st["kc"].shape
    tq.quantize_kv(st["layout"], st["pages"], st["kc"].reshape(B * C, H, d).cuda(),
                   st["vc"].reshape(B * C, H, d).cuda(), torch.from_numpy(st["slots"]).cuda(), st["kcb"], st["vcb"])
    scale = 1.0 / math.sqrt(d)
    pt = torch.from_numpy(st["pt"]).cuda()
    out = tq.prefill_attention(st["layout"], st["pages"], st["q"].cuda(), pt, torch.from_numpy(st["prefix"]).cuda(),
                               scale, st["kcb"], st["vcb"])
    qd = st["q"][0].cuda().contiguous()  # [C, Hq, d]: one decode row per chunk token
    lens = torch.tensor(61 + 1 + np.arange(C), dtype=torch.int32, device="cuda")
    dec = tq.decode_attention(st["layout"], st["pages"], qd, pt.expand(C, -1).contiguous(), lens, scale, st["kcb"],
                              st["vcb"])
    torch.cuda.synchronize()
    err = parity.attention_error(out[0].cpu().numpy(), dec.cpu().numpy().astype(np.float64))
    print(f"prefill vs decode rows: max relative difference {err:.2e}", flush=True)
    assert err <= parity.ATTN_TOL


@pytest.mark.parametrize("kfmt", [(4, 0), (2, 1)], ids=["k4v2", "k2pv2"])
def test_prefill_full_size_8b_layer(kfmt):
    """The 8B layer (8 KV heads, 32 query heads, d = 128, V2; K4, or K2 with the QJL sketch): the last 2048-token
    chunk of a 32768-token prompt after a 30720-token cached prefix, through tq_prefill_chunk; sampled rows of two
    KV heads' query heads against the oracle."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    wl = kvsynth.workloads()[1]
    H, Hq, d, T = wl.kv_heads, wl.q_heads, wl.head_dim, wl.seq_len
    C = 2048
    P = T - C
    kb, km = kfmt
    layout, Lo = parity.make_layout(H, d, kb, km, 2, 0)
    kcb, cbk = parity.device_codebook(d, kb, km, 11)
    vcb, cbv = parity.device_codebook(d, 2, 0, 12)
    pt, npages = kvsynth.page_table(1, T // 16, False)
    pages = torch.zeros(npages * Lo["page_bytes"], dtype=torch.uint8, device="cuda")
    k, v = kvsynth.make_kv(wl, 1, 0, T, device="cuda")
    tq.quantize_kv(layout, pages, k[:P], v[:P], torch.from_numpy(kvsynth.slots_for(pt, 0, 0, P)).cuda(), kcb, vcb)
    g = torch.Generator(device="cuda").manual_seed(9)
    q = torch.randn(1, C, Hq, d, generator=g, device="cuda").to(torch.bfloat16)
    print(f"prefill full size: chunk of 2048 after 30720 cached tokens, K {kfmt}", flush=True)
    out = tq.prefill_chunk(layout, pages, k[P:].unsqueeze(0).contiguous(), v[P:].unsqueeze(0).contiguous(),
                           torch.from_numpy(kvsynth.slots_for(pt, 0, P, T)).cuda(), q, torch.from_numpy(pt).cuda(),
                           torch.tensor([P], dtype=torch.int32, device="cuda"), wl.softmax_scale, kcb, vcb)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    pool = pages.cpu().numpy()
    rng = np.random.default_rng(4)
    rows = sorted(set([0, 1, 31, 32, C - 1] + rng.integers(0, C, 6).tolist()))
    qn = q.double().cpu().numpy()
    G = Hq // H
    ref = attention.prefill_attention(pool, Lo, cbk, cbv, qn, pt, [P], wl.softmax_scale, rows=[(0, i) for i in rows])
    for kvh in (0, 5):
        hs = slice(kvh * G, (kvh + 1) * G)
        err = parity.attention_error(out.cpu().numpy()[0, rows, hs].astype(np.float64), ref[0, rows, hs])
        print(f"  KV head {kvh}: rows {rows}: max relative error {err:.2e}", flush=True)
        assert err <= parity.ATTN_TOL, (kvh, err)


def test_prefill_empty_pages():
    """Page-table entries < 0 or >= num_pages inside a sequence are empty pages: their tokens get no weight (and
    the chunk's tokens that fall in them are not written). Reference: the oracle's dequantized records of the tokens
    of valid pages only, causal, through attention.reference_attention; decode on the same table agrees."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    H, d, Hq, P, C = 2, 128, 8, 70, 40
    fmt = (4, 0, 2, 0)
    st = _setup(H, d, Hq, 1, [P], C, fmt, seed=61)
    npages = st["pages"].numel() // st["Lo"]["page_bytes"]
    pt = st["pt"].copy()
    pt[0, 2] = -1       # inside the prefix
    pt[0, 5] = npages   # inside the chunk (positions 80 .. 95)
    # rebuild the pool through the edited table: the prefix, then the chunk with tq_prefill_chunk
    pages = torch.full_like(st["pages"], 0x5A)
    k, v = parity.seeded_kv(P, H, d, seed=61 * 10)
    tq.quantize_kv(st["layout"], pages, k.cuda(), v.cuda(), torch.from_numpy(kvsynth.slots_for(pt, 0, 0, P)).cuda(),
                   st["kcb"], st["vcb"])
    slots = kvsynth.slots_for(pt, 0, P, P + C)
    scale = 1.0 / math.sqrt(d)
    ptd = torch.from_numpy(pt).cuda()
    out = tq.prefill_chunk(st["layout"], pages, st["kc"].cuda(), st["vc"].cuda(), torch.from_numpy(slots).cuda(),
                           st["q"].cuda(), ptd, torch.tensor([P], dtype=torch.int32, device="cuda"), scale, st["kcb"],
                           st["vcb"])
    qd = st["q"][0].cuda().contiguous()
    lens = torch.tensor(P + 1 + np.arange(C), dtype=torch.int32, device="cuda")
    dec = tq.decode_attention(st["layout"], pages, qd, ptd.expand(C, -1).contiguous(), lens, scale, st["kcb"],
                              st["vcb"])
    torch.cuda.synchronize()
    pool = pages.cpu().numpy()
    T = P + C
    t = np.arange(T)
    valid = (pt[0, t // 16] >= 0) & (pt[0, t // 16] < npages)
    G = Hq // H
    q = st["q"][0].double().numpy()
    ref = np.zeros((C, Hq, d))
    for g in range(H):
        tv = t[valid]
        rk = codec.read_records(pool, st["Lo"], "k", pt[0, tv // 16], tv % 16, g)
        rv = codec.read_records(pool, st["Lo"], "v", pt[0, tv // 16], tv % 16, g)
        K = codec.dequantize(rk["codes"], rk["norm16"], st["cbk"])
        V = codec.dequantize(rv["codes"], rv["norm16"], st["cbv"])
        for i in range(C):
            n = int(np.sum(tv <= P + i))
            ref[i, g * G:(g + 1) * G] = attention.reference_attention(q[i, g * G:(g + 1) * G], K[:n], V[:n], scale)
    err = parity.attention_error(out[0].cpu().numpy(), ref)
    err_dec = parity.attention_error(dec.cpu().numpy(), ref)
    print(f"prefill with empty pages: max relative error {err:.2e} (decode {err_dec:.2e})", flush=True)
    assert err <= parity.ATTN_TOL and err_dec <= parity.ATTN_TOL

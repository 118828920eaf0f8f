"""The dense random (QR) rotation through the C ABI, against the oracle with a dense codebook:

  tq_rotate_rows          rows times a d x d matrix on the matrix cores, against fp64 numpy (relative to
                          the row norm, 2e-6)
  tq_quantize_kv_qr       records (codes, norms, sketch) against the oracle's encoding with R = Q, under the
                          code / norm / sketch rules of the other quantize tests
  tq_decode_attention_qr  against the oracle's decode attention (R = Q for K and V) run on the GPU's own
                          pool, max relative error <= 2e-3
"""
import math

import numpy as np
import pytest

import kvsynth
from oracle import attention, codec, rotation
from tests import parity

pytestmark = pytest.mark.gpu


def qr_codebooks(d, kb, km, vb, vm, seed):
    """Device codebook blobs, device fwd/inv matrices and the oracle's dense codebooks for K and V."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    out = {}
    for which, bits, mode, s in (("k", kb, km, seed), ("v", vb, vm, seed + 1)):
        sw = kvsynth.rotation_signs(s, d)
        S = kvsynth.qjl_projection(s, d) if mode == codec.PROD else None
        G = kvsynth.qr_gaussian(s, d)
        fwd, inv = tq.qr_rotation(d, G, sw)
        out[which] = dict(blob=torch.from_numpy(tq.build_codebook(d, bits, mode, sw, S)).cuda(),
                          fwd=torch.from_numpy(fwd).cuda(), inv=torch.from_numpy(inv).cuda(),
                          cb=codec.make_codebook(d, bits, mode, sw, S, dense=rotation.qr_rotation(G)))
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_rotate_rows_matches_fp64(d, dtype):
    import torch
    import kv_cache_quantization_wht_amd as tq

    print(f"rotate_rows d={d} {dtype}", flush=True)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    fwd, _ = tq.qr_rotation(d, kvsynth.qr_gaussian(7, d))
    g = torch.Generator().manual_seed(8)
    # row scales over several decades (fp16: within its range)
    spread, spike = (1.5, 30.0) if dtype == "f16" else (3.0, 1e3)
    for rows in (1, 15, 16, 17, 1000):
        x = torch.randn(rows, d, generator=g) * torch.exp(torch.randn(rows, 1, generator=g) * spread)
        x[0, :] = 0.0  # a zero row
        if rows > 2:
            x[2, 5] = spike * x[2].abs().max()  # one spike
        x = x.to(tdt)
        assert torch.isfinite(x).all()
        y = tq.rotate_rows(d, torch.from_numpy(fwd).cuda(), x.cuda()).cpu().double().numpy()
        ref = x.double().numpy() @ fwd.astype(np.float64).T
        scale = np.maximum(np.linalg.norm(x.double().numpy(), axis=1), 1e-300)
        err = np.abs(y - ref).max(axis=1) / scale
        assert np.all(y[0] == 0.0)
        assert err.max() <= 2e-6, (rows, err.max())


FORMATS = [  # (k_bits, k_mode, v_bits, v_mode)
    (4, 0, 2, 0),
    (3, 0, 3, 0),
    (2, 1, 2, 0),
    (8, 0, 8, 0),
]


def build_qr_cache(H, d, Hq, B, lens, fmt, seed, dtype="bf16", pps=None):
    import torch
    import kv_cache_quantization_wht_amd as tq

    kb, km, vb, vm = fmt
    layout, Lo = parity.make_layout(H, d, kb, km, vb, vm)
    c = qr_codebooks(d, kb, km, vb, vm, seed)
    npp = max(1, max((l + 15) // 16 for l in lens)) if pps is None else pps
    pt, npages = kvsynth.page_table(B, npp, True, seed=seed + 4, extra_pages=1)
    pages = torch.full((npages * Lo["page_bytes"],), 0x5A, dtype=torch.uint8, device="cuda")
    encs = []
    for b in range(B):
        if lens[b] == 0:
            continue
        k, v = parity.seeded_kv(lens[b], H, d, seed=seed * 10 + b, dtype=dtype)
        slots = kvsynth.slots_for(pt, b, 0, lens[b])
        tq.quantize_kv_qr(layout, pages, k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), c["k"]["blob"],
                          c["v"]["blob"], c["k"]["fwd"], c["v"]["fwd"])
        encs.append((b, slots, k.double().numpy(), v.double().numpy()))
    torch.cuda.synchronize()
    return dict(layout=layout, Lo=Lo, c=c, pt=pt, pages=pages, encs=encs, lens=np.array(lens, np.int32))


CASES = [  # name, H, d, Hq, B, lens, pages_per_split
    ("d128-gqa4", 2, 128, 8, 2, [300, 47], 0),
    ("d64-gqa8-splits", 1, 64, 8, 3, [0, 90, 33], 2),
    ("d128-mha-splits", 4, 128, 4, 1, [200], 4),
]


@pytest.mark.parametrize("fmt", FORMATS, ids=[f"k{f[0]}{'p' if f[1] else ''}v{f[2]}" for f in FORMATS])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_qr_quantize_and_attention(case, fmt):
    import torch
    import kv_cache_quantization_wht_amd as tq

    name, H, d, Hq, B, lens, pps = case
    print(f"qr case {name} fmt {fmt}", flush=True)
    st = build_qr_cache(H, d, Hq, B, lens, fmt, seed=len(name) + 7 * fmt[0])
    Lo, c = st["Lo"], st["c"]
    pool = st["pages"].cpu().numpy()
    rep = parity.Report()
    for b, slots, k, v in st["encs"]:
        page, slot = slots // 16, slots % 16
        for h in range(H):
            for which, x in (("k", k), ("v", v)):
                got = codec.read_records(pool, Lo, which, page, slot, h)
                one = parity.Report()
                parity.compare_records(got, codec.encode(x[:, h, :], c[which]["cb"]), c[which]["cb"], one, which)
                for key, val in one.items():
                    rep[key] = rep.get(key, 0) + val
    print(f"  records {rep}", flush=True)
    g = torch.Generator().manual_seed(5)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    out = tq.decode_attention_qr(st["layout"], st["pages"], q.cuda(), torch.from_numpy(st["pt"]).cuda(),
                                 torch.from_numpy(st["lens"]).cuda(), scale, c["k"]["blob"], c["v"]["blob"],
                                 c["k"]["fwd"], c["v"]["inv"], pages_per_split=pps)
    torch.cuda.synchronize()
    ref = attention.decode_attention(pool, Lo, c["k"]["cb"], c["v"]["cb"], q.double().numpy(), st["pt"], st["lens"],
                                     scale)
    err = parity.attention_error(out.cpu().numpy().astype(np.float64), ref)
    print(f"  attention max relative error {err:.2e}", flush=True)
    assert err <= parity.ATTN_TOL


def test_qr_full_size_8b_layer():
    """The 8B single-layer shape at full length (32768 tokens, 8 KV heads, 32 query heads, K4/V2) through
    tq_quantize_kv_qr and tq_decode_attention_qr in the automatic split plan: sampled records of every KV
    head and two KV heads' outputs against the oracle."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    wl = kvsynth.workloads()[1]
    H, Hq, d, T = wl.kv_heads, wl.q_heads, wl.head_dim, wl.seq_len
    layout, Lo = parity.make_layout(H, d, 4, 0, 2, 0)
    c = qr_codebooks(d, 4, 0, 2, 0, seed=11)
    pps = (T + 15) // 16
    pt, npages = kvsynth.page_table(1, pps, False)
    pages = torch.zeros(npages * Lo["page_bytes"], dtype=torch.uint8, device="cuda")
    k, v = kvsynth.make_kv(wl, 1, 0, T, device="cuda")
    tq.quantize_kv_qr(layout, pages, k, v, torch.from_numpy(kvsynth.slots_for(pt, 0, 0, T)).cuda(), c["k"]["blob"],
                      c["v"]["blob"], c["k"]["fwd"], c["v"]["fwd"])
    q = kvsynth.make_q(wl, 1, 0, 1, device="cuda")
    out = tq.decode_attention_qr(layout, pages, q, torch.from_numpy(pt).cuda(),
                                 torch.tensor([T], dtype=torch.int32, device="cuda"), wl.softmax_scale,
                                 c["k"]["blob"], c["v"]["blob"], c["k"]["fwd"], c["v"]["inv"])
    torch.cuda.synchronize()
    pool = pages.cpu().numpy()
    rng = np.random.default_rng(3)
    t = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 200)]))
    kt, vt = k[t].double().cpu().numpy(), v[t].double().cpu().numpy()
    rep = parity.Report()
    for h in range(H):
        for which, x in (("k", kt), ("v", vt)):
            got = codec.read_records(pool, Lo, which, pt[0, t // 16], t % 16, h)
            one = parity.Report()
            parity.compare_records(got, codec.encode(x[:, h, :], c[which]["cb"]), c[which]["cb"], one, which)
            for key, val in one.items():
                rep[key] = rep.get(key, 0) + val
    print(f"  records {rep}", flush=True)
    G = Hq // H
    for g in (0, 6):
        heads = [(0, hh) for hh in range(g * G, (g + 1) * G)]
        ref = attention.decode_attention(pool, Lo, c["k"]["cb"], c["v"]["cb"], q.double().cpu().numpy(), pt, [T],
                                         wl.softmax_scale, heads=heads)
        err = parity.attention_error(out.cpu().numpy()[:, g * G:(g + 1) * G].astype(np.float64),
                                     ref[:, g * G:(g + 1) * G])
        print(f"  KV head {g}: max relative error {err:.2e}", flush=True)
        assert err <= parity.ATTN_TOL, (g, err)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [(4, 2), (3, 3), (1, 8)])
def test_qr_fused_quantize_matches_two_passes(d, bits):
    """MSE keys and values: tq_quantize_kv_qr rotates inside the quantize kernel; its pages are byte-identical to
    tq_rotate_rows followed by tq_quantize_kv over the fp32 rows (the same arithmetic), ragged token count."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    kb, vb = bits
    H, n = 3, 333
    print(f"qr fused d={d} bits={bits}", flush=True)
    layout, Lo = parity.make_layout(H, d, kb, 0, vb, 0)
    c = qr_codebooks(d, kb, 0, vb, 0, seed=21)
    npages = (n + 15) // 16 + 1
    k, v = parity.seeded_kv(n, H, d, seed=22, dtype="bf16")
    k, v = k.cuda(), v.cuda()
    slots = torch.arange(n, dtype=torch.int64, device="cuda") + 16  # from page 1
    fused = torch.full((npages * Lo["page_bytes"],), 0x33, dtype=torch.uint8, device="cuda")
    tq.quantize_kv_qr(layout, fused, k, v, slots, c["k"]["blob"], c["v"]["blob"], c["k"]["fwd"], c["v"]["fwd"])
    two = torch.full_like(fused, 0x33)
    kr = tq.rotate_rows(d, c["k"]["fwd"], k)
    vr = tq.rotate_rows(d, c["v"]["fwd"], v)
    tq.quantize_kv(layout, two, kr, vr, slots, c["k"]["blob"], c["v"]["blob"])
    torch.cuda.synchronize()
    assert torch.equal(fused, two)

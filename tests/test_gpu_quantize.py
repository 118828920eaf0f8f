"""GPU quantize-on-write (tq_quantize_kv through the C ABI) against the CPU oracle."""
import numpy as np
import pytest

import kvsynth
from oracle import codec
from tests import parity

pytestmark = pytest.mark.gpu

CASES = [
    # H, d, k_bits, k_mode, v_bits, v_mode, dtype
    (1, 64, 4, 0, 2, 0, "f32"),
    (8, 128, 4, 0, 2, 0, "bf16"),
    (8, 128, 3, 0, 3, 0, "bf16"),
    (8, 128, 2, 1, 2, 0, "bf16"),
    (2, 128, 8, 0, 8, 0, "bf16"),
    (3, 128, 1, 0, 4, 0, "f16"),
    (2, 64, 3, 1, 1, 0, "f32"),
    (2, 64, 8, 0, 3, 0, "bf16"),
    (2, 128, 4, 1, 2, 1, "f32"),
    # 8-bit work-groups hold 8 passes of tokens, the others 2: several work-groups per head with ragged tails, and
    # a layer whose K and V widths take separate launches
    (2, 128, 8, 0, 8, 0, "bf16", 1301),
    (3, 128, 8, 0, 2, 0, "bf16", 1301),
    (2, 64, 4, 0, 8, 0, "f16", 2333),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "H{}d{}-K{}{}-V{}{}-{}{}".format(
    c[0], c[1], c[2], "p" if c[3] else "m", c[4], "p" if c[5] else "m", c[6], f"-T{c[7]}" if len(c) > 7 else ""))
def test_quantize_matches_oracle(case):
    H, d, kb, km, vb, vm, dt = case[:7]
    print(f"quantize case {case}", flush=True)
    layout, Lo = parity.make_layout(H, d, kb, km, vb, vm)
    n_tok = case[7] if len(case) > 7 else 301
    num_pages = (n_tok * 5 // 4 + 15) // 16  # a quarter of the slots left free (24 pages for 301 tokens)
    k, v = parity.seeded_kv(n_tok, H, d, seed=H * 1000 + d + 10 * kb + vb, dtype=dt)
    rng = np.random.Generator(np.random.Philox(5))
    slots = rng.permutation(num_pages * 16)[:n_tok].astype(np.int64)
    slots[[7, 100, 250]] = -1  # skipped tokens
    slots[11] = num_pages * 16 + 3  # out of range -> skipped
    kcb_dev, cbk = parity.device_codebook(d, kb, km, seed=11)
    vcb_dev, cbv = parity.device_codebook(d, vb, vm, seed=12)
    pages = parity.gpu_quantize_into_pool(layout, Lo, num_pages * Lo["page_bytes"], k, v, slots, kcb_dev, vcb_dev)
    pool = pages.cpu().numpy()

    # untouched bytes keep the fill pattern
    mask = parity.written_mask(Lo, num_pages, slots, H)
    assert np.all(pool[~mask] == 0xA5)

    rep = parity.Report()
    keep = (slots >= 0) & (slots < num_pages * 16)
    enc_k = parity.encode_all(k.float().numpy()[keep], cbk)
    enc_v = parity.encode_all(v.float().numpy()[keep], cbv)
    s = slots[keep]
    for h in range(H):
        for which, enc, cb in (("k", enc_k[h], cbk), ("v", enc_v[h], cbv)):
            got = codec.read_records(pool, Lo, which, s // 16, s % 16, h)
            parity.compare_records(got, enc, cb, rep, f"{which}{h}")
    print(rep)


def test_quantize_deterministic_and_idempotent():
    """Same input -> same bytes, on repeat and when the same tokens are written again (append path)."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    H, d = 8, 128
    layout, Lo = parity.make_layout(H, d, 4, 0, 2, 0)
    k, v = parity.seeded_kv(64, H, d, seed=3)
    slots = np.arange(64, dtype=np.int64)
    kcb, _ = parity.device_codebook(d, 4, 0, seed=1)
    vcb, _ = parity.device_codebook(d, 2, 0, seed=1)
    p1 = parity.gpu_quantize_into_pool(layout, Lo, 4 * Lo["page_bytes"], k, v, slots, kcb, vcb)
    p2 = parity.gpu_quantize_into_pool(layout, Lo, 4 * Lo["page_bytes"], k, v, slots, kcb, vcb)
    assert torch.equal(p1, p2)
    # one token at a time (decode-step appends) gives the same bytes as one batched call
    p3 = torch.full_like(p1, 0xA5)
    for t in range(64):
        tq.quantize_kv(layout, p3, k[t:t + 1].cuda(), v[t:t + 1].cuda(), torch.tensor([t], dtype=torch.int64).cuda(), kcb, vcb)
    torch.cuda.synchronize()
    assert torch.equal(p1, p3)


def test_quantize_noncontiguous_token_stride():
    """K/V rows taken from a wider buffer (token stride > heads * head_dim)."""
    import torch
    import kv_cache_quantization_wht_amd as tq

    H, d = 2, 128
    layout, Lo = parity.make_layout(H, d, 3, 0, 3, 0)
    k, v = parity.seeded_kv(40, H, d, seed=9)
    wide = torch.zeros(40, 3 * H, d, dtype=k.dtype)
    wide[:, :H] = k
    wide[:, H:2 * H] = v
    kcb, _ = parity.device_codebook(d, 3, 0, seed=2)
    vcb, _ = parity.device_codebook(d, 3, 0, seed=3)
    slots = torch.arange(40, dtype=torch.int64).cuda()
    pa = torch.zeros(3 * Lo["page_bytes"], dtype=torch.uint8, device="cuda")
    pb = torch.zeros_like(pa)
    wd = wide.cuda()
    tq.quantize_kv(layout, pa, wd[:, :H], wd[:, H:2 * H], slots, kcb, vcb)
    tq.quantize_kv(layout, pb, k.cuda(), v.cuda(), slots, kcb, vcb)
    torch.cuda.synchronize()
    assert torch.equal(pa, pb)

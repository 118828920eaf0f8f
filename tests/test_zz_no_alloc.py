"""tq_decode_attention_noalloc (the decode entry point that allocates nothing: its split partials live in the
library's fixed device array) against tq_decode_attention with a caller workspace, through the C ABI: two calls in
a row on one device, the second with a smaller input, each within the attention bar of the other (they run the same
kernels on the same plan, so the outputs are in fact identical) and of the oracle."""
import math

import numpy as np
import pytest

import kvsynth
from oracle import attention
from tests import parity

pytestmark = pytest.mark.gpu


def _case(H, d, Hq, B, lens, kb, vb, seed):
    import torch
    import kv_cache_quantization_wht_amd as tq

    layout, Lo = parity.make_layout(H, d, kb, 0, vb, 0)
    pps = max((l + 15) // 16 for l in lens)
    pt, npages = kvsynth.page_table(B, pps, True, seed=seed + 4, extra_pages=2)
    kcb, cbk = parity.device_codebook(d, kb, 0, seed=seed + 1)
    vcb, cbv = parity.device_codebook(d, vb, 0, seed=seed + 2)
    pages = torch.zeros(npages * Lo["page_bytes"], dtype=torch.uint8, device="cuda")
    for b in range(B):
        k, v = parity.seeded_kv(lens[b], H, d, seed=seed * 100 + b)
        tq.quantize_kv(layout, pages, k.cuda(), v.cuda(), torch.from_numpy(kvsynth.slots_for(pt, b, 0, lens[b])).cuda(),
                       kcb, vcb)
    g = torch.Generator().manual_seed(seed + 77)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16).cuda()
    return dict(layout=layout, Lo=Lo, pages=pages, pt=torch.from_numpy(pt).cuda(), ptn=pt, lens=lens,
                sl=torch.tensor(lens, dtype=torch.int32, device="cuda"), q=q, kcb=kcb, vcb=vcb, cbk=cbk, cbv=cbv)


def test_noalloc_matches_workspace_entry_point_twice():
    import torch
    import kv_cache_quantization_wht_amd as tq

    scale = 1 / math.sqrt(128)
    # the second call is smaller (fewer sequences, shorter, fewer runs) and finds the first call's partials in the
    # array; pages_per_split 4 forces several runs per sequence, so the partials are used
    for name, args, pps in (("large", (2, 128, 8, 3, [900, 333, 47], 4, 2, 5), 4),
                            ("small", (2, 128, 8, 1, [130], 4, 2, 6), 4),
                            ("auto-split", (8, 128, 32, 1, [2000], 4, 2, 7), 0)):
        print(f"noalloc case {name}", flush=True)
        c = _case(*args)
        B, Hq = c["q"].shape[0], c["q"].shape[1]
        need = tq.decode_workspace_bytes(c["layout"], B, Hq, c["pt"].shape[1], pps)
        assert need <= tq.NOALLOC_MAX_BYTES
        ref_out = tq.decode_attention(c["layout"], c["pages"], c["q"], c["pt"], c["sl"], scale, c["kcb"], c["vcb"],
                                      pages_per_split=pps)
        out = torch.full_like(ref_out, float("nan"))
        tq.decode_attention_noalloc(c["layout"], c["pages"], c["q"], c["pt"], c["sl"], scale, c["kcb"], c["vcb"], out,
                                    pages_per_split=pps)
        torch.cuda.synchronize()
        a = out.cpu().numpy().astype(np.float64)
        r = ref_out.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(a))
        err = parity.attention_error(a, r)
        orc = attention.decode_attention(c["pages"].cpu().numpy(), c["Lo"], c["cbk"], c["cbv"],
                                         c["q"].cpu().double().numpy(), c["ptn"], np.array(c["lens"]), scale)
        err_o = parity.attention_error(a, orc)
        print(f"  {name}: against tq_decode_attention {err:.2e} (identical: {bool(np.array_equal(a, r))}), "
              f"against the oracle {err_o:.2e}", flush=True)
        assert err <= parity.ATTN_TOL and err_o <= parity.ATTN_TOL
        assert np.array_equal(a, r)

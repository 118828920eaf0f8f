"""Brute-force GQA decode attention over the packed cache, in fp64.

Sources
  "Why the KV Cache Exists", "The KV Cache Solution" and "What's in the KV Cache":
    at each generation step the new token's query attends over the keys and values
    of every cached token of the sequence, per layer and per KV head (Llama-3.1
    uses 8 KV heads shared by the query heads, i.e. grouped-query attention).
  "Where This Fits in the Inference Stack", "TensorRT-LLM: Why Integration Is a
    Kernel Problem": the attention reads the quantized cache and dequantizes it
    (table lookup) before the score computation.
  "Closing - The Three-Step Summary", Step 1: the rotation keeps inner products, so
    scores may equally be formed in the rotated domain.

Readings adopted: query head h uses KV head floor(h / G), G = Hq / Hkv (the Llama
convention); no mask beyond the sequence length; a sequence of length 0 yields a
zero output. ``decode_attention`` dequantizes every cached vector back to the
original domain and applies softmax(scale * q . k) v exactly as defined.
``decode_attention_rotated`` forms the same quantity in the rotated domain (query
rotated once, values accumulated rotated, one inverse rotation at the end) and is
used to check the first against a second route. ``prefill_attention`` is the
causal attention of a chunk of new tokens over the same cache (a causal mask
in place of the sequence length; its reading is stated on the function).
"""
from __future__ import annotations

import math

import numpy as np

from . import codec

PAGE_TOKENS = codec.PAGE_TOKENS


def gather(pool, L, which, page_row, seq_len, head) -> dict:
    """Records of tokens 0..seq_len-1 of one sequence (page-table row) for one KV head."""
    t = np.arange(seq_len)
    pages = np.asarray(page_row, dtype=np.int64)[t // PAGE_TOKENS]
    return codec.read_records(pool, L, which, pages, t % PAGE_TOKENS, head)


def _softmax_weights(logits):
    m = np.max(logits, axis=-1, keepdims=True)
    e = np.exp(logits - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def decode_attention(pool, L, cb_k, cb_v, q, page_table, seq_lens, scale, heads=None):
    """out[b, h, :] = sum_t softmax_t(scale * <q[b,h], khat_t>) vhat_t  (fp64).

    ``heads`` optionally restricts the computation to a list of (b, h) pairs; other
    outputs are left as NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = L["H"]
    G = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    want = None if heads is None else set(map(tuple, heads))
    for b in range(B):
        T = int(seq_lens[b])
        for g in range(Hkv):
            hs = [h for h in range(g * G, (g + 1) * G) if want is None or (b, h) in want]
            if not hs:
                continue
            if T == 0:
                out[b, hs] = 0.0
                continue
            rk = gather(pool, L, "k", page_table[b], T, g)
            rv = gather(pool, L, "v", page_table[b], T, g)
            K = codec.dequantize(rk["codes"], rk["norm16"], cb_k, rk.get("gamma16"), rk.get("qjl"))
            V = codec.dequantize(rv["codes"], rv["norm16"], cb_v, rv.get("gamma16"), rv.get("qjl"))
            logits = scale * (q[b, hs] @ K.T)
            out[b, hs] = _softmax_weights(logits) @ V
    return out


def decode_attention_rotated(pool, L, cb_k, cb_v, q, page_table, seq_lens, scale):
    """Same result, computed with scores and value sums in the rotated domain."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = L["H"]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    q_rot = cb_k.rotate(q.reshape(-1, d)).reshape(B, Hq, d)
    for b in range(B):
        T = int(seq_lens[b])
        if T == 0:
            continue
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            rk = gather(pool, L, "k", page_table[b], T, g)
            rv = gather(pool, L, "v", page_table[b], T, g)
            Kr = codec.dequantize_rotated(rk["codes"], rk["norm16"], cb_k, rk.get("gamma16"), rk.get("qjl"))
            Vr = codec.dequantize_rotated(rv["codes"], rv["norm16"], cb_v, rv.get("gamma16"), rv.get("qjl"))
            w = _softmax_weights(scale * (q_rot[b, hs] @ Kr.T))
            out[b, hs] = cb_v.unrotate(w @ Vr)
    return out


def prefill_attention(pool, L, cb_k, cb_v, q, page_table, prefix_lens, scale, rows=None):
    """Causal attention of a chunk of new tokens over the packed cache (fp64).

    Sources: "Where This Fits in the Inference Stack", "Decode Throughput vs. Time to
    First Token" (prefill attention over long contexts is the bandwidth-bound regime
    the compressed cache also relieves); "Why the KV Cache Exists", "The KV Cache
    Solution" and "Prefix Caching" (the prompt's keys and values are computed once,
    stored, and later tokens attend to the stored prefix).

    Reading adopted: the chunk's own keys and values are written to the cache first
    (quantize-on-write), and every query reads them back quantized, like the prefix.
    q[b, i] is the query of the chunk's token i of sequence b, at position
    prefix_lens[b] + i; it attends to positions 0 .. prefix_lens[b] + i, itself
    included:
        out[b, i, h] = sum_{t <= P_b + i} softmax_t(scale <q[b,i,h], khat_t>) vhat_t
    with khat, vhat of KV head floor(h / G). ``rows`` optionally restricts the
    computation to a list of (b, i) pairs; other rows are left as NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, C, Hq, d = q.shape
    Hkv = L["H"]
    G = Hq // Hkv
    out = np.full((B, C, Hq, d), np.nan)
    for b in range(B):
        P = int(prefix_lens[b])
        want = list(range(C)) if rows is None else sorted({int(i) for bb, i in rows if int(bb) == b})
        if not want:
            continue
        pos = P + np.asarray(want)                       # position of each wanted query
        T = int(pos.max()) + 1                           # cached tokens any of them may see
        allowed = np.arange(T)[None, :] <= pos[:, None]  # [query, key]: causal, own token included
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            rk = gather(pool, L, "k", page_table[b], T, g)
            rv = gather(pool, L, "v", page_table[b], T, g)
            K = codec.dequantize(rk["codes"], rk["norm16"], cb_k, rk.get("gamma16"), rk.get("qjl"))
            V = codec.dequantize(rv["codes"], rv["norm16"], cb_v, rv.get("gamma16"), rv.get("qjl"))
            logits = scale * (q[b][want][:, hs] @ K.T)   # [query, head, key]
            logits = np.where(allowed[:, None, :], logits, -np.inf)
            out[b, want, hs] = _softmax_weights(logits) @ V
    return out


def reference_attention(q, K, V, scale):
    """softmax(scale q K^T) V for one query block q (G, d), K, V (T, d), all fp64."""
    return _softmax_weights(scale * (np.asarray(q) @ np.asarray(K).T)) @ np.asarray(V)


def relative_error(out, ref):
    """max over (b, h) of ||out - ref||_inf / ||ref||_inf (rows with zero reference use abs error)."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(out - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))

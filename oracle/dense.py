"""Uncompressed (bf16) paged KV cache and decode attention over it, in fp64 - the oracle of the comparator.

Test infrastructure only: read by the tests, the smoke check and the benchmark's CPU baseline.

Sources
  "Where This Fits in the Inference Stack", "What Changes When KV Cache Is 4x Smaller": decode reads the
    whole KV cache from HBM at every step; the compressed cache is measured against an uncompressed one.
  "Why the KV Cache Exists", "The KV Cache Solution": the new token's query attends over the keys and
    values of every cached token, per KV head (grouped-query attention, as in the compressed oracle).
  "What About PagedAttention?": the cache lives in fixed-size pages, allocated on demand.

Readings: a page holds 16 token slots of every KV head of a layer, K as [head][slot][d] bf16 then V as
[head][d][slot] bf16 (the values of each head transposed within the page); inputs are rounded to bf16 to
nearest, ties to even, from their fp32 value; attention is softmax(scale * q . k) v in fp64 over the
stored bf16 values. Parity pins: tests/pins.py (check_dense_*).
"""
from __future__ import annotations

import numpy as np

from . import attention

PAGE_TOKENS = 16


def page_layout(num_kv_heads: int, head_dim: int) -> dict:
    """Byte offsets of the K and V blocks of a dense page, and its size."""
    block = num_kv_heads * PAGE_TOKENS * head_dim * 2
    return {"H": num_kv_heads, "d": head_dim, "k": 0, "v": block, "page_bytes": 2 * block}


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of x rounded to nearest, ties to even, from its fp32 value."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _k_index(L, page, slot, head):
    """Element index (in bf16 units) of K[head][slot][0] of each page."""
    return (np.asarray(page, np.int64) * L["page_bytes"] + L["k"]) // 2 + (head * PAGE_TOKENS + np.asarray(slot)) * L["d"]


def _v_index(L, page, slot, head):
    """Element index (in bf16 units) of V[head][0][slot] of each page (coordinate i at + i * 16)."""
    return (np.asarray(page, np.int64) * L["page_bytes"] + L["v"]) // 2 + head * L["d"] * PAGE_TOKENS + np.asarray(slot)


def write(pool: np.ndarray, L: dict, slots, head: int, k, v) -> None:
    """Store the rows k, v [n, d] of KV head ``head`` at the global slots (page * 16 + offset)."""
    slots = np.asarray(slots, dtype=np.int64)
    words = pool.view(np.uint16)
    page, slot = slots // PAGE_TOKENS, slots % PAGE_TOKENS
    d = L["d"]
    ki = _k_index(L, page, slot, head)[:, None] + np.arange(d)[None, :]
    vi = _v_index(L, page, slot, head)[:, None] + (np.arange(d) * PAGE_TOKENS)[None, :]
    words[ki] = bf16_bits(k)
    words[vi] = bf16_bits(v)


def gather(pool: np.ndarray, L: dict, page_row, seq_len: int, head: int):
    """K, V [seq_len, d] (fp64) of tokens 0..seq_len-1 of one sequence for one KV head."""
    t = np.arange(seq_len)
    page = np.asarray(page_row, dtype=np.int64)[t // PAGE_TOKENS]
    slot = t % PAGE_TOKENS
    words = pool.view(np.uint16)
    d = L["d"]
    K = bf16_value(words[_k_index(L, page, slot, head)[:, None] + np.arange(d)[None, :]])
    V = bf16_value(words[_v_index(L, page, slot, head)[:, None] + (np.arange(d) * PAGE_TOKENS)[None, :]])
    return K, V


def decode_attention(pool, L, q, page_table, seq_lens, scale, heads=None):
    """out[b, h] = softmax_t(scale * <q[b, h], k_t>) v_t over the seq_lens[b] cached tokens (fp64);
    query head h reads KV head h // G. ``heads`` optionally restricts the (b, h) pairs computed."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    G = Hq // L["H"]
    out = np.full((B, Hq, d), np.nan)
    want = None if heads is None else set(map(tuple, heads))
    for b in range(B):
        T = int(seq_lens[b])
        for g in range(L["H"]):
            hs = [h for h in range(g * G, (g + 1) * G) if want is None or (b, h) in want]
            if not hs:
                continue
            if T == 0:
                out[b, hs] = 0.0
                continue
            K, V = gather(pool, L, page_table[b], T, g)
            out[b, hs] = attention.reference_attention(q[b, hs], K, V, scale)
    return out

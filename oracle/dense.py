"""Uncompressed paged KV caches (bf16, and FP8 E4M3 with a per-tensor scale) and decode attention over
them, in fp64 - the oracle of the comparators.

Test infrastructure only: read by the tests, the smoke check and the benchmark's CPU baseline.

Sources
  "Where This Fits in the Inference Stack", "What Changes When KV Cache Is 4x Smaller": decode reads the
    whole KV cache from HBM at every step; the compressed cache is measured against an uncompressed one.
  "Who Should Care" (its KV8 line), "The Three Layers of Compression" (the KV cache layer), "Quality vs.
    Compression: The Full Comparison": an 8-bit floating-point KV cache is the hardware-native 2x baseline
    that serving stacks ship today.
  "Why the KV Cache Exists", "The KV Cache Solution": the new token's query attends over the keys and
    values of every cached token, per KV head (grouped-query attention, as in the compressed oracle).
  "What About PagedAttention?": the cache lives in fixed-size pages, allocated on demand.

Readings: a page holds 16 token slots of every KV head of a layer, K as [head][slot][d] then V as
[head][d][slot] (the values of each head transposed within the page), one element = 2 bytes (bf16) or 1
byte (fp8). bf16: inputs rounded to nearest, ties to even, from their fp32 value. fp8: the pages name no
format, so the OCP 8-bit E4M3 format of serving stacks' FP8 caches is read (bias 7, no infinities, the all-ones
exponent-and-mantissa pattern is NaN, largest finite 448), with one scale per tensor (K, V): the stored byte
encodes the fp32 quotient x / scale, rounded to nearest, ties to even, saturated to +-448; a stored byte
stands for scale * its value. Attention is softmax(scale * q . k) v in fp64 over the stored values.
Parity pins: tests/pins.py (check_dense_*, check_fp8_*).
"""
from __future__ import annotations

import numpy as np

from . import attention

PAGE_TOKENS = 16
FP8_MAX = 448.0


def page_layout(num_kv_heads: int, head_dim: int, fmt: str = "bf16", k_scale: float = 1.0,
                v_scale: float = 1.0) -> dict:
    """Byte offsets of the K and V blocks of a dense page and its size; fp8 layouts carry their scales."""
    elem = {"bf16": 2, "fp8": 1}[fmt]
    block = num_kv_heads * PAGE_TOKENS * head_dim * elem
    return {"H": num_kv_heads, "d": head_dim, "fmt": fmt, "elem": elem, "k": 0, "v": block,
            "page_bytes": 2 * block, "k_scale": float(k_scale), "v_scale": float(v_scale)}


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of x rounded to nearest, ties to even, from its fp32 value."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def fp8_value(bits) -> np.ndarray:
    """Value of E4M3 bytes: exponent field e (bias 7) and mantissa m; e = 0 is subnormal (m * 2^-9);
    exponent and mantissa all ones is NaN."""
    b = np.asarray(bits, dtype=np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e, m = (b >> 3) & 15, b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((b & 0x7F) == 0x7F, np.nan, sign * mag)


def fp8_bits(x, scale: float = 1.0) -> np.ndarray:
    """E4M3 bytes of the fp32 quotient x / scale, rounded to nearest, ties to even, saturated to +-448."""
    y = np.asarray(x, dtype=np.float32) / np.float32(scale)  # fp32 quotient, correctly rounded
    a = np.minimum(np.abs(y.astype(np.float64)), FP8_MAX)
    sign = np.where(np.signbit(y), 0x80, 0)
    # below 2^-6 the grid step is 2^-9 (subnormals); above, 8 steps per binade; both round to nearest even
    sub = a < 2.0 ** -6
    e = np.floor(np.log2(np.where(sub, 1.0, a))).astype(np.int64)
    e = e - (np.exp2(e.astype(np.float64)) > a) + (np.exp2(e + 1.0) <= a)  # exact floor(log2 a)
    m = np.rint(np.where(sub, a * 2.0 ** 9, np.ldexp(a, 3 - e))).astype(np.int64)
    code = np.where(sub, m, ((e + 7) << 3) + m - 8)
    return (sign | code).astype(np.uint8)


def _encode(L, x, scale):
    return bf16_bits(x) if L["fmt"] == "bf16" else fp8_bits(x, scale)


def _decode(L, bits, scale):
    return bf16_value(bits) if L["fmt"] == "bf16" else scale * fp8_value(bits)


def _elems(pool, L):
    return pool.view(np.uint16) if L["elem"] == 2 else pool.view(np.uint8)


def _k_index(L, page, slot, head):
    """Element index of K[head][slot][0] of each page."""
    return (np.asarray(page, np.int64) * L["page_bytes"] + L["k"]) // L["elem"] + (head * PAGE_TOKENS + np.asarray(slot)) * L["d"]


def _v_index(L, page, slot, head):
    """Element index of V[head][0][slot] of each page (coordinate i at + i * 16)."""
    return (np.asarray(page, np.int64) * L["page_bytes"] + L["v"]) // L["elem"] + head * L["d"] * PAGE_TOKENS + np.asarray(slot)


def write(pool: np.ndarray, L: dict, slots, head: int, k, v) -> None:
    """Store the rows k, v [n, d] of KV head ``head`` at the global slots (page * 16 + offset)."""
    slots = np.asarray(slots, dtype=np.int64)
    el = _elems(pool, L)
    page, slot = slots // PAGE_TOKENS, slots % PAGE_TOKENS
    d = L["d"]
    ki = _k_index(L, page, slot, head)[:, None] + np.arange(d)[None, :]
    vi = _v_index(L, page, slot, head)[:, None] + (np.arange(d) * PAGE_TOKENS)[None, :]
    el[ki] = _encode(L, k, L["k_scale"])
    el[vi] = _encode(L, v, L["v_scale"])


def gather(pool: np.ndarray, L: dict, page_row, seq_len: int, head: int):
    """K, V [seq_len, d] (fp64 values the cache stands for) of tokens 0..seq_len-1 of one sequence for one
    KV head."""
    t = np.arange(seq_len)
    page = np.asarray(page_row, dtype=np.int64)[t // PAGE_TOKENS]
    slot = t % PAGE_TOKENS
    el = _elems(pool, L)
    d = L["d"]
    K = _decode(L, el[_k_index(L, page, slot, head)[:, None] + np.arange(d)[None, :]], L["k_scale"])
    V = _decode(L, el[_v_index(L, page, slot, head)[:, None] + (np.arange(d) * PAGE_TOKENS)[None, :]], L["v_scale"])
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

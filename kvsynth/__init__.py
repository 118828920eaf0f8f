"""Seeded synthetic inputs shared by the CPU oracle, the tests and the benchmark.

This module draws random numbers and lays out shapes; it holds none of the
quantizer's or the attention's arithmetic. Both the oracle and the HIP path
receive what it produces as plain inputs:

* the random sign vector of the Walsh-Hadamard rotation and the Gaussian QJL
  projection matrix (the two random objects the method draws once per model
  load, "Why the KV Cache Exists", section "Prefix Caching");
* synthetic K/V/q tensors shaped like Llama-3.1-8B / 70B KV caches ("Why the KV
  Cache Exists", section "What's in the KV Cache"), with the per-channel
  scale structure the community reports ("What the Paper Doesn't Tell You",
  Finding 1 and Finding 4);
* page tables (optionally shuffled) and write slots for 16-token pages.

Sign bits and the QJL projection come from SplitMix64 (Steele, Lea, Flood: "Fast
splittable pseudorandom number generators", OOPSLA 2014), the projection's normals
by the Box-Muller transform (Box and Muller, "A Note on the Generation of Random
Normal Deviates", 1958), so that a seed alone fixes them on every platform (the
library's seeded codebook build draws the same streams from its own code). The
other Gaussian draws (the dense rotation's matrix, bulk K/V/q data) come from
torch generators and are copied, never re-drawn, when both sides need them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
SIGN_STREAM = 0x5349474E  # "SIGN"
QJL_STREAM = 0x514A4C53  # "QJLS"
QR_STREAM = 0x51524753  # "QRGS"
PAGE_TOKENS = 16


def splitmix64(seed: int, n: int) -> np.ndarray:
    """First n outputs of SplitMix64 started from state ``seed`` (uint64 array).

    Output i is mix(seed + (i + 1) * golden_gamma) with Stafford's variant-13
    finaliser, as published with the generator.
    """
    with np.errstate(over="ignore"):
        i = np.arange(1, n + 1, dtype=np.uint64)
        z = (np.uint64(seed & MASK64) + i * np.uint64(GOLDEN_GAMMA)).astype(np.uint64)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def rotation_signs(seed: int, head_dim: int) -> np.ndarray:
    """Random sign vector of the rotation as ``head_dim/32`` uint32 words.

    Bit i (word i//32, LSB first) set means coordinate i is negated. The bits are
    the low-to-high bits of consecutive SplitMix64 outputs of stream
    ``seed ^ "SIGN"``. At head_dim=128 this is the 16-byte sign vector the
    community WHT rotation stores.
    """
    if head_dim % 32:
        raise ValueError("head_dim must be a multiple of 32")
    words64 = splitmix64(seed ^ SIGN_STREAM, (head_dim + 63) // 64)
    w32 = np.empty(2 * len(words64), dtype=np.uint32)
    w32[0::2] = (words64 & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    w32[1::2] = (words64 >> np.uint64(32)).astype(np.uint32)
    return w32[: head_dim // 32].copy()


def qjl_projection(seed: int, head_dim: int, rows: int | None = None) -> np.ndarray:
    """Gaussian projection for the QJL residual sketch: ``rows x head_dim`` fp32, iid N(0,1).

    Outputs 2k and 2k + 1 of SplitMix64 stream ``seed ^ "QJLS"`` give u1, u2 = ((x >> 11) + 0.5) * 2^-53 in (0, 1],
    and the Box-Muller pair r cos(2 pi u2), r sin(2 pi u2) with r = sqrt(-2 ln u1) fills entries 2k and 2k + 1 in
    row-major order (fp64, then rounded to fp32, nearest even). Scalar libm calls, in this order, so that the
    library's C++ draw of the same stream gives the same bits.
    """
    rows = head_dim if rows is None else rows
    n = rows * head_dim
    xs = [int(x) for x in splitmix64(seed ^ QJL_STREAM, n + (n & 1))]
    out = np.empty(n + (n & 1), dtype=np.float64)
    two_pi = 2.0 * math.pi
    for k in range(0, len(xs), 2):
        u1 = (float(xs[k] >> 11) + 0.5) * 2.0 ** -53
        u2 = (float(xs[k + 1] >> 11) + 0.5) * 2.0 ** -53
        r = math.sqrt(-2.0 * math.log(u1))
        t = two_pi * u2
        out[k] = r * math.cos(t)
        out[k + 1] = r * math.sin(t)
    return out[:n].astype(np.float32).reshape(rows, head_dim)


def qr_gaussian(seed: int, head_dim: int) -> np.ndarray:
    """The random draw of the dense (QR) rotation: a ``head_dim x head_dim`` fp64 matrix of iid N(0,1) entries,
    row-major (the orthogonal factor of its QR decomposition is the rotation)."""
    import torch

    g = torch.Generator(device="cpu").manual_seed((seed ^ QR_STREAM) & 0x7FFFFFFFFFFFFFFF)
    return torch.randn(head_dim, head_dim, generator=g, dtype=torch.float64).numpy()


# --------------------------------------------------------------------------------------------
# Workload descriptions (shapes, bit widths and input recipes).
# --------------------------------------------------------------------------------------------


@dataclass
class LayerBits:
    k_bits: int
    k_mode: int  # 0 = MSE, 1 = prod (MSE at bits-1 plus 1-bit QJL residual sketch)
    v_bits: int
    v_mode: int


@dataclass
class Workload:
    name: str
    layers: int
    kv_heads: int
    q_heads: int
    head_dim: int
    batch: int
    seq_len: int
    decode_steps: int
    dtype: str  # "f32" or "bf16"
    recipe: str
    bits: list = field(default_factory=list)  # LayerBits per layer
    shuffled_pages: bool = False
    prefill: bool = False

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def _uniform_bits(n, kb, km, vb, vm):
    return [LayerBits(kb, km, vb, vm) for _ in range(n)]


def workloads() -> list[Workload]:
    """The five synthetic workloads, smallest first."""
    w = []
    w.append(Workload("tiny-d64-gqa4-T1024", 1, 1, 4, 64, 1, 1024, 1, "f32", "outliers8",
                      _uniform_bits(1, 4, 0, 2, 0)))
    w.append(Workload("llama3.1-8b-1layer-T32768", 1, 8, 32, 128, 1, 32768, 128, "bf16", "lognormal-k50",
                      _uniform_bits(1, 4, 0, 2, 0)))
    w.append(Workload("llama3.1-8b-32layer-B32-T8192", 32, 8, 32, 128, 32, 8192, 32, "bf16", "outliers10",
                      _uniform_bits(32, 3, 0, 3, 0)))
    w.append(Workload("prod-k2qjl-B16-T131072", 1, 8, 32, 128, 16, 131072, 16, "bf16", "lognormal-kv",
                      _uniform_bits(1, 2, 1, 2, 0)))
    b70 = [LayerBits(8, 0, 8, 0) if (l < 2 or l >= 78) else LayerBits(4, 0, 2, 0) for l in range(80)]
    w.append(Workload("llama-70b-80layer-B4-T131072", 80, 8, 64, 128, 4, 131072, 64, "bf16", "normal-k100",
                      b70, shuffled_pages=True, prefill=True))
    return w


def data_seed(cfg_index: int, layer: int, which: str) -> int:
    return 1000 * cfg_index + 10 * layer + {"k": 0, "v": 1, "q": 2}[which]


def rotation_seed(layer: int, base: int = 0) -> int:
    return base + layer


def _gen(seed: int, device: str):
    import torch

    return torch.Generator(device=device).manual_seed(seed)


def make_kv(wl: Workload, cfg_index: int, layer: int, n_tok: int, device: str = "cpu", token_offset_seed: int = 0):
    """K and V for ``n_tok`` tokens of one layer: tensors [n_tok, kv_heads, head_dim].

    Recipes (per workload):
      outliers8   : iid N(0,1); two channels (chosen by the data seed) scaled by 8 in K and V.
      lognormal-k50: V ~ N(0,1); K = (50/e) * c * N(0,1), c ~ LogNormal(0,1) per (head, channel),
                    so that E||K|| / E||V|| is about 50.
      outliers10  : iid N(0,1); four channels per (layer, head) scaled by 10.
      lognormal-kv: K and V both N(0,1) times LogNormal(0,1) per-(head, channel) scales.
      normal-k100 : K ~ N(0, 100^2), V ~ N(0, 1).
    """
    import torch

    H, d = wl.kv_heads, wl.head_dim
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    gk = _gen(data_seed(cfg_index, layer, "k") + 7919 * token_offset_seed, device)
    gv = _gen(data_seed(cfg_index, layer, "v") + 7919 * token_offset_seed, device)
    gs = _gen(data_seed(cfg_index, layer, "k") + 555, "cpu")  # channel structure: fixed per layer
    k = torch.randn(n_tok, H, d, generator=gk, device=device, dtype=torch.float32)
    v = torch.randn(n_tok, H, d, generator=gv, device=device, dtype=torch.float32)
    r = wl.recipe
    if r == "outliers8":
        ch = torch.randperm(d, generator=gs)[:2]
        scale = torch.ones(d)
        scale[ch] = 8.0
        k = k * scale.to(device)
        v = v * scale.to(device)
    elif r == "lognormal-k50":
        c = torch.exp(torch.randn(H, d, generator=gs, dtype=torch.float32))
        k = k * (50.0 / math.e) * c.to(device)
    elif r == "outliers10":
        scale = torch.ones(H, d)
        for h in range(H):
            ch = torch.randperm(d, generator=gs)[:4]
            scale[h, ch] = 10.0
        k = k * scale.to(device)
        v = v * scale.to(device)
    elif r == "lognormal-kv":
        ck = torch.exp(torch.randn(H, d, generator=gs, dtype=torch.float32))
        cv = torch.exp(torch.randn(H, d, generator=gs, dtype=torch.float32))
        k = k * ck.to(device)
        v = v * cv.to(device)
    elif r == "normal-k100":
        k = k * 100.0
    else:
        raise ValueError(r)
    return k.to(dt), v.to(dt)


def make_q(wl: Workload, cfg_index: int, layer: int, batch: int, device: str = "cpu", step: int = 0, scale: float = 1.0):
    """Queries [batch, q_heads, head_dim], iid N(0, scale^2) in the workload's dtype."""
    import torch

    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    g = _gen(data_seed(cfg_index, layer, "q") + 7919 * step, device)
    q = torch.randn(batch, wl.q_heads, wl.head_dim, generator=g, device=device, dtype=torch.float32) * scale
    return q.to(dt)


def page_table(batch: int, pages_per_seq: int, shuffled: bool, seed: int = 12345, extra_pages: int = 0):
    """Page table [batch, pages_per_seq] int32 of distinct physical pages, and the pool size.

    Unshuffled: sequence b owns pages b*pages_per_seq + p. Shuffled: a seeded
    random permutation of all physical pages (plus ``extra_pages`` unused ones).
    """
    n = batch * pages_per_seq + extra_pages
    if shuffled:
        rng = np.random.Generator(np.random.Philox(seed))
        perm = rng.permutation(n).astype(np.int32)
    else:
        perm = np.arange(n, dtype=np.int32)
    return perm[: batch * pages_per_seq].reshape(batch, pages_per_seq).copy(), n


def slots_for(page_tab: np.ndarray, b: int, t0: int, t1: int) -> np.ndarray:
    """Global slots (page * 16 + offset) of tokens [t0, t1) of sequence b."""
    t = np.arange(t0, t1)
    return (page_tab[b, t // PAGE_TOKENS].astype(np.int64) * PAGE_TOKENS + (t % PAGE_TOKENS)).astype(np.int64)

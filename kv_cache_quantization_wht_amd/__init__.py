"""Python binding of the TurboQuant KV-cache library (``libtq.so``, C ABI in ``include/tq.h``).

Argument marshalling only: every step of the method runs in the library's HIP kernels (or, for
``build_codebook``, in its host code). PyTorch supplies device memory and streams. Function names
follow the C ABI without the ``tq_`` prefix. The library must have been built
(``python -m kv_cache_quantization_wht_amd.build``); nothing here falls back to another
implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

MSE = 0
PROD = 1
F32, BF16, F16 = 0, 1, 2
PAGE_TOKENS = 16

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")
_LIB = None

C_SYMBOLS = (
    "tq_strerror", "tq_codebook_bytes", "tq_build_codebook", "tq_build_codebook_seeded", "tq_page_layout",
    "tq_quantize_kv",
    "tq_decode_workspace_bytes", "tq_decode_attention", "tq_decode_partial", "tq_decode_combine",
    "tq_decode_step", "tq_decode_step_partial", "tq_decode_attention_noalloc",
    "tq_dense_page_bytes", "tq_dense_write_kv", "tq_dense_decode_workspace_bytes", "tq_dense_decode_attention",
    "tq_dense_fp8_page_bytes", "tq_dense_fp8_write_kv", "tq_dense_fp8_decode_attention",
    "tq_qr_rotation", "tq_rotate_rows", "tq_quantize_kv_qr_workspace_bytes", "tq_quantize_kv_qr",
    "tq_decode_qr_workspace_bytes", "tq_decode_attention_qr",
    "tq_prefill_attention", "tq_prefill_chunk", "tq_stream_read",
)


class _Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("head_dim", "num_kv_heads", "page_tokens", "k_bits", "k_mode", "v_bits", "v_mode")]


class _Offsets(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("k_codes", "k_norms", "k_qjl", "k_gamma", "v_codes", "v_norms", "v_qjl", "v_gamma", "page_bytes")]


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib().tq_strerror(status).decode()} ({status})")


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m kv_cache_quantization_wht_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        lib.tq_strerror.restype = ctypes.c_char_p
        lib.tq_strerror.argtypes = [i32]
        lib.tq_codebook_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        lib.tq_build_codebook.argtypes = [i32, i32, i32, vp, vp, vp, sz]
        lib.tq_build_codebook_seeded.argtypes = [i32, i32, i32, ctypes.c_uint64, vp, sz]
        lib.tq_stream_read.argtypes = [vp, sz, i32, vp, vp]
        lib.tq_page_layout.argtypes = [ctypes.POINTER(_Layout), ctypes.POINTER(_Offsets)]
        lib.tq_quantize_kv.argtypes = [ctypes.POINTER(_Layout), vp, i64, vp, vp, i32, i64, i64, i64, vp, vp, vp, vp]
        lib.tq_decode_workspace_bytes.argtypes = [ctypes.POINTER(_Layout), i32, i32, i32, i32, ctypes.POINTER(sz)]
        lib.tq_decode_attention.argtypes = [ctypes.POINTER(_Layout), vp, i64, vp, i32, i32, i32, vp, i32, vp,
                                            ctypes.c_float, i32, vp, vp, vp, sz, vp, vp]
        lib.tq_decode_partial.argtypes = [ctypes.POINTER(_Layout), vp, i64, vp, i32, i32, i32, vp, i32, vp,
                                            ctypes.c_float, i32, vp, vp, vp, sz, vp, vp]
        lib.tq_decode_combine.argtypes = [ctypes.POINTER(_Layout), vp, i64, vp, i32, i32, i32, vp, i32, vp,
                                            ctypes.c_float, i32, vp, vp, vp, sz, vp, vp]
        lib.tq_decode_attention_noalloc.argtypes = [ctypes.POINTER(_Layout), vp, i64, vp, i32, i32, i32, vp, i32,
                                                    vp, ctypes.c_float, i32, vp, vp, vp, vp]
        for nm in ("tq_decode_step", "tq_decode_step_partial"):
            getattr(lib, nm).argtypes = [ctypes.POINTER(_Layout), vp, i64, vp, vp, i32, vp, i32, i32, i32, vp, i32,
                                         vp, ctypes.c_float, i32, vp, vp, vp, sz, vp, vp]
        lib.tq_dense_page_bytes.argtypes = [i32, i32, ctypes.POINTER(sz)]
        lib.tq_dense_write_kv.argtypes = [i32, i32, vp, i64, vp, vp, i32, i64, vp, vp]
        lib.tq_dense_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
        lib.tq_dense_decode_attention.argtypes = [i32, i32, vp, i64, vp, i32, i32, i32, vp, i32, vp, ctypes.c_float,
                                                  i32, vp, sz, vp, vp]
        f32 = ctypes.c_float
        lib.tq_dense_fp8_page_bytes.argtypes = [i32, i32, ctypes.POINTER(sz)]
        lib.tq_dense_fp8_write_kv.argtypes = [i32, i32, vp, i64, vp, vp, i32, i64, vp, f32, f32, vp]
        lib.tq_dense_fp8_decode_attention.argtypes = [i32, i32, vp, i64, vp, i32, i32, i32, vp, i32, vp, f32, f32, f32,
                                                      i32, vp, sz, vp, vp]
        lay = ctypes.POINTER(_Layout)
        lib.tq_qr_rotation.argtypes = [i32, vp, vp, vp, vp]
        lib.tq_rotate_rows.argtypes = [i32, vp, vp, i32, i64, vp, vp]
        lib.tq_quantize_kv_qr_workspace_bytes.argtypes = [lay, i64, ctypes.POINTER(sz)]
        lib.tq_quantize_kv_qr.argtypes = [lay, vp, i64, vp, vp, i32, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.tq_decode_qr_workspace_bytes.argtypes = [lay, i32, i32, i32, i32, ctypes.POINTER(sz)]
        lib.tq_decode_attention_qr.argtypes = [lay, vp, i64, vp, i32, i32, i32, vp, i32, vp, f32, i32, vp, vp, vp,
                                               vp, vp, sz, vp, vp]
        lib.tq_prefill_attention.argtypes = [lay, vp, i64, vp, i32, i32, i32, i32, vp, i32, vp, f32, vp, vp, vp, vp]
        lib.tq_prefill_chunk.argtypes = [lay, vp, i64, vp, vp, i32, vp, vp, i32, i32, i32, i32, vp, i32, vp, f32, vp,
                                         vp, vp, vp]
        for name in C_SYMBOLS:
            getattr(lib, name).restype = ctypes.c_char_p if name == "tq_strerror" else ctypes.c_int
        _LIB = lib
    return _LIB


def _check(status: int, where: str):
    if status != 0:
        raise TQError(status, where)


@dataclass(frozen=True)
class Layout:
    head_dim: int
    num_kv_heads: int
    k_bits: int
    k_mode: int
    v_bits: int
    v_mode: int
    page_tokens: int = PAGE_TOKENS

    def c(self) -> _Layout:
        return _Layout(self.head_dim, self.num_kv_heads, self.page_tokens, self.k_bits, self.k_mode,
                       self.v_bits, self.v_mode)


def strerror(status: int) -> str:
    return _lib().tq_strerror(status).decode()


def codebook_bytes(head_dim: int, bits: int, mode: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib().tq_codebook_bytes(head_dim, bits, mode, ctypes.byref(out)), "tq_codebook_bytes")
    return out.value


def build_codebook(head_dim: int, bits: int, mode: int, sign_words, qjl_proj=None) -> np.ndarray:
    """Host codebook blob (uint8). ``sign_words``: head_dim/32 uint32; ``qjl_proj``: d x d fp32 (prod)."""
    sw = np.ascontiguousarray(sign_words, dtype=np.uint32)
    pj = None if qjl_proj is None else np.ascontiguousarray(qjl_proj, dtype=np.float32)
    n = codebook_bytes(head_dim, bits, mode)
    blob = np.zeros(n, dtype=np.uint8)
    _check(_lib().tq_build_codebook(head_dim, bits, mode, sw.ctypes.data,
                                    None if pj is None else pj.ctypes.data, blob.ctypes.data, n),
           "tq_build_codebook")
    return blob


def build_codebook_seeded(head_dim: int, bits: int, mode: int, seed: int) -> np.ndarray:
    """Host codebook blob (uint8) with the signs (and in prod mode S) drawn by the library from ``seed``."""
    n = codebook_bytes(head_dim, bits, mode)
    blob = np.zeros(n, dtype=np.uint8)
    _check(_lib().tq_build_codebook_seeded(head_dim, bits, mode, ctypes.c_uint64(seed & (2 ** 64 - 1)),
                                           blob.ctypes.data, n), "tq_build_codebook_seeded")
    return blob


def stream_read(buf, blocks: int, sink, stream=None) -> None:
    """Plain streaming read of the device tensor ``buf`` (tq_stream_read); ``sink``: a device uint32/int32 tensor."""
    _check(_lib().tq_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), blocks, sink.data_ptr(),
                                 _stream(stream)), "tq_stream_read")


def page_layout(layout: Layout) -> dict:
    o = _Offsets()
    _check(_lib().tq_page_layout(ctypes.byref(layout.c()), ctypes.byref(o)), "tq_page_layout")
    return {n: int(getattr(o, n)) for n, _ in _Offsets._fields_}


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_DT = {}


def _dtype_code(t) -> int:
    import torch

    if not _DT:
        _DT.update({torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16})
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _need(t, what, dtype=None, cuda=True):
    if cuda and not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")


def quantize_kv(layout: Layout, pages, k, v, slots, k_cb, v_cb, stream=None) -> None:
    """Quantize K, V [n_tok, num_kv_heads, head_dim] into ``pages`` at global ``slots`` (int64)."""
    import torch

    _need(pages, "pages", torch.uint8)
    _need(slots, "slots", torch.int64)
    _need(k, "k")
    _need(v, "v")
    if k.dtype != v.dtype:
        raise TypeError("k and v must share a dtype")
    if k.dim() != 3 or v.dim() != 3 or k.shape[1:] != (layout.num_kv_heads, layout.head_dim) or v.shape != k.shape:
        raise ValueError("k, v must be [n_tok, num_kv_heads, head_dim]")
    if k.stride(2) != 1 or k.stride(1) != layout.head_dim or v.stride(2) != 1 or v.stride(1) != layout.head_dim:
        raise ValueError("k, v rows must be contiguous per token")
    if not slots.is_contiguous() or slots.numel() != k.shape[0]:
        raise ValueError("slots must be a contiguous int64 vector with one entry per token")
    page_bytes = page_layout(layout)["page_bytes"]
    num_pages = pages.numel() // page_bytes
    _check(_lib().tq_quantize_kv(ctypes.byref(layout.c()), pages.data_ptr(), num_pages, k.data_ptr(), v.data_ptr(),
                                 _dtype_code(k), k.shape[0], k.stride(0), v.stride(0), slots.data_ptr(),
                                 k_cb.data_ptr(), v_cb.data_ptr(), _stream(stream)), "tq_quantize_kv")


def decode_workspace_bytes(layout: Layout, batch: int, num_q_heads: int, max_pages_per_seq: int,
                           pages_per_split: int = 0) -> int:
    out = ctypes.c_size_t()
    _check(_lib().tq_decode_workspace_bytes(ctypes.byref(layout.c()), batch, num_q_heads, max_pages_per_seq,
                                            pages_per_split, ctypes.byref(out)), "tq_decode_workspace_bytes")
    return out.value


def _decode_call(entry: str, layout: Layout, pages, q, page_table, seq_lens, softmax_scale, k_cb, v_cb,
                 workspace, out, pages_per_split, stream):
    import torch

    _need(pages, "pages", torch.uint8)
    _need(q, "q")
    _need(page_table, "page_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 3 or q.shape[2] != layout.head_dim or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, num_q_heads, head_dim] tensor")
    B, Hq, _ = q.shape
    if page_table.dim() != 2 or page_table.shape[0] != B or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous [batch, max_pages_per_seq] int32 tensor")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must hold one int32 per sequence")
    maxp = page_table.shape[1]
    need = decode_workspace_bytes(layout, B, Hq, maxp, pages_per_split)
    if workspace is None:
        if entry != "tq_decode_attention":
            raise ValueError(f"{entry} needs the caller's workspace (shared by the two passes)")
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(B, Hq, layout.head_dim, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor shaped like q")
    page_bytes = page_layout(layout)["page_bytes"]
    num_pages = pages.numel() // page_bytes
    _check(getattr(_lib(), entry)(ctypes.byref(layout.c()), pages.data_ptr(), num_pages, q.data_ptr(),
                                  _dtype_code(q), B, Hq, page_table.data_ptr(), maxp, seq_lens.data_ptr(),
                                  float(softmax_scale), pages_per_split, k_cb.data_ptr(), v_cb.data_ptr(),
                                  workspace.data_ptr(), workspace.numel(), out.data_ptr(), _stream(stream)),
           entry)
    return out


def decode_attention(layout: Layout, pages, q, page_table, seq_lens, softmax_scale, k_cb, v_cb,
                     workspace=None, out=None, pages_per_split: int = 0, stream=None):
    """Decode attention for q [batch, num_q_heads, head_dim]; returns fp32 out of the same shape."""
    return _decode_call("tq_decode_attention", layout, pages, q, page_table, seq_lens, softmax_scale, k_cb, v_cb,
                        workspace, out, pages_per_split, stream)


NOALLOC_MAX_BYTES = 4 << 20  # TQ_DECODE_NOALLOC_MAX_BYTES


def decode_attention_noalloc(layout: Layout, pages, q, page_table, seq_lens, softmax_scale, k_cb, v_cb, out,
                             pages_per_split: int = 0, stream=None):
    """decode_attention with the split partials in the library's fixed device array (tq_decode_attention_noalloc):
    no workspace, and ``out`` (fp32, shaped like q) is the caller's. Calls on one device must not overlap."""
    import torch

    _need(pages, "pages", torch.uint8)
    _need(q, "q")
    _need(page_table, "page_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(out, "out", torch.float32)
    if q.dim() != 3 or q.shape[2] != layout.head_dim or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, num_q_heads, head_dim] tensor")
    B, Hq, _ = q.shape
    if page_table.dim() != 2 or page_table.shape[0] != B or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous [batch, max_pages_per_seq] int32 tensor")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must hold one int32 per sequence")
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor shaped like q")
    num_pages = pages.numel() // page_layout(layout)["page_bytes"]
    _check(_lib().tq_decode_attention_noalloc(ctypes.byref(layout.c()), pages.data_ptr(), num_pages, q.data_ptr(),
                                              _dtype_code(q), B, Hq, page_table.data_ptr(), page_table.shape[1],
                                              seq_lens.data_ptr(), float(softmax_scale), pages_per_split,
                                              k_cb.data_ptr(), v_cb.data_ptr(), out.data_ptr(), _stream(stream)),
           "tq_decode_attention_noalloc")
    return out


def decode_partial(layout: Layout, pages, q, page_table, seq_lens, softmax_scale, k_cb, v_cb, workspace,
                   out=None, pages_per_split: int = 0, stream=None):
    """First pass of decode_attention (split-K scan into ``workspace``); same arguments."""
    return _decode_call("tq_decode_partial", layout, pages, q, page_table, seq_lens, softmax_scale, k_cb, v_cb,
                        workspace, out, pages_per_split, stream)


def decode_combine(layout: Layout, pages, q, page_table, seq_lens, softmax_scale, k_cb, v_cb, workspace,
                   out=None, pages_per_split: int = 0, stream=None):
    """Second pass of decode_attention (merge of the runs, inverse rotation into ``out``); same arguments."""
    return _decode_call("tq_decode_combine", layout, pages, q, page_table, seq_lens, softmax_scale, k_cb, v_cb,
                        workspace, out, pages_per_split, stream)


def decode_step(layout: Layout, pages, k_new, v_new, q, page_table, seq_lens, softmax_scale, k_cb, v_cb,
                workspace=None, out=None, pages_per_split: int = 0, stream=None, first_pass_only: bool = False):
    """Append the new token of each sequence (k_new, v_new [batch, num_kv_heads, head_dim], position
    seq_lens[b] - 1) and run decode attention for q [batch, num_q_heads, head_dim]; returns fp32 out.
    ``first_pass_only`` calls tq_decode_step_partial (finish with decode_combine on the same workspace)."""
    import torch

    _need(pages, "pages", torch.uint8)
    _need(q, "q")
    _need(page_table, "page_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, name)
        if t.dim() != 3 or t.shape[1] != layout.num_kv_heads or t.shape[2] != layout.head_dim or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [batch, num_kv_heads, head_dim] tensor")
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must share a dtype")
    if q.dim() != 3 or q.shape[2] != layout.head_dim or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, num_q_heads, head_dim] tensor")
    B, Hq, _ = q.shape
    if k_new.shape[0] != B or v_new.shape[0] != B:
        raise ValueError("k_new / v_new need one row per sequence")
    if page_table.dim() != 2 or page_table.shape[0] != B or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous [batch, max_pages_per_seq] int32 tensor")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must hold one int32 per sequence")
    maxp = page_table.shape[1]
    need = decode_workspace_bytes(layout, B, Hq, maxp, pages_per_split)
    if workspace is None:
        if first_pass_only:
            raise ValueError("the first pass alone needs the caller's workspace (shared with decode_combine)")
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(B, Hq, layout.head_dim, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor shaped like q")
    num_pages = pages.numel() // page_layout(layout)["page_bytes"]
    entry = "tq_decode_step_partial" if first_pass_only else "tq_decode_step"
    _check(getattr(_lib(), entry)(ctypes.byref(layout.c()), pages.data_ptr(), num_pages, k_new.data_ptr(),
                                 v_new.data_ptr(), _dtype_code(k_new), q.data_ptr(), _dtype_code(q), B, Hq,
                                 page_table.data_ptr(), maxp, seq_lens.data_ptr(), float(softmax_scale),
                                 pages_per_split, k_cb.data_ptr(), v_cb.data_ptr(), workspace.data_ptr(),
                                 workspace.numel(), out.data_ptr(), _stream(stream)), entry)
    return out


# --------------------------------------------------------------------------------------------------
# Uncompressed comparators: the same paged decode attention over a bf16 cache and over an FP8 (E4M3,
# one scale per tensor) cache (K [head][slot][d], V [head][d][slot] per page).
# --------------------------------------------------------------------------------------------------

def dense_page_bytes(head_dim: int, num_kv_heads: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib().tq_dense_page_bytes(head_dim, num_kv_heads, ctypes.byref(out)), "tq_dense_page_bytes")
    return out.value


def dense_fp8_page_bytes(head_dim: int, num_kv_heads: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib().tq_dense_fp8_page_bytes(head_dim, num_kv_heads, ctypes.byref(out)), "tq_dense_fp8_page_bytes")
    return out.value


def _dense_write_args(head_dim, num_kv_heads, pages, k, v, slots):
    import torch

    _need(pages, "pages", torch.uint8)
    _need(slots, "slots", torch.int64)
    _need(k, "k")
    _need(v, "v")
    if k.dtype != v.dtype or k.shape != v.shape or k.dim() != 3 or k.shape[1:] != (num_kv_heads, head_dim):
        raise ValueError("k, v must be [n_tok, num_kv_heads, head_dim] of one dtype")
    if not (k.is_contiguous() and v.is_contiguous() and slots.is_contiguous()) or slots.numel() != k.shape[0]:
        raise ValueError("k, v, slots must be contiguous, one slot per token")


def dense_write_kv(head_dim: int, num_kv_heads: int, pages, k, v, slots, stream=None) -> None:
    """Write K, V [n_tok, num_kv_heads, head_dim] (contiguous) as bf16 into dense ``pages`` at ``slots``."""
    _dense_write_args(head_dim, num_kv_heads, pages, k, v, slots)
    num_pages = pages.numel() // dense_page_bytes(head_dim, num_kv_heads)
    _check(_lib().tq_dense_write_kv(head_dim, num_kv_heads, pages.data_ptr(), num_pages, k.data_ptr(), v.data_ptr(),
                                    _dtype_code(k), k.shape[0], slots.data_ptr(), _stream(stream)), "tq_dense_write_kv")


def dense_fp8_write_kv(head_dim: int, num_kv_heads: int, pages, k, v, slots, k_scale: float, v_scale: float,
                       stream=None) -> None:
    """Write K, V [n_tok, num_kv_heads, head_dim] (contiguous) as E4M3 bytes of x / scale into FP8 dense
    ``pages`` at ``slots``."""
    _dense_write_args(head_dim, num_kv_heads, pages, k, v, slots)
    num_pages = pages.numel() // dense_fp8_page_bytes(head_dim, num_kv_heads)
    _check(_lib().tq_dense_fp8_write_kv(head_dim, num_kv_heads, pages.data_ptr(), num_pages, k.data_ptr(),
                                        v.data_ptr(), _dtype_code(k), k.shape[0], slots.data_ptr(), float(k_scale),
                                        float(v_scale), _stream(stream)), "tq_dense_fp8_write_kv")


def dense_decode_workspace_bytes(head_dim: int, num_kv_heads: int, batch: int, num_q_heads: int,
                                 max_pages_per_seq: int, pages_per_split: int = 0) -> int:
    out = ctypes.c_size_t()
    _check(_lib().tq_dense_decode_workspace_bytes(head_dim, num_kv_heads, batch, num_q_heads, max_pages_per_seq,
                                                  pages_per_split, ctypes.byref(out)), "tq_dense_decode_workspace_bytes")
    return out.value


def _dense_decode_args(head_dim, num_kv_heads, pages, q, page_table, seq_lens, workspace, out, pages_per_split):
    import torch

    _need(pages, "pages", torch.uint8)
    _need(q, "q")
    _need(page_table, "page_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 3 or q.shape[2] != head_dim or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, num_q_heads, head_dim] tensor")
    B, Hq, _ = q.shape
    if page_table.dim() != 2 or page_table.shape[0] != B or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous [batch, max_pages_per_seq] int32 tensor")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must hold one int32 per sequence")
    maxp = page_table.shape[1]
    if workspace is None:
        need = dense_decode_workspace_bytes(head_dim, num_kv_heads, B, Hq, maxp, pages_per_split)
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(B, Hq, head_dim, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor shaped like q")
    return B, Hq, maxp, workspace, out


def dense_decode_attention(head_dim: int, num_kv_heads: int, pages, q, page_table, seq_lens, softmax_scale,
                           workspace=None, out=None, pages_per_split: int = 0, stream=None):
    """Decode attention over a dense bf16 pool for q [batch, num_q_heads, head_dim]; returns fp32 out."""
    B, Hq, maxp, workspace, out = _dense_decode_args(head_dim, num_kv_heads, pages, q, page_table, seq_lens,
                                                     workspace, out, pages_per_split)
    num_pages = pages.numel() // dense_page_bytes(head_dim, num_kv_heads)
    _check(_lib().tq_dense_decode_attention(head_dim, num_kv_heads, pages.data_ptr(), num_pages, q.data_ptr(),
                                            _dtype_code(q), B, Hq, page_table.data_ptr(), maxp, seq_lens.data_ptr(),
                                            float(softmax_scale), pages_per_split, workspace.data_ptr(),
                                            workspace.numel(), out.data_ptr(), _stream(stream)),
           "tq_dense_decode_attention")
    return out


def dense_fp8_decode_attention(head_dim: int, num_kv_heads: int, pages, q, page_table, seq_lens, softmax_scale,
                               k_scale: float, v_scale: float, workspace=None, out=None, pages_per_split: int = 0,
                               stream=None):
    """Decode attention over an FP8 (E4M3, per-tensor scales) dense pool; returns fp32 out."""
    B, Hq, maxp, workspace, out = _dense_decode_args(head_dim, num_kv_heads, pages, q, page_table, seq_lens,
                                                     workspace, out, pages_per_split)
    num_pages = pages.numel() // dense_fp8_page_bytes(head_dim, num_kv_heads)
    _check(_lib().tq_dense_fp8_decode_attention(head_dim, num_kv_heads, pages.data_ptr(), num_pages, q.data_ptr(),
                                                _dtype_code(q), B, Hq, page_table.data_ptr(), maxp,
                                                seq_lens.data_ptr(), float(softmax_scale), float(k_scale),
                                                float(v_scale), pages_per_split, workspace.data_ptr(),
                                                workspace.numel(), out.data_ptr(), _stream(stream)),
           "tq_dense_fp8_decode_attention")
    return out


# --------------------------------------------------------------------------------------------------
# Dense random (QR) rotation in place of the WHT: the rotation matrices (host), the row rotation on the
# matrix cores, and quantize / decode attention with it.
# --------------------------------------------------------------------------------------------------

def qr_rotation(head_dim: int, gauss, sign_words=None):
    """(fwd, inv) fp32 [head_dim, head_dim] numpy arrays: fwd = diag(s) H Q / sqrt(d) for Q the orthogonal QR
    factor of ``gauss`` (fp64 [head_dim, head_dim]) and s the codebook's ``sign_words``; inv = fwd^T."""
    g = np.ascontiguousarray(gauss, dtype=np.float64)
    if g.shape != (head_dim, head_dim):
        raise ValueError("gauss must be [head_dim, head_dim]")
    sw = None if sign_words is None else np.ascontiguousarray(sign_words, dtype=np.uint32)
    fwd = np.empty((head_dim, head_dim), np.float32)
    inv = np.empty((head_dim, head_dim), np.float32)
    _check(_lib().tq_qr_rotation(head_dim, g.ctypes.data, None if sw is None else sw.ctypes.data, fwd.ctypes.data,
                                 inv.ctypes.data), "tq_qr_rotation")
    return fwd, inv


def rotate_rows(head_dim: int, mat, x, y=None, stream=None):
    """y[r] = mat x[r] for x [..., head_dim] (contiguous, fp32 / bf16 / f16); returns fp32 y shaped like x."""
    import torch

    _need(mat, "mat", torch.float32)
    _need(x, "x")
    if x.shape[-1] != head_dim or not x.is_contiguous() or not mat.is_contiguous() or mat.shape != (head_dim, head_dim):
        raise ValueError("x must be contiguous [..., head_dim] and mat [head_dim, head_dim]")
    if y is None:
        y = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _need(y, "y", torch.float32)
    if y.shape != x.shape or not y.is_contiguous():
        raise ValueError("y must be a contiguous fp32 tensor shaped like x")
    _check(_lib().tq_rotate_rows(head_dim, mat.data_ptr(), x.data_ptr(), _dtype_code(x), x.numel() // head_dim,
                                 y.data_ptr(), _stream(stream)), "tq_rotate_rows")
    return y


def quantize_kv_qr(layout: Layout, pages, k, v, slots, k_cb, v_cb, k_rot, v_rot, workspace=None, stream=None):
    """quantize_kv with the dense rotation: k, v contiguous [n_tok, num_kv_heads, head_dim]; k_rot, v_rot the
    device fp32 ``fwd`` matrices of qr_rotation built with the codebooks' sign words."""
    import torch

    _need(pages, "pages", torch.uint8)
    _need(slots, "slots", torch.int64)
    _need(k, "k")
    _need(v, "v")
    _need(k_rot, "k_rot", torch.float32)
    _need(v_rot, "v_rot", torch.float32)
    if k.dtype != v.dtype or k.shape != v.shape or k.dim() != 3 or k.shape[1:] != (layout.num_kv_heads, layout.head_dim):
        raise ValueError("k, v must be [n_tok, num_kv_heads, head_dim] of one dtype")
    if not (k.is_contiguous() and v.is_contiguous() and slots.is_contiguous()) or slots.numel() != k.shape[0]:
        raise ValueError("k, v, slots must be contiguous, one slot per token")
    out = ctypes.c_size_t()
    _check(_lib().tq_quantize_kv_qr_workspace_bytes(ctypes.byref(layout.c()), k.shape[0], ctypes.byref(out)),
           "tq_quantize_kv_qr_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(max(out.value, 16), dtype=torch.uint8, device=k.device)
    num_pages = pages.numel() // page_layout(layout)["page_bytes"]
    _check(_lib().tq_quantize_kv_qr(ctypes.byref(layout.c()), pages.data_ptr(), num_pages, k.data_ptr(), v.data_ptr(),
                                    _dtype_code(k), k.shape[0], slots.data_ptr(), k_cb.data_ptr(), v_cb.data_ptr(),
                                    k_rot.data_ptr(), v_rot.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                    _stream(stream)), "tq_quantize_kv_qr")


def decode_qr_workspace_bytes(layout: Layout, batch: int, num_q_heads: int, max_pages_per_seq: int,
                              pages_per_split: int = 0) -> int:
    out = ctypes.c_size_t()
    _check(_lib().tq_decode_qr_workspace_bytes(ctypes.byref(layout.c()), batch, num_q_heads, max_pages_per_seq,
                                               pages_per_split, ctypes.byref(out)), "tq_decode_qr_workspace_bytes")
    return out.value


def decode_attention_qr(layout: Layout, pages, q, page_table, seq_lens, softmax_scale, k_cb, v_cb, k_rot, v_inv,
                        workspace=None, out=None, pages_per_split: int = 0, stream=None):
    """decode_attention over a cache written by quantize_kv_qr: k_rot the keys' ``fwd`` matrix, v_inv the
    values' ``inv`` matrix (device fp32)."""
    import torch

    _need(pages, "pages", torch.uint8)
    _need(q, "q")
    _need(page_table, "page_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(k_rot, "k_rot", torch.float32)
    _need(v_inv, "v_inv", torch.float32)
    if q.dim() != 3 or q.shape[2] != layout.head_dim or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, num_q_heads, head_dim] tensor")
    B, Hq, _ = q.shape
    if page_table.dim() != 2 or page_table.shape[0] != B or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous [batch, max_pages_per_seq] int32 tensor")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must hold one int32 per sequence")
    maxp = page_table.shape[1]
    if workspace is None:
        need = decode_qr_workspace_bytes(layout, B, Hq, maxp, pages_per_split)
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(B, Hq, layout.head_dim, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor shaped like q")
    num_pages = pages.numel() // page_layout(layout)["page_bytes"]
    _check(_lib().tq_decode_attention_qr(ctypes.byref(layout.c()), pages.data_ptr(), num_pages, q.data_ptr(),
                                         _dtype_code(q), B, Hq, page_table.data_ptr(), maxp, seq_lens.data_ptr(),
                                         float(softmax_scale), pages_per_split, k_cb.data_ptr(), v_cb.data_ptr(),
                                         k_rot.data_ptr(), v_inv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                         out.data_ptr(), _stream(stream)), "tq_decode_attention_qr")
    return out


def _prefill_args(layout: Layout, pages, q, page_table, prefix_lens, out):
    import torch

    _need(pages, "pages", torch.uint8)
    _need(q, "q")
    _need(page_table, "page_table", torch.int32)
    _need(prefix_lens, "prefix_lens", torch.int32)
    if q.dim() != 4 or q.shape[3] != layout.head_dim or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, chunk_len, num_q_heads, head_dim] tensor")
    B, C, Hq, _ = q.shape
    if page_table.dim() != 2 or page_table.shape[0] != B or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous [batch, max_pages_per_seq] int32 tensor")
    if prefix_lens.numel() != B or not prefix_lens.is_contiguous():
        raise ValueError("prefix_lens must hold one int32 per sequence")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor shaped like q")
    num_pages = pages.numel() // page_layout(layout)["page_bytes"]
    return B, C, Hq, num_pages, out


def prefill_attention(layout: Layout, pages, q, page_table, prefix_lens, softmax_scale, k_cb, v_cb, out=None,
                      stream=None):
    """Causal attention of a chunk q [batch, chunk_len, num_q_heads, head_dim] at positions prefix_lens[b] + i
    over the packed cache (the chunk's own keys and values already in it); returns fp32 out shaped like q."""
    B, C, Hq, num_pages, out = _prefill_args(layout, pages, q, page_table, prefix_lens, out)
    _check(_lib().tq_prefill_attention(ctypes.byref(layout.c()), pages.data_ptr(), num_pages, q.data_ptr(),
                                       _dtype_code(q), B, C, Hq, page_table.data_ptr(), page_table.shape[1],
                                       prefix_lens.data_ptr(), float(softmax_scale), k_cb.data_ptr(), v_cb.data_ptr(),
                                       out.data_ptr(), _stream(stream)), "tq_prefill_attention")
    return out


def prefill_chunk(layout: Layout, pages, k, v, slots, q, page_table, prefix_lens, softmax_scale, k_cb, v_cb, out=None,
                  stream=None):
    """Quantize the chunk's k, v [batch, chunk_len, num_kv_heads, head_dim] into ``slots`` (int64, one per token),
    then prefill_attention of q over the cache; returns fp32 out shaped like q."""
    import torch

    B, C, Hq, num_pages, out = _prefill_args(layout, pages, q, page_table, prefix_lens, out)
    _need(slots, "slots", torch.int64)
    for name, t in (("k", k), ("v", v)):
        _need(t, name)
        if t.shape != (B, C, layout.num_kv_heads, layout.head_dim) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [batch, chunk_len, num_kv_heads, head_dim] tensor")
    if k.dtype != v.dtype:
        raise TypeError("k and v must share a dtype")
    if not slots.is_contiguous() or slots.numel() != B * C:
        raise ValueError("slots must be a contiguous int64 vector with one entry per chunk token")
    _check(_lib().tq_prefill_chunk(ctypes.byref(layout.c()), pages.data_ptr(), num_pages, k.data_ptr(), v.data_ptr(),
                                   _dtype_code(k), slots.data_ptr(), q.data_ptr(), _dtype_code(q), B, C, Hq,
                                   page_table.data_ptr(), page_table.shape[1], prefix_lens.data_ptr(),
                                   float(softmax_scale), k_cb.data_ptr(), v_cb.data_ptr(), out.data_ptr(),
                                   _stream(stream)), "tq_prefill_chunk")
    return out

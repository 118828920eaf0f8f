"""Plant plausible mistakes in the CPU oracle and check that a pin catches each one.

Every mutant is applied with monkeypatch for the duration of one test only; the
oracle's files are never modified. A mutant that no pin rejects would mean the
pins leave that part of the oracle unchecked.
"""
import math

import numpy as np
import pytest

from oracle import attention, codec, dense, lloyd_max, rotation
from tests import pins


def _caught(*checks):
    failures = 0
    for chk in checks:
        try:
            chk()
        except AssertionError:
            failures += 1
    return failures


def test_mutant_thresholds_not_midpoints(monkeypatch):
    orig = lloyd_max.thresholds_of
    monkeypatch.setattr(lloyd_max, "thresholds_of", lambda c: orig(c) + 0.05 * (np.asarray(c)[1:] - np.asarray(c)[:-1]))
    assert _caught(pins.check_max_1960_table, pins.check_centroid_condition_by_quadrature)


def test_mutant_levels_off_by_one_percent(monkeypatch):
    orig = lloyd_max.positive_levels
    monkeypatch.setattr(lloyd_max, "positive_levels", lambda b, **kw: 1.01 * orig(b, **kw))
    assert _caught(pins.check_max_1960_table, pins.check_one_bit_closed_form)


def test_mutant_rotation_normalised_by_d(monkeypatch):
    monkeypatch.setattr(rotation, "rotation_matrix",
                        lambda sw, d: rotation.hadamard(d) * rotation.sign_vector(sw, d)[None, :] / d)
    assert _caught(pins.check_rotation_orthogonal)


def test_mutant_signs_after_hadamard(monkeypatch):
    monkeypatch.setattr(rotation, "rotation_matrix",
                        lambda sw, d: rotation.sign_vector(sw, d)[:, None] * rotation.hadamard(d) / math.sqrt(d))
    assert _caught(pins.check_rotation_first_column, pins.check_fast_transform_agrees)


def test_mutant_sign_bits_msb_first(monkeypatch):
    def msb_first(sw, d):
        w = np.asarray(sw, dtype=np.uint32)
        i = np.arange(d)
        bit = (w[i // 32] >> (31 - i % 32).astype(np.uint32)) & np.uint32(1)
        return np.where(bit == 1, -1.0, 1.0)

    monkeypatch.setattr(rotation, "sign_vector", msb_first)
    assert _caught(pins.check_sign_bits)


def test_mutant_ties_go_down(monkeypatch):
    orig = codec.encode

    def ties_down(x, cb):
        e = orig(x, cb)
        e.codes = e.codes - np.isin(e.y * math.sqrt(cb.head_dim), cb.thresholds)
        return e

    monkeypatch.setattr(codec, "encode", ties_down)
    assert _caught(pins.check_zero_vector)


def test_mutant_big_endian_packing(monkeypatch):
    def big_endian(codes, b):
        c = np.asarray(codes, dtype=np.int64)
        N, d = c.shape
        bits = ((c[:, :, None] >> np.arange(b)[None, None, :]) & 1).astype(np.uint8).reshape(N, d * b)
        return np.packbits(bits, axis=1, bitorder="big")

    monkeypatch.setattr(codec, "pack_codes", big_endian)
    assert _caught(pins.check_packing_by_hand)


def test_mutant_wrong_qjl_constant(monkeypatch):
    orig = codec.dequantize_rotated

    def wrong_const(codes, norm16, cb, gamma16=None, qjl=None):
        g = None if gamma16 is None else np.asarray(gamma16) * (2.0 / math.pi)  # sqrt(2/pi) instead of sqrt(pi/2)
        return orig(codes, norm16, cb, g, qjl)

    monkeypatch.setattr(codec, "dequantize_rotated", wrong_const)
    assert _caught(pins.check_qjl_unbiased)


def test_mutant_dequantize_ignores_norm(monkeypatch):
    orig = codec.dequantize_rotated
    monkeypatch.setattr(codec, "dequantize_rotated",
                        lambda codes, norm16, cb, gamma16=None, qjl=None: orig(codes, np.ones_like(norm16), cb, gamma16, qjl))
    assert _caught(pins.check_inner_product_bias)


def test_mutant_gqa_head_mapping_modulo(monkeypatch):
    orig = attention.decode_attention

    def modulo_mapping(pool, L, cb_k, cb_v, q, page_table, seq_lens, scale, heads=None):
        q = np.asarray(q, dtype=np.float64)
        B, Hq, d = q.shape
        Hkv = L["H"]
        G = Hq // Hkv
        sigma = np.array([(h % Hkv) * G + h // Hkv for h in range(Hq)])
        q2 = np.empty_like(q)
        q2[:, sigma] = q
        return orig(pool, L, cb_k, cb_v, q2, page_table, seq_lens, scale)[:, sigma]

    monkeypatch.setattr(attention, "decode_attention", modulo_mapping)
    assert _caught(pins.check_attention_vs_torch_sdpa)


def test_mutant_scale_dropped(monkeypatch):
    orig = attention.decode_attention
    monkeypatch.setattr(attention, "decode_attention",
                        lambda pool, L, cb_k, cb_v, q, pt, sl, scale, heads=None: orig(pool, L, cb_k, cb_v, q, pt, sl, 1.0, heads))
    assert _caught(pins.check_attention_vs_torch_sdpa)


def test_mutant_v_layout_slot_major(monkeypatch):
    orig = codec._code_byte_index

    def slot_major(L, which, page, slot, head):
        if which == "v":
            L2 = dict(L)
            L2["k_codes"], L2["k_b"] = L["v_codes"], L["v_b"]
            return orig(L2, "k", page, slot, head)
        return orig(L, which, page, slot, head)

    monkeypatch.setattr(codec, "_code_byte_index", slot_major)
    assert _caught(pins.check_layout_positions)


@pytest.mark.parametrize("scale", [0.5, 2.0])
def test_mutant_norm_scaled(monkeypatch, scale):
    orig = codec.encode

    def scaled(x, cb):
        e = orig(x, cb)
        e.norm16 = codec.fp16_round(e.norm16 * scale)
        return e

    monkeypatch.setattr(codec, "encode", scaled)
    assert _caught(pins.check_vector_mse)


def test_mutant_codes_stored_as_plain_index(monkeypatch):
    monkeypatch.setattr(codec, "stored_code", lambda index, b: np.asarray(index, dtype=np.int64))
    assert _caught(pins.check_encode_known_cells, pins.check_code_map_by_hand)


def test_mutant_dense_bf16_truncates(monkeypatch):
    monkeypatch.setattr(dense, "bf16_bits",
                        lambda x: (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16))
    assert _caught(pins.check_dense_bf16_rounding)


def test_mutant_dense_v_token_major(monkeypatch):
    # V stored like K ([head][slot][d]) instead of coordinate-major within the page
    monkeypatch.setattr(dense, "_v_index",
                        lambda L, page, slot, head: (np.asarray(page, np.int64) * L["page_bytes"] + L["v"]) // 2
                        + (head * dense.PAGE_TOKENS + np.asarray(slot)) * L["d"])

    def write(pool, L, slots, head, k, v):
        slots = np.asarray(slots, dtype=np.int64)
        words = pool.view(np.uint16)
        page, slot = slots // dense.PAGE_TOKENS, slots % dense.PAGE_TOKENS
        d = L["d"]
        words[dense._k_index(L, page, slot, head)[:, None] + np.arange(d)[None, :]] = dense.bf16_bits(k)
        words[dense._v_index(L, page, slot, head)[:, None] + np.arange(d)[None, :]] = dense.bf16_bits(v)

    monkeypatch.setattr(dense, "write", write)
    assert _caught(pins.check_dense_layout_by_hand)


def test_mutant_dense_wrong_kv_head(monkeypatch):
    # query head h reading KV head h % H instead of h // G
    orig = dense.gather

    def gather(pool, L, page_row, seq_len, head):
        return orig(pool, L, page_row, seq_len, (head + 1) % L["H"])

    monkeypatch.setattr(dense, "gather", gather)
    assert _caught(pins.check_dense_attention_vs_torch_sdpa)


def test_mutant_fp8_truncates(monkeypatch):
    # round toward zero instead of to nearest: step down one code wherever the nearest value overshoots
    orig = dense.fp8_bits

    def trunc(x, scale=1.0):
        b = orig(x, scale).astype(np.int64)
        y = np.abs(np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float64)
        over = (np.abs(dense.fp8_value(b)) > y) & ((b & 0x7F) > 0)
        return (b - over).astype(np.uint8)

    monkeypatch.setattr(dense, "fp8_bits", trunc)
    assert _caught(pins.check_fp8_rounding_vs_torch) and _caught(pins.check_fp8_rounding_brute_force)


def test_mutant_fp8_overflow_to_nan(monkeypatch):
    orig = dense.fp8_bits

    def nosat(x, scale=1.0):
        b = orig(x, scale)
        big = np.abs(np.asarray(x, dtype=np.float32) / np.float32(scale)) > 464
        return np.where(big, b | 0x7F, b).astype(np.uint8)

    monkeypatch.setattr(dense, "fp8_bits", nosat)
    assert _caught(pins.check_fp8_rounding_brute_force)


def test_mutant_fp8_scale_multiplies_on_write(monkeypatch):
    orig = dense.fp8_bits
    monkeypatch.setattr(dense, "fp8_bits", lambda x, scale=1.0: orig(np.asarray(x, np.float32) * np.float32(scale)))
    assert _caught(pins.check_fp8_scale_and_layout_by_hand) and _caught(pins.check_dense_fp8_attention_vs_torch_sdpa)


def test_mutant_fp8_read_ignores_scale(monkeypatch):
    orig = dense._decode
    monkeypatch.setattr(dense, "_decode", lambda L, bits, scale: orig(L, bits, 1.0))
    assert _caught(pins.check_fp8_scale_and_layout_by_hand, pins.check_dense_fp8_attention_vs_torch_sdpa) == 2


def test_mutant_fp8_subnormal_step(monkeypatch):
    orig = dense.fp8_value

    def value(bits):
        v = orig(bits)
        b = np.asarray(bits, dtype=np.int64)
        return np.where(((b >> 3) & 15) == 0, v / 2, v)

    monkeypatch.setattr(dense, "fp8_value", value)
    assert _caught(pins.check_fp8_value_table)


def test_mutant_qr_no_sign_convention(monkeypatch):
    monkeypatch.setattr(rotation, "qr_rotation", lambda g: np.linalg.qr(np.asarray(g, dtype=np.float64))[0])
    assert _caught(pins.check_qr_rotation_factorization) and _caught(pins.check_qr_rotation_gram_schmidt)


def test_mutant_dense_rotation_transposed(monkeypatch):
    monkeypatch.setattr(codec.Codebook, "rotate", lambda self, u: np.asarray(u, dtype=np.float64) @ self.R
                        if self.dense is not None else rotation.rotate(u, self.sign_words))
    assert _caught(pins.check_dense_rotation_reduces_to_known_paths)


def test_mutant_dense_unrotate_transposed(monkeypatch):
    monkeypatch.setattr(codec.Codebook, "unrotate", lambda self, y: np.asarray(y, dtype=np.float64) @ self.R.T
                        if self.dense is not None else rotation.unrotate(y, self.sign_words))
    assert _caught(pins.check_dense_rotation_reduces_to_known_paths) and _caught(pins.check_dense_rotation_mse)


def _prefill_with_mask(rule):
    """The prefill oracle with its causal rule replaced: rule(t, P, i) -> allowed."""
    def prefill(pool, L, cb_k, cb_v, q, page_table, prefix_lens, scale, rows=None):
        q = np.asarray(q, dtype=np.float64)
        B, C, Hq, d = q.shape
        G = Hq // L["H"]
        out = np.full((B, C, Hq, d), np.nan)
        for b in range(B):
            P = int(prefix_lens[b])
            want = list(range(C)) if rows is None else sorted({i for bb, i in rows if bb == b})
            T = P + max(want) + 1
            allowed = np.array([[rule(t, P, i) for t in range(T)] for i in want])
            for g in range(L["H"]):
                rk = attention.gather(pool, L, "k", page_table[b], T, g)
                rv = attention.gather(pool, L, "v", page_table[b], T, g)
                K = codec.dequantize(rk["codes"], rk["norm16"], cb_k, rk.get("gamma16"), rk.get("qjl"))
                V = codec.dequantize(rv["codes"], rv["norm16"], cb_v)
                lg = scale * (q[b][want][:, g * G:(g + 1) * G] @ K.T)
                lg = np.where(allowed[:, None, :], lg, -np.inf)
                out[b, want, g * G:(g + 1) * G] = attention._softmax_weights(lg) @ V
        return out
    return prefill


@pytest.mark.parametrize("rule", [
    lambda t, P, i: t < P + i or t == 0,  # own token excluded
    lambda t, P, i: t <= i,               # prefix ignored
    lambda t, P, i: True,                 # no mask: the whole chunk visible
    lambda t, P, i: t <= P + i + 1,       # one token of look-ahead
], ids=["own-token-excluded", "prefix-ignored", "unmasked", "lookahead"])
def test_mutant_prefill_mask(monkeypatch, rule):
    monkeypatch.setattr(attention, "prefill_attention", _prefill_with_mask(rule))
    assert _caught(pins.check_prefill_vs_torch_sdpa, pins.check_prefill_special_cases)


def test_mutant_prefill_mask_control(monkeypatch):
    """The mutant scaffold with the true rule passes the pins (so the cases above fail for their rule)."""
    monkeypatch.setattr(attention, "prefill_attention", _prefill_with_mask(lambda t, P, i: t <= P + i))
    assert not _caught(pins.check_prefill_vs_torch_sdpa, pins.check_prefill_special_cases)

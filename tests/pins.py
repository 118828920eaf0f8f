"""Checks that pin the CPU oracle to facts fixed outside it.

Each ``check_*`` raises AssertionError when the oracle disagrees with a closed
form, a textbook table, a library routine, brute force or a statistical law. The
tests call them on the oracle as written, and ``test_oracle_mutations`` calls them
again with plausible mistakes planted in the oracle to show that each mistake is
caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.integrate import quad

import kvsynth
from oracle import attention, codec, dense, lloyd_max, rotation

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
PANTER_DITE = math.sqrt(3.0) * math.pi / 2.0  # high-resolution Gaussian constant, ~2.7207


def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


# --------------------------------------------------------------------------------------------
# Lloyd-Max codebook
# --------------------------------------------------------------------------------------------


def check_one_bit_closed_form():
    """1 bit: levels +-sqrt(2/pi) (half-normal mean), distortion 1 - 2/pi."""
    c = lloyd_max.levels(1)
    assert np.allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], rtol=0, atol=1e-14), c
    D = lloyd_max.distortion(c, lloyd_max.thresholds_of(c))
    assert abs(D - (1 - 2 / math.pi)) < 1e-14, D


def check_max_1960_table():
    """Levels, thresholds and distortion agree with Max (1960) Table I within its printed precision."""
    with open(os.path.join(GOLDEN, "max1960_gaussian.json")) as f:
        tab = json.load(f)["levels"]
    for n_levels, row in tab.items():
        b = int(round(math.log2(int(n_levels))))
        c = lloyd_max.levels(b)
        t = lloyd_max.thresholds_of(c)
        half = len(c) // 2
        for got, want in zip(c[half:], row["outputs"]):
            unit = 10.0 ** (math.floor(math.log10(abs(want))) - 3)
            assert abs(got - want) <= 1.5 * unit, (n_levels, got, want)
        for got, want in zip(t[half - 1:], row["thresholds"]):
            unit = 1e-4 if want == 0 else 10.0 ** (math.floor(math.log10(abs(want))) - 3)
            assert abs(got - want) <= 1.5 * unit, (n_levels, got, want)
        D = lloyd_max.distortion(c, t)
        assert abs(D - row["distortion"]) <= 1e-3 * row["distortion"], (n_levels, D)


def check_centroid_condition_by_quadrature(bits_list=(1, 2, 3, 4, 8)):
    """Each level equals the Gaussian conditional mean of its cell, by adaptive quadrature."""
    for b in bits_list:
        c = lloyd_max.levels(b)
        t = lloyd_max.thresholds_of(c)
        edges = np.concatenate([[-np.inf], t, [np.inf]])
        for j in range(len(c)):
            lo, hi = edges[j], edges[j + 1]
            if lo < 0 < hi:
                continue  # only for the 1-bit case straddling zero, which is symmetric
            m0 = quad(_phi, lo, hi, epsabs=0, epsrel=1e-13, limit=200)[0]
            m1 = quad(lambda x: x * _phi(x), lo, hi, epsabs=0, epsrel=1e-13, limit=200)[0]
            assert abs(m1 / m0 - c[j]) <= 1e-9 * max(1.0, abs(c[j])), (b, j, m1 / m0, c[j])


def check_distortion_by_quadrature(bits_list=(1, 2, 3, 4)):
    for b in bits_list:
        c = lloyd_max.levels(b)
        t = lloyd_max.thresholds_of(c)
        edges = np.concatenate([[-np.inf], t, [np.inf]])
        D = sum(quad(lambda x, cj=cj: (x - cj) ** 2 * _phi(x), edges[j], edges[j + 1], epsabs=1e-15, epsrel=1e-12)[0]
                for j, cj in enumerate(c))
        assert abs(D - lloyd_max.distortion(c, t)) < 1e-11, (b, D)


def check_local_optimality(bits_list=(2, 3, 4)):
    """Moving any positive level by +-1e-3 (with its thresholds re-centred) raises the distortion."""
    for b in bits_list:
        c = lloyd_max.levels(b)
        D0 = lloyd_max.distortion(c, lloyd_max.thresholds_of(c))
        for j in range(len(c) // 2, len(c)):
            for eps in (-1e-3, 1e-3):
                c2 = c.copy()
                c2[j] += eps
                c2[len(c) - 1 - j] -= eps
                assert lloyd_max.distortion(c2, lloyd_max.thresholds_of(c2)) > D0, (b, j, eps)


def check_distortion_values_and_bound():
    """Distortions ~0.363, 0.118, 0.0345, 0.0095 (b = 1..4); D_b * 4^b under the 2.72 factor."""
    want = {1: 0.3634, 2: 0.1175, 3: 0.03455, 4: 0.009501}
    for b, w in want.items():
        c = lloyd_max.levels(b)
        D = lloyd_max.distortion(c, lloyd_max.thresholds_of(c))
        assert abs(D - w) < 2e-4 * w + 5e-6, (b, D)
    for b in (1, 2, 3, 4, 8):
        c = lloyd_max.levels(b)
        D = lloyd_max.distortion(c, lloyd_max.thresholds_of(c))
        assert D * 4 ** b <= PANTER_DITE, (b, D * 4 ** b)
    c = lloyd_max.levels(8)
    D8 = lloyd_max.distortion(c, lloyd_max.thresholds_of(c))
    assert abs(D8 * 4 ** 8 / PANTER_DITE - 1.0) < 0.02, D8 * 4 ** 8


def check_scalar_mse_monte_carlo(n=400_000, seed=5):
    """Quantizing N(0,1) samples with the stored (fp16) codebook reaches D_b within Monte Carlo error."""
    rng = np.random.Generator(np.random.Philox(seed))
    x = rng.standard_normal(n)
    for b in (1, 2, 3, 4):
        cb = codec.make_codebook(64, b, codec.MSE, np.zeros(2, np.uint32))
        idx = np.searchsorted(cb.thresholds, x, side="right")
        err = (x - cb.levels16[idx]) ** 2
        c = lloyd_max.levels(b)
        D = lloyd_max.distortion(c, lloyd_max.thresholds_of(c))
        assert abs(err.mean() - D) < 5 * err.std() / math.sqrt(n), (b, err.mean(), D)


# --------------------------------------------------------------------------------------------
# Rotation
# --------------------------------------------------------------------------------------------


def check_hadamard_closed_form(dims=(1, 2, 4, 8, 64, 128)):
    """Sylvester's matrix is H[i, j] = (-1)^popcount(i & j) and H_2n = kron(H_2, H_n)."""
    for d in dims:
        H = rotation.hadamard(d)
        i = np.arange(d)
        pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
        assert np.array_equal(H, np.where(pc % 2 == 0, 1.0, -1.0)), d
        if d >= 2:
            assert np.array_equal(H, np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), rotation.hadamard(d // 2))), d


def check_rotation_orthogonal(d=128, seed=3):
    sw = kvsynth.rotation_signs(seed, d)
    R = rotation.rotation_matrix(sw, d)
    assert np.allclose(R @ R.T, np.eye(d), atol=1e-13)
    rng = np.random.Generator(np.random.Philox(seed))
    x, z = rng.standard_normal((2, 7, d))
    assert np.allclose(np.linalg.norm(rotation.rotate(x, sw), axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(np.sum(rotation.rotate(x, sw) * rotation.rotate(z, sw), axis=1), np.sum(x * z, axis=1), atol=1e-12)
    assert np.allclose(rotation.unrotate(rotation.rotate(x, sw), sw), x, atol=1e-13)


def check_rotation_first_column(d=128, seed=9):
    """R e_0 = s_0 / sqrt(d) * (1, ..., 1): signs act before the Hadamard matrix."""
    sw = kvsynth.rotation_signs(seed, d)
    s = rotation.sign_vector(sw, d)
    for j in (0, 1, 5):
        e = np.zeros((1, d))
        e[0, j] = 1.0
        col = rotation.rotate(e, sw)[0]
        assert np.allclose(np.abs(col), 1 / math.sqrt(d), atol=1e-15)
        if j == 0:
            assert np.allclose(col, s[0] / math.sqrt(d), atol=1e-15)


def check_sign_bits():
    """Bit i of word i//32, LSB first, set -> coordinate i negated."""
    w = np.array([0b1011, 0x80000000], dtype=np.uint32)
    s = rotation.sign_vector(w, 64)
    want = np.ones(64)
    want[[0, 1, 3, 63]] = -1
    assert np.array_equal(s, want)


def check_fast_transform_agrees(d=128, seed=4):
    """An in-place butterfly (fast WHT) applied to s * u, over sqrt(d), equals the matrix route."""
    sw = kvsynth.rotation_signs(seed, d)
    s = rotation.sign_vector(sw, d)
    rng = np.random.Generator(np.random.Philox(seed))
    u = rng.standard_normal((5, d))
    v = (u * s).copy()
    h = 1
    while h < d:
        for start in range(0, d, 2 * h):
            a = v[:, start:start + h].copy()
            b = v[:, start + h:start + 2 * h].copy()
            v[:, start:start + h] = a + b
            v[:, start + h:start + 2 * h] = a - b
        h *= 2
    assert np.allclose(v / math.sqrt(d), rotation.rotate(u, sw), atol=1e-12)


def check_gaussianization(d=128, n=20000, seed=11):
    """Channels with log-normal scales make raw coordinates heavy-tailed; rotated coordinates of the
    unit vectors are close to Gaussian (kurtosis near 3), which signs alone do not achieve."""
    rng = np.random.Generator(np.random.Philox(seed))
    x = rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))
    k_raw = np.mean(x ** 4) / np.mean(x ** 2) ** 2
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    sw = kvsynth.rotation_signs(seed, d)
    y = rotation.rotate(u, sw).ravel()
    k_rot = np.mean(y ** 4) / np.mean(y ** 2) ** 2
    z = (u * rotation.sign_vector(sw, d)).ravel()
    k_signs = np.mean(z ** 4) / np.mean(z ** 2) ** 2
    assert k_raw > 20, k_raw
    assert 2.5 < k_rot < 3.1, k_rot
    assert k_signs > 10, k_signs


# --------------------------------------------------------------------------------------------
# Codec
# --------------------------------------------------------------------------------------------


def check_packing_by_hand():
    """Hand-packed bytes of a known code sequence (little-endian bit stream)."""
    codes = np.zeros((1, 64), np.int64)
    codes[0, :4] = [1, 2, 3, 0]
    assert codec.pack_codes(codes, 2)[0, 0] == 0b00_11_10_01  # 0x39
    codes = np.zeros((1, 64), np.int64)
    codes[0, :3] = [5, 6, 7]  # 101 110 111 -> bits 0..8 = 1,0,1, 0,1,1, 1,1,1
    p = codec.pack_codes(codes, 3)[0]
    assert p[0] == 0b11_110_101 and p[1] == 0b1, p[:2]
    codes = np.zeros((1, 64), np.int64)
    codes[0, :2] = [0xA, 0x3]
    assert codec.pack_codes(codes, 4)[0, 0] == 0x3A
    z = np.zeros((1, 16), bool)
    z[0, [0, 9, 15]] = True
    assert list(codec.pack_bits(z)[0]) == [0x01, 0x82]


def check_pack_roundtrip(seed=2):
    rng = np.random.Generator(np.random.Philox(seed))
    for b in codec.SUPPORTED_BITS:
        for d in (64, 128):
            c = rng.integers(0, 1 << b, size=(9, d))
            p = codec.pack_codes(c, b)
            assert p.shape == (9, d * b // 8)
            assert np.array_equal(codec.unpack_codes(p, b, d), c)


def check_compression_ratios():
    """One fp16 norm per 128 coordinates: 3 bits -> 5.12x, 4 bits -> ~3.9x, vs fp16."""
    for bits, want in ((3, 5.12), (4, 256 / 66)):
        L = codec.page_layout(1, 128, bits, codec.MSE, bits, codec.MSE)
        per_vec = (L["k_norms"] - L["k_codes"] + 32) / 16  # codes + norm bytes per vector
        assert abs(256.0 / per_vec - want) < 1e-12, (bits, 256.0 / per_vec)
    L = codec.page_layout(8, 128, 4, codec.MSE, 2, codec.MSE)
    assert (L["k_codes"], L["k_norms"], L["v_codes"], L["v_norms"], L["page_bytes"]) == (0, 8192, 8448, 12544, 12800)
    L = codec.page_layout(8, 128, 2, codec.PROD, 2, codec.MSE)
    assert (L["k_codes"], L["k_norms"], L["k_qjl"], L["k_gamma"], L["v_codes"], L["page_bytes"]) == \
        (0, 2048, 2304, 4352, 4608, 4608 + 4096 + 256)


def check_layout_positions():
    """Bytes of one record land where the layout says (hand-computed offsets)."""
    d, H = 64, 2
    L = codec.page_layout(H, d, 4, codec.MSE, 2, codec.MSE)
    # K codes: 2*16*32 = 1024; norms 64; V codes at 1088: 2*8*16*2 = 512; V norms at 1600; page 1664
    assert (L["k_norms"], L["v_codes"], L["v_norms"], L["page_bytes"]) == (1024, 1088, 1600, 1664)
    pool = np.zeros(3 * L["page_bytes"], np.uint8)
    enc = codec.Encoded(codes=np.arange(d)[None, :] % 4, norm16=np.array([1.5]), norm=np.array([1.5]), y=None)
    slot = 2 * 16 + 5  # page 2, slot 5
    codec.write_records(pool, L, "v", [slot], 1, enc)
    base = 2 * L["page_bytes"]
    stream = codec.pack_codes(enc.codes, 2)[0]  # 16 bytes
    for j in range(d // 8):  # piece j = stream bytes 2j, 2j+1 at [head 1][j][slot 5]
        off = base + 1088 + ((1 * 8 + j) * 16 + 5) * 2
        assert list(pool[off:off + 2]) == list(stream[2 * j:2 * j + 2]), j
    noff = base + 1600 + (1 * 16 + 5) * 2
    assert pool[noff:noff + 2].view(np.float16)[0] == 1.5
    codec.write_records(pool, L, "k", [slot], 0, enc)
    koff = base + (0 * 16 + 5) * 32
    assert list(pool[koff:koff + 32]) == list(codec.pack_codes(enc.codes, 4)[0])


def check_code_map_by_hand():
    """Sign-magnitude codes: the top bit marks the non-negative half, the rest count the rank from zero."""
    assert list(codec.stored_code(np.arange(4), 2)) == [1, 0, 2, 3]
    assert list(codec.stored_code(np.arange(16), 4)) == [7, 6, 5, 4, 3, 2, 1, 0, 8, 9, 10, 11, 12, 13, 14, 15]
    assert list(codec.stored_code([0, 1], 1)) == [0, 1]
    for b in (1, 2, 3, 4, 8):
        i = np.arange(1 << b)
        assert np.array_equal(codec.level_index(codec.stored_code(i, b), b), i)


def check_encode_known_cells(d=64, seed=6):
    """A vector built so that its rotated coordinates sit exactly on chosen levels encodes to the codes
    read off by hand: level k of the ascending table -> sign-magnitude code of k."""
    sw = kvsynth.rotation_signs(seed, d)
    for b in (2, 3, 4):
        cb = codec.make_codebook(d, b, codec.MSE, sw)
        L = 1 << b
        yp = np.empty(d)
        yp[:L] = cb.levels16  # coordinates 0..L-1 sit on the levels (cell centres)
        rest = d - L
        fill = math.sqrt((d - np.sum(yp[:L] ** 2)) / rest)  # so that ||y'|| = sqrt(d), i.e. y = y'/sqrt(d) is a unit vector
        yp[L:] = fill * np.where(np.arange(rest) % 2 == 0, 1.0, -1.0)
        x = 3.0 * rotation.unrotate((yp / math.sqrt(d))[None, :], sw)
        e = codec.encode(x, cb)
        half = L // 2
        want = [half - 1 - k if k < half else k for k in range(L)]
        assert list(e.codes[0, :L]) == want, (b, list(e.codes[0, :L]), want)


def check_zero_vector():
    """A zero vector stores norm 0 and the first non-negative level (y = 0 lies on the middle threshold)."""
    for b in (1, 2, 3, 4, 8):
        cb = codec.make_codebook(64, b, codec.MSE, kvsynth.rotation_signs(0, 64))
        e = codec.encode(np.zeros((1, 64)), cb)
        assert e.norm16[0] == 0.0
        assert np.all(e.codes == (1 << b) // 2), (b, e.codes[0, :4])


def check_vector_mse(d=128, n=3000, seed=21):
    """Full pipeline on iid Gaussian vectors: E||u - uhat||^2 matches D_b (sphere vs Gaussian: 3%)."""
    rng = np.random.Generator(np.random.Philox(seed))
    x = rng.standard_normal((n, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    for b in (1, 2, 3, 4):
        cb = codec.make_codebook(d, b, codec.MSE, kvsynth.rotation_signs(seed, d))
        e = codec.encode(x, cb)
        uh = codec.dequantize(e.codes, np.ones(n), cb)
        mse = np.mean(np.sum((u - uh) ** 2, axis=1))
        c = lloyd_max.levels(b)
        D = lloyd_max.distortion(c, lloyd_max.thresholds_of(c))
        assert abs(mse / D - 1) < 0.03, (b, mse, D)
        # with the stored fp16 norms the relative reconstruction error of x itself is the same
        xh = codec.dequantize(e.codes, e.norm16, cb)
        rel = np.mean(np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1))
        assert abs(rel / D - 1) < 0.03, (b, rel, D)
        assert np.array_equal(e.norm16, np.linalg.norm(x, axis=1).astype(np.float16).astype(np.float64))


def check_inner_product_bias(d=128, seeds=300, seed=31):
    """Averaged over rotations, <q, xhat> ~ (1 - D_b) <q, x>: the MSE quantizer shrinks inner products
    (about 3% at 3 bits)."""
    rng = np.random.Generator(np.random.Philox(seed))
    x = rng.standard_normal((1, d))
    q = x[0] + 0.5 * rng.standard_normal(d)
    n = np.linalg.norm(x)
    for b, tol in ((1, 0.03), (3, 0.004)):
        ratios = []
        for s in range(seeds):
            cb = codec.make_codebook(d, b, codec.MSE, kvsynth.rotation_signs(1000 + s, d))
            e = codec.encode(x, cb)
            xh = codec.dequantize(e.codes, np.array([n]), cb)[0]
            ratios.append(q @ xh / (q @ x[0]))
        c = lloyd_max.levels(b)
        D = lloyd_max.distortion(c, lloyd_max.thresholds_of(c))
        assert abs(np.mean(ratios) - (1 - D)) < tol, (b, np.mean(ratios), 1 - D)


def check_qjl_unbiased(d=128, trials=1500, seed=41):
    """prod mode: averaged over projection matrices S, <q, khat> = <q, x> (no shrinkage)."""
    rng = np.random.Generator(np.random.Philox(seed))
    x = rng.standard_normal((1, d))
    q = x[0] + 0.7 * rng.standard_normal(d)
    sw = kvsynth.rotation_signs(seed, d)
    n = np.linalg.norm(x)
    est = []
    for t in range(trials):
        S = rng.standard_normal((d, d)).astype(np.float32)
        cb = codec.make_codebook(d, 2, codec.PROD, sw, S)
        e = codec.encode(x, cb)
        kh = codec.dequantize(e.codes, np.array([n]), cb, np.array([e.gamma[0]]), e.qjl)[0]
        est.append(q @ kh)
    est = np.array(est)
    true = q @ x[0]
    assert abs(est.mean() - true) < 4 * est.std() / math.sqrt(trials), (est.mean(), true, est.std())
    # the MSE-only estimate with the same 1-bit codebook is biased by the factor (1 - D_1)
    cb1 = codec.make_codebook(d, 1, codec.MSE, sw)
    e1 = codec.encode(x, cb1)
    mse_only = q @ codec.dequantize(e1.codes, np.array([n]), cb1)[0]
    assert abs(mse_only - true) > 4 * est.std() / math.sqrt(trials)
    # variance bound of the sign estimator: Var <= pi/2 * gamma^2 ||q||^2 n^2 / m
    cbp = codec.make_codebook(d, 2, codec.PROD, sw, rng.standard_normal((d, d)))
    g = codec.encode(x, cbp).gamma[0]
    assert est.var() <= math.pi / 2 * (g * n) ** 2 * (q @ q) / d * 1.2


def check_determinism(d=128):
    """Same seeds and input -> identical stored bytes."""
    sw = kvsynth.rotation_signs(77, d)
    S = kvsynth.qjl_projection(77, d)
    x = np.random.Generator(np.random.Philox(1)).standard_normal((40, d))
    L = codec.page_layout(1, d, 2, codec.PROD, 3, codec.MSE)
    pools = []
    for _ in range(2):
        pool = np.zeros(4 * L["page_bytes"], np.uint8)
        for which, cb in (("k", codec.make_codebook(d, 2, codec.PROD, sw, S)), ("v", codec.make_codebook(d, 3, codec.MSE, sw))):
            codec.write_records(pool, L, which, np.arange(40) + 3, 0, codec.encode(x, cb))
        pools.append(pool)
    assert np.array_equal(pools[0], pools[1])


# --------------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------------


def build_cache(H, d, Hq, B, lens, kb, km, vb, vm, seed=0, shuffled=True, q_scale=1.0, dense=False):
    """Encode random K/V for B sequences into a page pool; returns everything the checks need. ``dense``:
    QR rotations (their own draws for K and V) in place of the WHT."""
    rng = np.random.Generator(np.random.Philox(seed))
    sw_k = kvsynth.rotation_signs(seed + 1, d)
    sw_v = kvsynth.rotation_signs(seed + 2, d)
    S = kvsynth.qjl_projection(seed + 3, d)
    dk = rotation.qr_rotation(kvsynth.qr_gaussian(seed + 5, d)) if dense else None
    dv = rotation.qr_rotation(kvsynth.qr_gaussian(seed + 6, d)) if dense else None
    cbk = codec.make_codebook(d, kb, km, sw_k, S if km == codec.PROD else None, dense=dk)
    cbv = codec.make_codebook(d, vb, vm, sw_v, S if vm == codec.PROD else None, dense=dv)
    L = codec.page_layout(H, d, kb, km, vb, vm)
    pps = max(1, max((l + 15) // 16 for l in lens))
    pt, npages = kvsynth.page_table(B, pps, shuffled, seed=seed + 4)
    pool = np.zeros(npages * L["page_bytes"], np.uint8)
    K = rng.standard_normal((B, pps * 16, H, d)) * np.exp(rng.standard_normal((H, d)))
    V = rng.standard_normal((B, pps * 16, H, d))
    for b in range(B):
        sl = kvsynth.slots_for(pt, b, 0, lens[b])
        for h in range(H):
            codec.write_records(pool, L, "k", sl, h, codec.encode(K[b, :lens[b], h], cbk))
            codec.write_records(pool, L, "v", sl, h, codec.encode(V[b, :lens[b], h], cbv))
    q = rng.standard_normal((B, Hq, d)) * q_scale
    return dict(pool=pool, L=L, cbk=cbk, cbv=cbv, pt=pt, lens=np.array(lens), q=q, K=K, V=V)


def check_attention_two_routes():
    for (kb, km, vb, vm) in ((4, 0, 2, 0), (2, 1, 2, 0), (3, 0, 2, 1), (8, 0, 8, 0)):
        c = build_cache(2, 64, 8, 2, [37, 70], kb, km, vb, vm, seed=kb + 10 * km)
        o1 = attention.decode_attention(c["pool"], c["L"], c["cbk"], c["cbv"], c["q"], c["pt"], c["lens"], 0.125)
        o2 = attention.decode_attention_rotated(c["pool"], c["L"], c["cbk"], c["cbv"], c["q"], c["pt"], c["lens"], 0.125)
        assert attention.relative_error(o1, o2) < 1e-10


def check_attention_vs_torch_sdpa():
    """Against torch's scaled_dot_product_attention (fp64, CPU) on the dequantized cache, GQA expanded
    with repeat_interleave."""
    import torch

    H, d, Hq, B = 2, 64, 8, 2
    lens = [45, 45]
    c = build_cache(H, d, Hq, B, lens, 4, 0, 2, 0, seed=5)
    out = attention.decode_attention(c["pool"], c["L"], c["cbk"], c["cbv"], c["q"], c["pt"], c["lens"], 0.2)
    for b in range(B):
        Ks, Vs = [], []
        for h in range(H):
            rk = attention.gather(c["pool"], c["L"], "k", c["pt"][b], lens[b], h)
            rv = attention.gather(c["pool"], c["L"], "v", c["pt"][b], lens[b], h)
            Ks.append(codec.dequantize(rk["codes"], rk["norm16"], c["cbk"]))
            Vs.append(codec.dequantize(rv["codes"], rv["norm16"], c["cbv"]))
        Kt = torch.tensor(np.stack(Ks)).repeat_interleave(Hq // H, dim=0)
        Vt = torch.tensor(np.stack(Vs)).repeat_interleave(Hq // H, dim=0)
        qt = torch.tensor(c["q"][b])[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=0.2)[:, 0, :].numpy()
        assert np.allclose(out[b], ref, rtol=1e-10, atol=1e-12), b


def check_attention_special_cases():
    # one cached token: the output is that token's dequantized value
    c = build_cache(1, 64, 4, 1, [1], 4, 0, 2, 0, seed=8)
    out = attention.decode_attention(c["pool"], c["L"], c["cbk"], c["cbv"], c["q"], c["pt"], c["lens"], 0.125)
    rv = attention.gather(c["pool"], c["L"], "v", c["pt"][0], 1, 0)
    v0 = codec.dequantize(rv["codes"], rv["norm16"], c["cbv"])[0]
    assert np.allclose(out[0], v0[None, :], atol=1e-13)
    # all keys equal: uniform weights, output = mean of dequantized values
    d = 64
    L = codec.page_layout(1, d, 4, 0, 2, 0)
    pool = np.zeros(4 * L["page_bytes"], np.uint8)
    cbk = codec.make_codebook(d, 4, 0, kvsynth.rotation_signs(1, d))
    cbv = codec.make_codebook(d, 2, 0, kvsynth.rotation_signs(2, d))
    rng = np.random.Generator(np.random.Philox(3))
    k = np.repeat(rng.standard_normal((1, d)), 50, axis=0)
    v = rng.standard_normal((50, d))
    pt = np.array([[3, 0, 2, 1]], np.int32)
    sl = kvsynth.slots_for(pt, 0, 0, 50)
    codec.write_records(pool, L, "k", sl, 0, codec.encode(k, cbk))
    codec.write_records(pool, L, "v", sl, 0, codec.encode(v, cbv))
    q = rng.standard_normal((1, 4, d))
    out = attention.decode_attention(pool, L, cbk, cbv, q, pt, [50], 0.3)
    ev = codec.encode(v, cbv)
    assert np.allclose(out[0], codec.dequantize(ev.codes, ev.norm16, cbv).mean(axis=0)[None, :], atol=1e-13)
    # zero-length sequence -> zeros
    out = attention.decode_attention(pool, L, cbk, cbv, q, pt, [0], 0.3)
    assert np.all(out == 0)


def _prefill_cache(H, d, Hq, B, prefix, C, kb, km, vb, vm, seed):
    """A cache holding prefix + chunk tokens per sequence, and chunk queries [B, C, Hq, d]."""
    c = build_cache(H, d, Hq, B, [p + C for p in prefix], kb, km, vb, vm, seed=seed)
    rng = np.random.Generator(np.random.Philox(seed + 100))
    c["qc"] = rng.standard_normal((B, C, Hq, d))
    c["prefix"] = np.asarray(prefix)
    return c


def check_prefill_vs_torch_sdpa():
    """Chunk attention against torch's scaled_dot_product_attention (fp64, CPU) on the dequantized cache with
    an explicit boolean mask (query i sees keys 0 .. P + i), GQA expanded with repeat_interleave."""
    import torch

    H, d, Hq, B, C = 2, 64, 8, 2, 21
    prefix = [0, 35]
    for (kb, km, vb, vm) in ((4, 0, 2, 0), (2, 1, 3, 0)):
        c = _prefill_cache(H, d, Hq, B, prefix, C, kb, km, vb, vm, seed=70 + kb)
        out = attention.prefill_attention(c["pool"], c["L"], c["cbk"], c["cbv"], c["qc"], c["pt"], c["prefix"], 0.15)
        for b in range(B):
            T = prefix[b] + C
            Ks, Vs = [], []
            for h in range(H):
                rk = attention.gather(c["pool"], c["L"], "k", c["pt"][b], T, h)
                rv = attention.gather(c["pool"], c["L"], "v", c["pt"][b], T, h)
                Ks.append(codec.dequantize(rk["codes"], rk["norm16"], c["cbk"], rk.get("gamma16"), rk.get("qjl")))
                Vs.append(codec.dequantize(rv["codes"], rv["norm16"], c["cbv"]))
            Kt = torch.tensor(np.stack(Ks)).repeat_interleave(Hq // H, dim=0)  # [Hq, T, d]
            Vt = torch.tensor(np.stack(Vs)).repeat_interleave(Hq // H, dim=0)
            qt = torch.tensor(c["qc"][b]).transpose(0, 1)                     # [Hq, C, d]
            mask = torch.ones(C, T, dtype=torch.bool).tril(diagonal=prefix[b])
            ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=0.15)
            assert np.allclose(out[b], ref.transpose(0, 1).numpy(), rtol=1e-10, atol=1e-12), (kb, b)


def check_prefill_special_cases():
    """Zero queries weigh every visible token equally: row i is the mean of the dequantized values of tokens
    0 .. P + i; with no prefix the first row is token 0's value whatever its query; a restricted row set gives
    the same rows."""
    H, d, Hq, C = 1, 64, 2, 19
    for P in (0, 16, 29):
        c = _prefill_cache(H, d, Hq, 1, [P], C, 3, 0, 2, 0, seed=80 + P)
        rv = attention.gather(c["pool"], c["L"], "v", c["pt"][0], P + C, 0)
        V = codec.dequantize(rv["codes"], rv["norm16"], c["cbv"])
        zero = attention.prefill_attention(c["pool"], c["L"], c["cbk"], c["cbv"], np.zeros_like(c["qc"]), c["pt"],
                                           [P], 0.3)
        for i in range(C):
            assert np.allclose(zero[0, i], V[: P + i + 1].mean(axis=0)[None, :], atol=1e-13), (P, i)
        full = attention.prefill_attention(c["pool"], c["L"], c["cbk"], c["cbv"], c["qc"], c["pt"], [P], 0.3)
        if P == 0:
            assert np.allclose(full[0, 0], V[0][None, :], atol=1e-13)
        some = attention.prefill_attention(c["pool"], c["L"], c["cbk"], c["cbv"], c["qc"], c["pt"], [P], 0.3,
                                           rows=[(0, 3), (0, C - 1)])
        assert np.array_equal(some[0, [3, C - 1]], full[0, [3, C - 1]])
        assert np.isnan(some[0, 0]).all()


def check_prefill_rows_are_decode_steps():
    """Row i of a chunk is the decode attention of its query at sequence length P + i + 1 (a second route: the
    decode oracle's own gather and softmax at each length)."""
    H, d, Hq, B, C = 2, 64, 4, 2, 18
    prefix = [5, 40]
    c = _prefill_cache(H, d, Hq, B, prefix, C, 4, 0, 3, 0, seed=90)
    out = attention.prefill_attention(c["pool"], c["L"], c["cbk"], c["cbv"], c["qc"], c["pt"], c["prefix"], 0.2)
    for i in range(C):
        ref = attention.decode_attention(c["pool"], c["L"], c["cbk"], c["cbv"], c["qc"][:, i], c["pt"],
                                         c["prefix"] + i + 1, 0.2)
        assert attention.relative_error(out[:, i], ref) < 1e-12, i


def check_page_table_invariance():
    """The same tokens stored through a shuffled or an identity page table give identical outputs."""
    outs = []
    for shuffled in (False, True):
        c = build_cache(2, 64, 4, 2, [33, 64], 3, 0, 3, 0, seed=12, shuffled=shuffled)
        outs.append(attention.decode_attention(c["pool"], c["L"], c["cbk"], c["cbv"], c["q"], c["pt"], c["lens"], 0.125))
    assert np.array_equal(outs[0], outs[1])


def check_attention_error_shrinks_with_bits():
    """Attention over the quantized cache approaches exact attention as bits grow."""
    errs = []
    for bits in (2, 4, 8):
        c = build_cache(1, 128, 4, 1, [256], bits, 0, bits, 0, seed=14, q_scale=0.3)
        out = attention.decode_attention(c["pool"], c["L"], c["cbk"], c["cbv"], c["q"], c["pt"], c["lens"], 1 / math.sqrt(128))
        ref = attention.reference_attention(c["q"][0], c["K"][0, :256, 0], c["V"][0, :256, 0], 1 / math.sqrt(128))
        errs.append(np.max(np.abs(out[0] - ref)))
    assert errs[0] > errs[1] > errs[2], errs
    # the error scales like the square root of the per-coordinate distortion, within a factor 2
    for bits, e in zip((4, 8), errs[1:]):
        D = {b: lloyd_max.distortion(lloyd_max.levels(b), lloyd_max.thresholds_of(lloyd_max.levels(b))) for b in (2, bits)}
        ratio = (e / errs[0]) / math.sqrt(D[bits] / D[2])
        assert 0.5 < ratio < 2.0, (bits, ratio)


# --------------------------------------------------------------------------------------------
# Uncompressed comparator (bf16 pages)
# --------------------------------------------------------------------------------------------


def check_dense_bf16_rounding(seed=51):
    """Round-to-nearest-even to bf16 against torch's conversion, ties and carries included."""
    import torch

    rng = np.random.Generator(np.random.Philox(seed))
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    u = x.view(np.uint32)
    ties = np.concatenate([(u[:500] & 0xFFFF0000) | 0x8000, (u[500:1000] | 0x10000) & 0xFFFF0000 | 0x8000,
                           np.array([0x3F7FFFFF, 0x3F7F8000, 0x3F808000, 0x00000000, 0x80000000], np.uint32)])
    x = np.concatenate([x, ties.view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(dense.bf16_bits(x), want)
    assert np.array_equal(dense.bf16_value(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).double().numpy())


def check_dense_layout_by_hand():
    """Byte positions of one token written by hand: K row contiguous, V column strided by 16 slots."""
    H, d = 2, 8
    L = dense.page_layout(H, d)
    assert L["page_bytes"] == 2 * (H * 16 * d * 2) and L["v"] == H * 16 * d * 2
    pool = np.zeros(3 * L["page_bytes"], np.uint8)
    k = np.arange(1, 9, dtype=np.float64)[None]  # exactly representable in bf16
    v = -np.arange(1, 9, dtype=np.float64)[None]
    dense.write(pool, L, [19], 1, k, v)  # page 1, slot 3, head 1
    w = pool.view(np.uint16)
    for i in range(d):
        kb = L["page_bytes"] + ((1 * 16 + 3) * d + i) * 2
        vb = L["page_bytes"] + L["v"] + ((1 * d + i) * 16 + 3) * 2
        assert w[kb // 2] == np.float32(i + 1).view(np.uint32) >> 16
        assert w[vb // 2] == np.float32(-(i + 1)).view(np.uint32) >> 16
    assert np.count_nonzero(w) == 2 * d


def check_dense_attention_vs_torch_sdpa():
    """Against torch's scaled_dot_product_attention (fp64, CPU) on the stored bf16 values, GQA expanded."""
    import torch

    H, d, Hq, B, lens = 2, 64, 8, 2, [45, 70]
    rng = np.random.Generator(np.random.Philox(52))
    L = dense.page_layout(H, d)
    pt, npages = kvsynth.page_table(B, 5, True, seed=53)
    pool = np.zeros(npages * L["page_bytes"], np.uint8)
    K = rng.standard_normal((B, 80, H, d))
    V = rng.standard_normal((B, 80, H, d))
    for b in range(B):
        for h in range(H):
            dense.write(pool, L, kvsynth.slots_for(pt, b, 0, lens[b]), h, K[b, :lens[b], h], V[b, :lens[b], h])
    q = rng.standard_normal((B, Hq, d))
    out = dense.decode_attention(pool, L, q, pt, lens, 0.2)
    for b in range(B):
        Kt = torch.tensor(K[b, :lens[b]].transpose(1, 0, 2)).to(torch.bfloat16).double().repeat_interleave(Hq // H, 0)
        Vt = torch.tensor(V[b, :lens[b]].transpose(1, 0, 2)).to(torch.bfloat16).double().repeat_interleave(Hq // H, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q[b])[:, None, :], Kt, Vt, scale=0.2)
        assert np.allclose(out[b], ref[:, 0, :].numpy(), rtol=1e-10, atol=1e-12), b


def check_dense_special_cases():
    """One cached token gives its (bf16) value; equal keys give the mean value; length 0 gives zeros."""
    H, d = 1, 64
    L = dense.page_layout(H, d)
    rng = np.random.Generator(np.random.Philox(54))
    pool = np.zeros(4 * L["page_bytes"], np.uint8)
    pt = np.array([[2, 0, 3, 1]], np.int32)
    k = np.repeat(rng.standard_normal((1, d)), 40, axis=0)
    v = rng.standard_normal((40, d))
    dense.write(pool, L, kvsynth.slots_for(pt, 0, 0, 40), 0, k, v)
    q = rng.standard_normal((1, 4, d))
    vb = dense.bf16_value(dense.bf16_bits(v))
    assert np.allclose(dense.decode_attention(pool, L, q, pt, [1], 0.3)[0], vb[0][None, :], atol=1e-13)
    assert np.allclose(dense.decode_attention(pool, L, q, pt, [40], 0.3)[0], vb.mean(axis=0)[None, :], atol=1e-13)
    assert np.all(dense.decode_attention(pool, L, q, pt, [0], 0.3) == 0)


# --------------------------------------------------------------------------------------------
# Uncompressed comparator (FP8 E4M3 pages, one scale per tensor)
# --------------------------------------------------------------------------------------------


def check_fp8_value_table():
    """Every byte's value against torch's float8_e4m3fn, NaN patterns included."""
    import torch

    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e4m3fn).double().numpy()
    got = dense.fp8_value(b)
    assert np.array_equal(np.isnan(want), np.isnan(got)) and np.isnan(got).sum() == 2
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    assert dense.fp8_value(0x7E) == 448.0 and dense.fp8_value(0x01) == 2.0 ** -9 and dense.fp8_value(0x08) == 2.0 ** -6


def check_fp8_rounding_vs_torch(seed=55):
    """Round-to-nearest-even to E4M3 against torch's conversion: random values over the whole range, every
    representable value and every midpoint between neighbours (the ties), both signs."""
    import torch

    rng = np.random.Generator(np.random.Philox(seed))
    x = (rng.standard_normal(40000) * np.exp(rng.uniform(-14, 7, 40000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    b = np.arange(0x7F, dtype=np.uint8)
    vals = dense.fp8_value(b)
    mids = (vals[1:] + vals[:-1]) / 2  # exact in fp32
    x = np.concatenate([x, vals, mids, -vals, -mids]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(dense.fp8_bits(x), want)


def check_fp8_rounding_brute_force(seed=56):
    """Nearest finite E4M3 value by exhaustive search, ties to the even code; saturation above 448."""
    rng = np.random.Generator(np.random.Philox(seed))
    y = np.concatenate([rng.uniform(-460, 460, 3000), rng.standard_normal(3000) * 0.02,
                        np.float64([464.0, 1e6, -1e30, 449.0, 2 ** -10, -(2 ** -10), 3 * 2 ** -11])]).astype(np.float32)
    codes = np.arange(256)
    vals = dense.fp8_value(codes)
    fin = ~np.isnan(vals)
    got = dense.fp8_bits(y)
    for yi, gi in zip(y.astype(np.float64), got):
        sign = 0x80 if np.signbit(yi) else 0
        cand = codes[fin & ((codes & 0x80) == sign)]
        dist = np.abs(np.abs(dense.fp8_value(cand)) - min(abs(yi), 448.0))
        best = cand[dist == dist.min()]
        best = best[(best & 1) == 0] if len(best) > 1 else best
        assert len(best) == 1 and best[0] == gi, (yi, gi, best)


def check_fp8_scale_and_layout_by_hand():
    """The scale divides before rounding and multiplies on read; byte positions of one token written by hand
    (K row contiguous, V column strided by 16 slots, 1 byte per element)."""
    H, d = 2, 8
    L = dense.page_layout(H, d, "fp8", k_scale=0.5, v_scale=4.0)
    assert L["page_bytes"] == 2 * H * 16 * d and L["v"] == H * 16 * d
    pool = np.zeros(3 * L["page_bytes"], np.uint8)
    k = np.arange(1, 9, dtype=np.float64)[None] * 0.5  # k / 0.5 = 1..8, exact in E4M3
    v = -np.arange(1, 9, dtype=np.float64)[None] * 4.0  # v / 4 = -1..-8
    dense.write(pool, L, [19], 1, k, v)  # page 1, slot 3, head 1
    for i in range(d):
        kb = L["page_bytes"] + (1 * 16 + 3) * d + i
        vb = L["page_bytes"] + L["v"] + (1 * d + i) * 16 + 3
        assert dense.fp8_value(pool[kb]) == i + 1 and dense.fp8_value(pool[vb]) == -(i + 1)
    assert np.count_nonzero(pool) == 2 * d
    K, V = dense.gather(pool, L, [0, 1], 20, 1)
    assert np.array_equal(K[19], k[0]) and np.array_equal(V[19], v[0]) and not K[:19].any()


def check_dense_fp8_attention_vs_torch_sdpa():
    """Against torch's scaled_dot_product_attention (fp64, CPU) on scale * E4M3(x / scale) made by torch's
    own conversion, GQA expanded."""
    import torch

    H, d, Hq, B, lens, ks, vs = 2, 64, 8, 2, [45, 70], 0.25, 3.0
    rng = np.random.Generator(np.random.Philox(57))
    L = dense.page_layout(H, d, "fp8", k_scale=ks, v_scale=vs)
    pt, npages = kvsynth.page_table(B, 5, True, seed=58)
    pool = np.zeros(npages * L["page_bytes"], np.uint8)
    K = rng.standard_normal((B, 80, H, d))
    V = rng.standard_normal((B, 80, H, d)) * 20
    for b in range(B):
        for h in range(H):
            dense.write(pool, L, kvsynth.slots_for(pt, b, 0, lens[b]), h, K[b, :lens[b], h], V[b, :lens[b], h])
    q = rng.standard_normal((B, Hq, d))
    out = dense.decode_attention(pool, L, q, pt, lens, 0.2)

    def f8(x, s):
        return (torch.tensor(x).float() / s).to(torch.float8_e4m3fn).double() * s

    for b in range(B):
        Kt = f8(K[b, :lens[b]].transpose(1, 0, 2), ks).repeat_interleave(Hq // H, 0)
        Vt = f8(V[b, :lens[b]].transpose(1, 0, 2), vs).repeat_interleave(Hq // H, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q[b])[:, None, :], Kt, Vt, scale=0.2)
        assert np.allclose(out[b], ref[:, 0, :].numpy(), rtol=1e-10, atol=1e-12), b



# --------------------------------------------------------------------------------------------
# Dense random (QR) rotation
# --------------------------------------------------------------------------------------------


def check_qr_rotation_factorization(d=64, seed=61):
    """Q is orthogonal, Q^T G is upper triangular with a positive diagonal and Q (Q^T G) = G."""
    G = kvsynth.qr_gaussian(seed, d)
    Q = rotation.qr_rotation(G)
    assert np.abs(Q.T @ Q - np.eye(d)).max() < 1e-13 and np.abs(Q @ Q.T - np.eye(d)).max() < 1e-13
    T = Q.T @ G
    assert np.abs(np.tril(T, -1)).max() < 1e-12 and np.all(np.diag(T) > 0)
    assert np.abs(Q @ np.triu(T) - G).max() < 1e-12


def check_qr_rotation_gram_schmidt(d=8, seed=62):
    """Against classical Gram-Schmidt on the columns of G written out by hand (the QR with a positive
    triangular diagonal is unique)."""
    G = kvsynth.qr_gaussian(seed, d)
    cols = []
    for j in range(d):
        v = [G[i][j] for i in range(d)]
        for q in cols:
            dot = sum(q[i] * G[i][j] for i in range(d))
            v = [v[i] - dot * q[i] for i in range(d)]
        nrm = math.sqrt(sum(t * t for t in v))
        cols.append([t / nrm for t in v])
    Q = np.array(cols).T
    assert np.abs(rotation.qr_rotation(G) - Q).max() < 1e-12
    # a triangular G with a positive diagonal is its own T: Q = I
    U = np.triu(G) + np.diag(np.abs(np.diag(G)) + 1.0 - np.diag(G))
    assert np.abs(rotation.qr_rotation(U) - np.eye(d)).max() < 1e-14


def check_dense_rotation_reduces_to_known_paths(d=64, n=400, seed=63):
    """The codec's dense branch against the two rotations it can reproduce: the WHT matrix given as a dense
    matrix encodes and decodes exactly as the sign-vector codebook does, and the identity quantizes the
    coordinates of u themselves."""
    rng = np.random.Generator(np.random.Philox(seed))
    x = rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))
    sw = kvsynth.rotation_signs(seed, d)
    for b in (2, 4):
        cw = codec.make_codebook(d, b, codec.MSE, sw)
        cd = codec.make_codebook(d, b, codec.MSE, np.zeros(d // 32, np.uint32), dense=rotation.rotation_matrix(sw, d))
        ew, ed = codec.encode(x, cw), codec.encode(x, cd)
        assert np.array_equal(ew.codes, ed.codes) and np.array_equal(ew.norm16, ed.norm16)
        assert np.abs(codec.dequantize(ed.codes, ed.norm16, cd) - codec.dequantize(ew.codes, ew.norm16, cw)).max() < 1e-12
        ci = codec.make_codebook(d, b, codec.MSE, sw, dense=np.eye(d))
        ei = codec.encode(x, ci)
        u = x / np.linalg.norm(x, axis=1, keepdims=True)
        want = np.searchsorted(ci.thresholds, (u * math.sqrt(d)).astype(np.float32).astype(np.float64), side="right")
        assert np.array_equal(codec.level_index(ei.codes, b), want)
        # no rotation: the reconstruction is the per-coordinate quantization of u itself
        assert np.abs(codec.dequantize(ei.codes, np.ones(n), ci) - ci.levels16[want] / math.sqrt(d)).max() < 1e-15


def check_dense_rotation_mse(d=128, n=3000, seed=64):
    """Gaussian vectors through a QR rotation: E||u - uhat||^2 matches the Lloyd-Max distortion D_b, as for the
    WHT; outlier channels (x 10 on four coordinates) are spread by the rotation just as well."""
    rng = np.random.Generator(np.random.Philox(seed))
    x = rng.standard_normal((n, d))
    x[:, :4] *= 10.0
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    Q = rotation.qr_rotation(kvsynth.qr_gaussian(seed, d))
    for b in (2, 3, 4):
        cb = codec.make_codebook(d, b, codec.MSE, np.zeros(d // 32, np.uint32), dense=Q)
        e = codec.encode(x, cb)
        mse = np.mean(np.sum((u - codec.dequantize(e.codes, np.ones(n), cb)) ** 2, axis=1))
        c = lloyd_max.levels(b)
        D = lloyd_max.distortion(c, lloyd_max.thresholds_of(c))
        assert abs(mse / D - 1) < 0.05, (b, mse, D)


def check_dense_attention_two_routes():
    """Decode attention with QR-rotated K and V: dequantize-then-attend equals attend-in-the-rotated-domain."""
    for (kb, km, vb, vm) in ((4, 0, 2, 0), (3, 0, 3, 0)):
        c = build_cache(2, 64, 8, 2, [37, 70], kb, km, vb, vm, seed=70 + kb, dense=True)
        o1 = attention.decode_attention(c["pool"], c["L"], c["cbk"], c["cbv"], c["q"], c["pt"], c["lens"], 0.125)
        o2 = attention.decode_attention_rotated(c["pool"], c["L"], c["cbk"], c["cbv"], c["q"], c["pt"], c["lens"], 0.125)
        assert attention.relative_error(o1, o2) < 1e-10

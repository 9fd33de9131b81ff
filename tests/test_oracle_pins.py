"""Pins of the CPU oracle against things other than itself.

Each test fixes part of the oracle by a closed form, a hand-worked value
(``tests/golden``), a special case that reduces to a library routine, or an
invariant of the mathematics, so that a plausible slip in the oracle (a
dropped term, a wrong sign or index, a transposed operand, a wrong rounding)
fails at least one of them.  All run on the CPU.
"""
from __future__ import annotations

import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.linalg
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128


def _golden(name):
    fields = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            fields[key] = vals
    return fields


def _unpack(codes_bytes: np.ndarray) -> np.ndarray:
    lo = (codes_bytes & 0xF).astype(np.int32)
    hi = (codes_bytes >> 4).astype(np.int32)
    c = np.empty(codes_bytes.size * 2, np.int32)
    c[0::2] = np.where(lo >= 8, lo - 16, lo)
    c[1::2] = np.where(hi >= 8, hi - 16, hi)
    return c


def _block_hadamard(n: int, bh: int) -> np.ndarray:
    """Block-diagonal Sylvester matrix from scipy (unnormalised)."""
    if bh == 0:
        return np.eye(n)
    return scipy.linalg.block_diag(*([scipy.linalg.hadamard(bh)] * (n // bh))).astype(np.float64)


# --------------------------------------------------------------------------
# fp16 conversion
# --------------------------------------------------------------------------

def test_f16_to_f32_exhaustive_against_numpy():
    """Every one of the 65,536 half bit patterns widens to numpy's value and
    (non-NaN) narrows back to itself."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    for h in range(65536):
        got = np.float32(oracle.f16_bits_to_f32(h))
        r = ref[h]
        if np.isnan(r):
            assert np.isnan(got)
            continue
        assert got.view(np.uint32) == r.view(np.uint32), hex(h)
        assert oracle.f32_to_f16_bits(got) == h, hex(h)


def test_f32_to_f16_rounding_sweep_against_numpy():
    """Round-to-nearest-even narrowing on a float sweep that includes every
    exact midpoint between neighbouring halves of several binades, the
    subnormal range, overflow and signed zeros; numpy's astype(float16) is an
    IEEE round-to-nearest-even conversion."""
    r = np.random.default_rng(7)
    vals = [np.float32(0.0), np.float32(-0.0), np.float32(65504), np.float32(65519.99),
            np.float32(65520), np.float32(1e6), np.float32(2.0 ** -25), np.float32(2.0 ** -26),
            np.float32(3 * 2.0 ** -26)]
    halves = np.arange(0, 0x7C00, 7, dtype=np.uint16).view(np.float16).astype(np.float32)
    nxt = (np.arange(0, 0x7C00, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float32)
    mids = ((halves.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)
    vals += list(mids) + list(-mids)
    vals += list(r.standard_normal(20000).astype(np.float32) * np.float32(10.0) **
                 r.integers(-8, 5, 20000).astype(np.float32))
    for v in vals:
        v = np.float32(v)
        want = np.array([v], np.float32).astype(np.float16).view(np.uint16)[0]
        assert oracle.f32_to_f16_bits(v) == want, (float(v), hex(want))


# --------------------------------------------------------------------------
# Rotation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bh", [32, 64, 128])
def test_hadamard_scale_is_nearest_float_of_inverse_sqrt(bh):
    """c_B = round-to-nearest binary32 of 1/sqrt(Bh), decided with 50 digits."""
    getcontext().prec = 50
    exact = Decimal(1) / Decimal(bh).sqrt()
    c = oracle.hadamard_scale(bh)
    lo = np.nextafter(c, np.float32(0))
    hi = np.nextafter(c, np.float32(1))
    err = abs(Decimal(float(c)) - exact)
    assert err <= abs(Decimal(float(lo)) - exact)
    assert err <= abs(Decimal(float(hi)) - exact)
    expect = {32: 0x3E3504F3, 64: 0x3E000000, 128: 0x3DB504F3}[bh]
    assert np.float32(c).view(np.uint32) == expect


@pytest.mark.parametrize("bh", [2, 4, 8, 16, 32, 64, 128])
def test_fwht_equals_block_sylvester_matrix_on_small_integers(bh):
    """On small integers every partial sum is exact in fp32, so the butterfly
    network must equal the dense block-diagonal Sylvester product exactly."""
    r = np.random.default_rng(bh)
    H = _block_hadamard(D, bh)
    for _ in range(5):
        x = r.integers(-8, 9, D).astype(np.float32)
        got = oracle.fwht_f32(x, bh)
        want = H @ x.astype(np.float64)
        assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("bh", [4, 32, 128])
def test_fwht_of_unit_vectors_gives_signed_columns(bh):
    """FWHT(e_k)[j] = (-1)^popcount(j & k) inside k's block, 0 elsewhere."""
    for k in range(0, D, 7):
        x = np.zeros(D, np.float32)
        x[k] = 1.0
        got = oracle.fwht_f32(x, bh)
        b0 = (k // bh) * bh
        want = np.zeros(D)
        for j in range(bh):
            want[b0 + j] = (-1.0) ** bin(j & (k - b0)).count("1")
        assert np.array_equal(got, want)


def test_fwht_butterfly_order_golden():
    g = _golden("fwht_order_bh4.txt")
    x = np.array([float(v) for v in g["input"]], np.float32)
    want = np.array([float(v) for v in g["output"]], np.float32)
    got = oracle.fwht_f32(x, 4)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("bh", [32, 64, 128])
def test_rotation_is_involutive_and_norm_preserving(bh):
    r = np.random.default_rng(11 + bh)
    x = r.standard_normal((4, D)) * 3
    y = oracle.rotate_f64(x, bh)
    assert np.allclose(oracle.rotate_f64(y, bh), x, atol=1e-12)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    # against scipy's Hadamard divided by sqrt(Bh)
    R = _block_hadamard(D, bh) / math.sqrt(bh)
    assert np.allclose(y, x @ R.T, atol=1e-12)
    # fp32 path used by quantization: R(Rx) = x within 1e-6
    c = oracle.hadamard_scale(bh)
    x32 = (r.standard_normal(D) * 3).astype(np.float32)
    once = oracle.fwht_f32(x32, bh) * c
    twice = oracle.fwht_f32(once, bh) * c
    assert np.max(np.abs(twice - x32)) <= 1e-6 * max(1.0, np.max(np.abs(x32)))


@pytest.mark.parametrize("bh", [32, 64])
def test_rotation_stays_inside_its_block(bh):
    r = np.random.default_rng(5)
    for blk in range(D // bh):
        x = np.zeros(D, np.float32)
        x[blk * bh:(blk + 1) * bh] = r.standard_normal(bh)
        y = oracle.fwht_f32(x, bh)
        outside = np.ones(D, bool)
        outside[blk * bh:(blk + 1) * bh] = False
        assert np.all(y[outside] == 0)
        assert np.any(y[~outside] != 0)


def test_rotated_dot_product_identity():
    """(R q).(R k) = q.k: the identity that lets decode rotate the query."""
    r = np.random.default_rng(3)
    for bh in (32, 64, 128):
        q = r.standard_normal(D)
        k = r.standard_normal(D)
        assert abs(oracle.rotate_f64(q, bh) @ oracle.rotate_f64(k, bh) - q @ k) < 1e-9


# --------------------------------------------------------------------------
# Quantization
# --------------------------------------------------------------------------

def test_worked_example_bh0_golden():
    g = _golden("worked_example_bh0.txt")
    x = np.zeros(int(g["head_dim"][0]), np.float16)
    vals = [float(v) for v in g["input"]]
    x[:len(vals)] = vals
    codes, scale = oracle.quantize_vector(x, 0)
    assert scale == int(g["scale_bits"][0], 16)
    want_codes = [int(v) for v in g["codes"]]
    assert list(_unpack(codes)[:len(want_codes)]) == want_codes
    want_bytes = [int(v, 16) for v in g["bytes"]]
    assert list(codes[:len(want_bytes)]) == want_bytes
    assert np.all(codes[len(want_bytes):] == 0)


def test_subnormal_scale_reaches_the_clamp_golden():
    g = _golden("subnormal_scale_clamp.txt")
    x = np.zeros(int(g["head_dim"][0]), np.float16)
    units = [int(v) for v in g["input_units_of_2^-24"]]
    x[:len(units)] = np.array(units, np.float64) * 2.0 ** -24
    codes, scale = oracle.quantize_vector(x, 0)
    assert scale == int(g["scale_bits"][0], 16)
    assert list(_unpack(codes)[:2]) == [int(v) for v in g["codes"]]
    assert list(codes[:2]) == [int(v, 16) for v in g["bytes"]]


def test_zero_vector_gives_zero_scale_and_codes():
    for bh in (0, 32, 64, 128):
        codes, scale = oracle.quantize_vector(np.zeros(D, np.float16), bh)
        assert scale == 0 and not codes.any()


def test_worked_tie_under_rotation_bh64():
    """With Bh = 64, 1/sqrt(64) = 1/8 is exact.  Pick a target y of
    half-integers with absmax 7 and set x = H y / 8; x is exactly
    representable in fp16, the FWHT reproduces 8 y exactly, the scale is 1,
    and the codes are round-half-even(y), known in advance."""
    r = np.random.default_rng(2024)
    H = _block_hadamard(D, 64)
    for _ in range(20):
        y = r.integers(-14, 15, D) / 2.0
        y[r.integers(0, D)] = 7.0 * r.choice([-1, 1])
        y = np.clip(y, -7, 7)
        x = H @ y / 8.0  # H is symmetric and H.H = 64 I per block
        xh = x.astype(np.float16)
        assert np.array_equal(xh.astype(np.float64), x), "x must be exact in fp16"
        codes, scale = oracle.quantize_vector(xh, 64)
        assert scale == 0x3C00
        assert np.array_equal(_unpack(codes), np.rint(y).astype(np.int32))


def test_one_hot_spreads_to_equal_magnitude_codes():
    """A single channel spreads over its whole block with equal magnitude:
    codes are +-7 with the signs of the Hadamard column, 0 elsewhere."""
    for bh in (32, 64, 128):
        for k in (0, 5, 77, 127):
            x = np.zeros(D, np.float16)
            x[k] = 3.0
            codes, scale = oracle.quantize_vector(x, bh)
            c = _unpack(codes)
            b0 = (k // bh) * bh
            want = np.zeros(D, np.int32)
            for j in range(bh):
                want[b0 + j] = 7 * (-1) ** bin(j & (k - b0)).count("1")
            assert np.array_equal(c, want), (bh, k)


@pytest.mark.parametrize("bh", [0, 32, 64, 128])
def test_quantization_error_bound_and_code_range(bh):
    """|y - s16 c| <= s16/2 (1 + 2^-20) for a normal fp16 scale; |c| <= 7 and
    -8 never occurs; the absmax element has |c| = 7.  y is the oracle's own
    fp32 rotation of x (FWHT then x c_B), pinned separately above."""
    r = np.random.default_rng(100 + bh)
    for trial in range(200):
        x = r.standard_normal(D).astype(np.float32)
        x[r.choice(D, 4, replace=False)] *= 20
        x *= np.float32(10.0 ** r.uniform(-3, 2))
        xh = x.astype(np.float16)
        codes, s16 = oracle.quantize_vector(xh, bh)
        c = _unpack(codes)
        y = xh.astype(np.float32)
        if bh:
            y = oracle.fwht_f32(y, bh) * oracle.hadamard_scale(bh)
        s = float(np.array([s16], np.uint16).view(np.float16)[0])
        assert s >= 2.0 ** -14, "trial inputs keep the scale normal"
        assert np.all(np.abs(c) <= 7)
        err = np.abs(y.astype(np.float64) - s * c)
        assert np.all(err <= s / 2 * (1 + 2.0 ** -20))
        assert abs(c[np.argmax(np.abs(y))]) == 7


def test_rotation_reduces_error_on_outlier_channels():
    """The pages' central claim, in miniature: with 4 channels x20 per vector,
    rotated INT4 reconstructs with much lower MSE than naive INT4."""
    r = np.random.default_rng(9)
    ch = r.choice(D, 4, replace=False)
    mse = {}
    for bh in (0, 32, 64, 128):
        tot = 0.0
        for _ in range(300):
            x = r.standard_normal(D)
            x[ch] *= 20
            xh = x.astype(np.float16)
            codes, s16 = oracle.quantize_vector(xh, bh)
            s = float(np.array([s16], np.uint16).view(np.float16)[0])
            rec = _unpack(codes) * s
            if bh:
                rec = oracle.rotate_f64(rec, bh)
            tot += np.mean((rec - xh.astype(np.float64)) ** 2)
        mse[bh] = tot / 300
    assert mse[32] < 0.5 * mse[0] and mse[64] < 0.5 * mse[0] and mse[128] < 0.5 * mse[0]


# --------------------------------------------------------------------------
# Placement
# --------------------------------------------------------------------------

def test_placement_golden_and_nothing_else_changes():
    g = _golden("placement_small.txt")
    hkv, P, npg = int(g["num_kv_heads"][0]), int(g["page_size"][0]), int(g["num_pages"][0])
    pt = np.array([int(v) for v in g["page_table"]], np.int32).reshape(2, 2)
    tb = oracle.tile_bytes(D, P)
    assert tb == 1056
    r = np.random.default_rng(1)
    canary_k = r.integers(0, 256, npg * hkv * tb).astype(np.uint8)
    canary_v = r.integers(0, 256, npg * hkv * tb).astype(np.uint8)
    kp, vp = canary_k.copy().reshape(npg, hkv, tb), canary_v.copy().reshape(npg, hkv, tb)
    k = (r.standard_normal((1, hkv, D)) * 3).astype(np.float16)
    v = (r.standard_normal((1, hkv, D)) * 3).astype(np.float16)
    oracle.kv_quant_append(k, v, [int(g["token_seq"][0])], [int(g["token_pos"][0])], pt, kp, vp,
                           had_block=32, page_size=P)
    rng_ = [int(v) for v in g["changed_ranges"]]
    mask = np.zeros(npg * hkv * tb, bool)
    for a, b in zip(rng_[0::2], rng_[1::2]):
        mask[a:b] = True
    for pool, canary, src in ((kp, canary_k, k), (vp, canary_v, v)):
        flat = pool.reshape(-1)
        assert np.array_equal(flat[~mask], canary[~mask])
        # the changed bytes are exactly the quantized vectors
        for h in range(hkv):
            codes, s16 = oracle.quantize_vector(src[0, h], 32)
            a = rng_[4 * h]
            assert np.array_equal(flat[a:a + 64], codes)
            sa = rng_[4 * h + 2]
            assert int(flat[sa]) | (int(flat[sa + 1]) << 8) == s16


def test_fp16_append_placement_matches_hand_worked_golden():
    """The fp16 baseline append writes each token's rows exactly at the byte
    ranges worked by hand in tests/golden/placement_fp16_small.txt (pool
    [num_pages][Hkv][P][D] fp16), as the rows' own fp16 bytes, and touches no
    other byte of a canary-filled pool."""
    g = _golden("placement_fp16_small.txt")
    hkv, P, npg = int(g["num_kv_heads"][0]), int(g["page_size"][0]), int(g["num_pages"][0])
    pt = np.array([int(v) for v in g["page_table"]], np.int32).reshape(2, 2)
    seqs = [int(v) for v in g["token_seq"]]
    poss = [int(v) for v in g["token_pos"]]
    T = len(seqs)
    r = np.random.default_rng(2)
    nbytes = npg * hkv * P * D * 2
    canary_k = r.integers(0, 256, nbytes).astype(np.uint8)
    canary_v = r.integers(0, 256, nbytes).astype(np.uint8)
    kp = canary_k.copy().view(np.float16).reshape(npg, hkv, P, D)
    vp = canary_v.copy().view(np.float16).reshape(npg, hkv, P, D)
    k = (r.standard_normal((T, hkv, D)) * 3).astype(np.float16)
    v = (r.standard_normal((T, hkv, D)) * 3).astype(np.float16)
    oracle.kv_append_fp16(k, v, np.array(seqs, np.int32), np.array(poss, np.int32), pt, kp, vp, P)
    rng_ = [int(x) for x in g["changed_ranges"]]
    mask = np.zeros(nbytes, bool)
    for a, b in zip(rng_[0::2], rng_[1::2]):
        assert b - a == 2 * D
        mask[a:b] = True
    for pool, canary, src in ((kp, canary_k, k), (vp, canary_v, v)):
        flat = pool.reshape(-1).view(np.uint8)
        assert np.array_equal(flat[~mask], canary[~mask])
        for t in range(T):
            for h in range(hkv):
                a = rng_[2 * (t * hkv + h)]
                assert np.array_equal(flat[a:a + 2 * D], src[t, h].view(np.uint8))


def test_append_under_permuted_page_table_matches_vector_quantizer():
    """Every token of every sequence lands in the slot its page table names,
    holding exactly its quantized vector and scale."""
    r = np.random.default_rng(4)
    B, hkv, P, lens = 3, 2, 16, [37, 16, 50]
    maxp = 4
    npg = B * maxp + 2
    perm = r.permutation(npg).astype(np.int32)
    pt = perm[:B * maxp].reshape(B, maxp)
    seq = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(lens)])
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in lens])
    order = r.permutation(seq.size)
    seq, pos = seq[order], pos[order]
    k = (r.standard_normal((seq.size, hkv, D)) * 2).astype(np.float16)
    v = (r.standard_normal((seq.size, hkv, D)) * 2).astype(np.float16)
    tb = oracle.tile_bytes(D, P)
    kp = np.zeros((npg, hkv, tb), np.uint8)
    vp = np.zeros((npg, hkv, tb), np.uint8)
    oracle.kv_quant_append(k, v, seq, pos, pt, kp, vp, had_block=64, page_size=P)
    for t in range(seq.size):
        page = pt[seq[t], pos[t] // P]
        slot = pos[t] % P
        for h in range(hkv):
            for pool, src in ((kp, k), (vp, v)):
                codes, s16 = oracle.quantize_vector(src[t, h], 64)
                pg = pool[page].reshape(-1)          # codes of both heads, then their scales
                c0 = (h * P + slot) * 64
                s0 = hkv * P * 64 + (h * P + slot) * 2
                assert np.array_equal(pg[c0:c0 + 64], codes)
                assert int(pg[s0]) | (int(pg[s0 + 1]) << 8) == s16


def test_append_rejects_out_of_range_page():
    kp = np.zeros((2, 1, 1056), np.uint8)
    vp = np.zeros_like(kp)
    k = np.zeros((1, 1, D), np.float16)
    with pytest.raises(RuntimeError):
        oracle.kv_quant_append(k, k, [0], [40], np.array([[0, 1]], np.int32), kp, vp, 0, 16)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def _softmax_attention_np(q, K, V, scale):
    """Independent dense reference via scipy.special.softmax and numpy matmul.
    q [Hq][D], K/V [L][Hkv][D]."""
    hq, hkv = q.shape[0], K.shape[1]
    g = hq // hkv
    out = np.zeros((hq, q.shape[1]))
    for h in range(hq):
        kk = K[:, h // g, :]
        w = scipy.special.softmax((kk @ q[h]) * scale)
        out[h] = w @ V[:, h // g, :]
    return out


def _build_cache(r, L, hkv, P, bh, npg_extra=2, fp16=False, outliers=True):
    need = (L + P - 1) // P
    npg = need + npg_extra
    perm = r.permutation(npg).astype(np.int32)
    pt = perm[:need].reshape(1, need)
    K = r.standard_normal((L, hkv, D))
    V = r.standard_normal((L, hkv, D))
    if outliers:
        K[:, :, [3, 40]] *= 20
        V[:, :, [7, 90]] *= 20
    K, V = K.astype(np.float16), V.astype(np.float16)
    if fp16:
        kp = np.zeros((npg, hkv, P, D), np.float16)
        vp = np.zeros_like(kp)
        oracle.kv_append_fp16(K, V, np.zeros(L, np.int32), np.arange(L, dtype=np.int32), pt, kp, vp, P)
    else:
        tb = oracle.tile_bytes(D, P)
        kp = np.zeros((npg, hkv, tb), np.uint8)
        vp = np.zeros_like(kp)
        oracle.kv_quant_append(K, V, np.zeros(L, np.int32), np.arange(L, dtype=np.int32), pt,
                               kp, vp, had_block=bh, page_size=P)
    return K, V, pt, kp, vp


def test_fp16_decode_equals_dense_softmax():
    """Paging + GQA + softmax scale: the fp16 baseline over a shuffled page
    table equals scipy softmax attention on the original K/V within 1e-6."""
    r = np.random.default_rng(12)
    L, hkv, hq, P = 45, 2, 8, 16
    K, V, pt, kp, vp = _build_cache(r, L, hkv, P, 0, fp16=True)
    q = r.standard_normal((1, hq, D)).astype(np.float16)
    scale = 1 / math.sqrt(D)
    got = oracle.paged_decode_attn_fp16(q, kp, vp, pt, [L], hkv, P, scale)
    want = _softmax_attention_np(q[0].astype(np.float64), K.astype(np.float64),
                                 V.astype(np.float64), np.float32(scale))
    assert np.max(np.abs(got[0] - want)) < 1e-6
    dense = oracle.dense_decode_f64(q[0], K, V, np.float32(scale))
    assert np.max(np.abs(dense - want)) < 1e-12


@pytest.mark.parametrize("bh", [0, 32, 128])
def test_int4_decode_equals_dense_softmax_on_dequantized_unrotated_cache(bh):
    """Query rotation, inverse output rotation, paging and GQA together: the
    INT4 decode equals dense softmax attention over the cache read back,
    dequantized and rotated back to the original basis with scipy's Hadamard."""
    r = np.random.default_rng(20 + bh)
    L, hkv, hq, P = 53, 2, 8, 16
    _, _, pt, kp, vp = _build_cache(r, L, hkv, P, bh)
    q = r.standard_normal((1, hq, D)).astype(np.float16)
    scale = 1 / math.sqrt(D)
    got = oracle.paged_decode_attn_int4(q, kp, vp, pt, [L], hkv, P, bh, scale)
    Rt = (_block_hadamard(D, bh) / math.sqrt(bh)) if bh else np.eye(D)
    Kd = np.stack([oracle.dequantize_pool(kp, pt, L, 0, h, D, P) for h in range(hkv)], 1) @ Rt.T
    Vd = np.stack([oracle.dequantize_pool(vp, pt, L, 0, h, D, P) for h in range(hkv)], 1) @ Rt.T
    want = _softmax_attention_np(q[0].astype(np.float64), Kd, Vd, np.float32(scale))
    assert np.max(np.abs(got[0] - want)) < 1e-5


def test_int4_decode_single_token_returns_its_value():
    r = np.random.default_rng(30)
    _, _, pt, kp, vp = _build_cache(r, 1, 1, 16, 64)
    q = r.standard_normal((1, 4, D)).astype(np.float16)
    got = oracle.paged_decode_attn_int4(q, kp, vp, pt, [1], 1, 16, 64, 0.088)
    v0 = (oracle.dequantize_pool(vp, pt, 1, 0, 0, D, 16)[0] @ (scipy.linalg.block_diag(
        *[scipy.linalg.hadamard(64)] * 2) / 8.0).T)
    for h in range(4):
        assert np.max(np.abs(got[0, h] - v0)) < 1e-6


def test_int4_decode_zero_query_is_mean_of_values():
    r = np.random.default_rng(31)
    L = 40
    _, _, pt, kp, vp = _build_cache(r, L, 1, 16, 32)
    q = np.zeros((1, 4, D), np.float16)
    got = oracle.paged_decode_attn_int4(q, kp, vp, pt, [L], 1, 16, 32, 0.088)
    R = _block_hadamard(D, 32) / math.sqrt(32)
    mean = (oracle.dequantize_pool(vp, pt, L, 0, 0, D, 16) @ R.T).mean(0)
    assert np.max(np.abs(got[0, 0] - mean)) < 1e-6


def test_decode_zero_length_gives_zero_row_and_ignores_page_table():
    r = np.random.default_rng(32)
    _, _, pt, kp, vp = _build_cache(r, 20, 1, 16, 32)
    q = r.standard_normal((2, 4, D)).astype(np.float16)
    pt2 = np.vstack([pt, np.full_like(pt, -1)])
    got = oracle.paged_decode_attn_int4(q, kp, vp, pt2, [20, 0], 1, 16, 32, 0.088)
    assert np.all(got[1] == 0) and np.any(got[0] != 0)


def test_decode_is_invariant_to_page_permutation():
    """The same logical cache under two different physical placements."""
    r = np.random.default_rng(33)
    L, P, hkv = 70, 16, 2
    K = r.standard_normal((L, hkv, D)).astype(np.float16)
    V = r.standard_normal((L, hkv, D)).astype(np.float16)
    q = r.standard_normal((1, 8, D)).astype(np.float16)
    outs = []
    for seed in (0, 1):
        perm = np.random.default_rng(seed).permutation(6).astype(np.int32)
        pt = perm[:5].reshape(1, 5)
        tb = oracle.tile_bytes(D, P)
        kp = np.zeros((6, hkv, tb), np.uint8)
        vp = np.zeros_like(kp)
        oracle.kv_quant_append(K, V, np.zeros(L, np.int32), np.arange(L, dtype=np.int32), pt, kp, vp,
                               64, P)
        outs.append(oracle.paged_decode_attn_int4(q, kp, vp, pt, [L], hkv, P, 64, 0.088))
    assert np.array_equal(outs[0], outs[1])

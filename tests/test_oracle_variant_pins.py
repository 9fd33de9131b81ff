"""Pins of the oracle's quantizer variants (per-group scales, scale search,
randomized Hadamard, MXFP4) against things other than the oracle itself:
hand-worked values (``tests/golden``), special cases that reduce to the
pinned token-wise method, closed forms of the formats, invariants, and an
independent read-back of the stored bytes.  CPU only."""
from __future__ import annotations

import math
import os

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


def _vector_from(fields):
    x = np.zeros(int(fields["head_dim"][0]), np.float16)
    at = fields.get("input_at", [])
    for i in range(0, len(at), 2):
        x[int(at[i])] = np.float16(float(at[i + 1]))
    if "fill" in fields:
        a, n, v = fields["fill"]
        x[int(a):int(a) + int(n)] = np.float16(float(v))
    return x


def _unpack(codes_bytes):
    lo = (codes_bytes & 0xF).astype(np.int32)
    hi = (codes_bytes >> 4).astype(np.int32)
    c = np.empty(codes_bytes.size * 2, np.int32)
    c[0::2] = lo
    c[1::2] = hi
    return c


def _int4(nib):
    return np.where(nib >= 8, nib - 16, nib)


E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # the format's magnitudes, by code


def _readback(codes, scales, cfg):
    """Independent decode of one stored vector (rotated basis): nibbles,
    fp16 scales through numpy, E8M0 as 2^(byte - 127), E2M1 by table."""
    nib = _unpack(codes)
    G = cfg.scale_group
    if cfg.format == oracle.FMT_INT4:
        s = np.frombuffer(scales.tobytes(), dtype="<f2").astype(np.float64)
        return _int4(nib) * np.repeat(s, G)
    s = 2.0 ** (scales.astype(np.float64) - 127.0)
    mag = E2M1[nib & 7]
    return np.where(nib & 8, -mag, mag) * np.repeat(s, G)


def _rot(bh):
    if bh == 0:
        return np.eye(D)
    return scipy.linalg.block_diag(*([scipy.linalg.hadamard(bh)] * (D // bh))) / math.sqrt(bh)


def _signs(mask):
    return np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(D)])


def _outlier_rows(n, seed, k=8, mult=50.0):
    r = np.random.default_rng(seed)
    ch = r.choice(D, k, replace=False)
    x = r.standard_normal((n, D)).astype(np.float32)
    x[:, ch] *= mult
    return x.astype(np.float16), ch


# ----------------------------------------------------------------------------
# INT4 with per-group scales
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("bh", [0, 32, 64, 128])
def test_group_of_128_is_the_token_wise_method(bh):
    """scale_group = 128 is the method itself: byte for byte the pinned
    token-wise quantizer, for every block size."""
    r = np.random.default_rng(bh)
    cfg = oracle.qcfg(oracle.FMT_INT4, bh, 128, 0)
    for _ in range(50):
        x = (r.standard_normal(D) * r.choice([0.01, 1, 30])).astype(np.float16)
        c0, s0 = oracle.quantize_vector(x, bh)
        c1, s1 = oracle.quantize_vector_cfg(x, cfg)
        assert np.array_equal(c0, c1)
        assert int(np.frombuffer(s1.tobytes(), "<u2")[0]) == s0


def test_group_scales_hand_worked():
    g = _golden("group_scales_bh0_g32.txt")
    cfg = oracle.qcfg(oracle.FMT_INT4, 0, int(g["group"][0]), 0)
    codes, scales = oracle.quantize_vector_cfg(_vector_from(g), cfg)
    want_scales = [int(v, 16) for v in g["scale_bits"]]
    assert list(np.frombuffer(scales.tobytes(), "<u2")) == want_scales
    want = np.zeros(D // 2, np.uint8)
    at = g["bytes_at"]
    for i in range(0, len(at), 2):
        want[int(at[i])] = int(at[i + 1], 16)
    assert np.array_equal(codes, want)


@pytest.mark.parametrize("bh,G", [(0, 32), (32, 32), (64, 64), (128, 32), (0, 64)])
def test_group_scales_bounds_and_absmax_codes(bh, G):
    """In every group with a normal fp16 scale: |y - s c| <= s/2 (1 + 2^-20),
    |c| <= 7, the group's absmax element has |c| = 7; an all-zero group has
    scale 0 and zero codes."""
    r = np.random.default_rng(7 + bh + G)
    cfg = oracle.qcfg(oracle.FMT_INT4, bh, G, 0)
    R = _rot(bh)
    for _ in range(40):
        x = (r.standard_normal(D) * 3).astype(np.float16)
        x[:G] = 0 if r.random() < 0.3 else x[:G]
        codes, scales = oracle.quantize_vector_cfg(x, cfg)
        y = R @ x.astype(np.float64)
        c = _int4(_unpack(codes))
        s = np.frombuffer(scales.tobytes(), "<f2").astype(np.float64)
        for gi in range(D // G):
            sl = slice(gi * G, (gi + 1) * G)
            if s[gi] == 0:
                assert np.all(c[sl] == 0) and np.max(np.abs(y[sl])) < 1e-3
                continue
            assert np.all(np.abs(c[sl]) <= 7)
            assert np.all(np.abs(y[sl] - s[gi] * c[sl]) <= s[gi] / 2 * (1 + 2 ** -20) + 1e-6 * np.abs(y[sl]))
            assert abs(c[sl][np.argmax(np.abs(y[sl]))]) == 7


def test_group_scales_lower_error_on_outlier_channels():
    """The claim the variant is for: on keys with a few x50 outlier channels,
    one scale per Hadamard block of 32 gives less than half the
    reconstruction error of one scale per token (both rotated, Bh 32)."""
    x, _ = _outlier_rows(200, 3)
    tok = oracle.qcfg(oracle.FMT_INT4, 32, 128, 0)
    blk = oracle.qcfg(oracle.FMT_INT4, 32, 32, 0)
    e_tok = np.mean([np.mean((oracle.reconstruct_cfg(v, tok) - v.astype(np.float64)) ** 2) for v in x])
    e_blk = np.mean([np.mean((oracle.reconstruct_cfg(v, blk) - v.astype(np.float64)) ** 2) for v in x])
    assert e_blk < 0.5 * e_tok


# ----------------------------------------------------------------------------
# Scale search
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["scale_search_g32.txt", "scale_search_tie_g32.txt"])
def test_scale_search_hand_worked(name):
    g = _golden(name)
    cfg = oracle.qcfg(oracle.FMT_INT4, 0, int(g["group"][0]), 1)
    codes, scales = oracle.quantize_vector_cfg(_vector_from(g), cfg)
    assert list(np.frombuffer(scales.tobytes(), "<u2")) == [int(v, 16) for v in g["scale_bits"]]
    at = g["bytes_at"]
    for i in range(0, len(at), 2):
        assert codes[int(at[i])] == int(at[i + 1], 16), at[i]


def test_scale_search_candidates_are_clipping_ratios():
    """The chosen scale is one of the 8 candidates fp16(fp32(m a)/7), a =
    16/16 .. 9/16, and on a vector with no outlier (all entries equal in
    magnitude) no clipping can pay: the search keeps a = 1."""
    r = np.random.default_rng(5)
    cfg = oracle.qcfg(oracle.FMT_INT4, 0, 32, 1)
    f16 = lambda v: float(np.float16(np.float32(v)))
    for _ in range(30):
        x = (r.standard_normal(D) * 2).astype(np.float16)
        _, scales = oracle.quantize_vector_cfg(x, cfg)
        s = np.frombuffer(scales.tobytes(), "<f2").astype(np.float64)
        for gi in range(4):
            m = np.float32(np.max(np.abs(x[gi * 32:(gi + 1) * 32].astype(np.float32))))
            cands = [f16(np.float32(np.float32(m * np.float32((16 - k) / 16)) / np.float32(7))) for k in range(8)]
            assert s[gi] in cands
    x = np.where(r.random(D) < 0.5, -1.5, 1.5).astype(np.float16)
    _, scales = oracle.quantize_vector_cfg(x, cfg)
    assert np.all(np.frombuffer(scales.tobytes(), "<f2") == np.float16(1.5 / 7))


def test_scale_search_lowers_error_on_outlier_channels():
    """Clipping search lowers the mean reconstruction error against absmax/7
    on outlier-heavy keys (rotated, block scales), and never makes any single
    group's error more than marginally worse."""
    x, _ = _outlier_rows(200, 4)
    plain = oracle.qcfg(oracle.FMT_INT4, 32, 32, 0)
    srch = oracle.qcfg(oracle.FMT_INT4, 32, 32, 1)
    e_p = np.array([np.mean((oracle.reconstruct_cfg(v, plain) - v.astype(np.float64)) ** 2) for v in x])
    e_s = np.array([np.mean((oracle.reconstruct_cfg(v, srch) - v.astype(np.float64)) ** 2) for v in x])
    assert e_s.mean() < 0.9 * e_p.mean()
    assert np.all(e_s <= e_p * 1.01 + 1e-9)


# ----------------------------------------------------------------------------
# Randomized Hadamard (random +-1 diagonal before the rotation)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("bh,G", [(32, 32), (64, 128), (128, 32)])
def test_sign_mask_is_negated_input(bh, G):
    """Quantizing x with the sign mask S equals quantizing S x without it,
    byte for byte (negation is exact)."""
    r = np.random.default_rng(bh + G)
    mask = int(r.integers(0, 2 ** 63)) | (int(r.integers(0, 2 ** 63)) << 64)
    S = _signs(mask)
    with_s = oracle.qcfg(oracle.FMT_INT4, bh, G, 0, mask)
    without = oracle.qcfg(oracle.FMT_INT4, bh, G, 0, 0)
    for _ in range(20):
        x = (r.standard_normal(D) * 4).astype(np.float16)
        a = oracle.quantize_vector_cfg(x, with_s)
        b = oracle.quantize_vector_cfg((x.astype(np.float64) * S).astype(np.float16), without)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_reconstruction_undoes_signs_and_rotation():
    """For a vector the quantizer represents exactly (x = S R y with y integer
    codes of absmax 7 per group, R = H/8 at Bh 64), the reconstruction
    returns x itself: the inverse of R S is S R."""
    r = np.random.default_rng(9)
    mask = int(r.integers(0, 2 ** 62)) << 3
    S = _signs(mask)
    cfg = oracle.qcfg(oracle.FMT_INT4, 64, 64, 0, mask)
    H = _rot(64)
    for _ in range(10):
        y = r.integers(-7, 8, size=D).astype(np.float64)
        y[0], y[64] = 7, -7
        x = S * (H @ y)
        assert np.array_equal(x, x.astype(np.float16).astype(np.float64))   # multiples of 1/8, |x| <= 56
        back = oracle.reconstruct_cfg(x.astype(np.float16), cfg)
        assert np.max(np.abs(back - x)) < 1e-12


# ----------------------------------------------------------------------------
# MXFP4
# ----------------------------------------------------------------------------

def test_e2m1_values_are_the_format_table():
    assert [oracle.e2m1_value(c) for c in range(8)] == list(E2M1)
    assert [oracle.e2m1_value(c + 8) for c in range(8)] == list(-E2M1)


def test_e2m1_rounding_hand_worked():
    g = _golden("e2m1_rounding.txt")
    vals = [float(v) for v in g["values"]]
    x = np.zeros(D, np.float16)
    x[:len(vals)] = np.array(vals, np.float16)
    codes, scales = oracle.quantize_vector_cfg(x, oracle.qcfg(oracle.FMT_MXFP4, 0, 32))
    nib = _unpack(codes)
    assert list(nib[:len(vals)]) == [int(c) for c in g["codes"]]
    assert int(scales[0]) == int(g["scale_byte"][0])
    assert np.all(scales[1:] == 0) and np.all(nib[32:] == 0)   # zero groups: byte 0, zero codes


def test_e8m0_exponent_is_floor_log2_minus_2():
    """Over every positive finite fp16 value as a group's absmax, the shared
    scale byte is floor(log2 m) - 2 + 127."""
    cfg = oracle.qcfg(oracle.FMT_MXFP4, 0, 32)
    for bits in range(1, 0x7C00, 7):
        m = np.array([bits], np.uint16).view(np.float16)[0]
        x = np.zeros(D, np.float16)
        x[5] = m
        x[6] = -m / np.float16(3)
        _, scales = oracle.quantize_vector_cfg(x, cfg)
        assert int(scales[0]) == math.floor(math.log2(float(m))) - 2 + 127, float(m)


def test_mxfp4_element_error_bound():
    """Each element's error is at most half the E2M1 spacing at its magnitude
    times the shared scale, except where it saturates at 6 (a clip of at most
    2 scale units, since the absmax is below 8 scale units)."""
    r = np.random.default_rng(12)
    cfg = oracle.qcfg(oracle.FMT_MXFP4, 32, 32)
    R = _rot(32)
    half_gap = np.array([0.25, 0.25, 0.25, 0.25, 0.5, 0.5, 1.0, 1.0])   # per code: half the gap to a neighbour
    for _ in range(40):
        x = (r.standard_normal(D) * r.choice([0.01, 1, 20])).astype(np.float16)
        codes, scales = oracle.quantize_vector_cfg(x, cfg)
        y = R @ x.astype(np.float64)
        got = _readback(codes, scales, cfg)
        s = np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32)
        nib = _unpack(codes)
        sat = (nib & 7) == 7
        bound = np.where(sat, 2.0 * s, half_gap[nib & 7] * s) * (1 + 1e-6)
        assert np.all(np.abs(y - got) <= bound)
        assert np.all(np.abs(y) / s < 8)


# ----------------------------------------------------------------------------
# Attention over a variant's cache
# ----------------------------------------------------------------------------

def _pool_case(cfg, lens, P=16, hkv=2, hq=8, seed=0, x_fn=None):
    r = np.random.default_rng(seed)
    B = len(lens)
    need = [max(1, -(-L // P)) for L in lens]
    perm = r.permutation(sum(need) + 2).astype(np.int32)
    pt = np.full((B, max(need)), -1, np.int32)
    off = 0
    for b in range(B):
        pt[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    tb = oracle.tile_bytes_cfg(D, P, cfg)
    kp = r.integers(0, 256, size=(perm.size, hkv, tb)).astype(np.uint8)
    vp = r.integers(0, 256, size=(perm.size, hkv, tb)).astype(np.uint8)
    ks, vs = [], []
    for b, L in enumerate(lens):
        k = x_fn(r, (L, hkv, D)) if x_fn else (r.standard_normal((L, hkv, D)) * 2).astype(np.float16)
        v = x_fn(r, (L, hkv, D)) if x_fn else (r.standard_normal((L, hkv, D)) * 2).astype(np.float16)
        oracle.kv_quant_append_cfg(k, v, np.full(L, b, np.int32), np.arange(L, dtype=np.int32), pt, kp, vp, cfg, P)
        ks.append(k)
        vs.append(v)
    q = (r.standard_normal((B, hq, D))).astype(np.float16)
    return kp, vp, pt, np.array(lens, np.int32), q, ks, vs


def _softmax_attention(q, K, V, scale):
    z = scale * (K @ q)
    w = scipy.special.softmax(z)
    return w @ V


@pytest.mark.parametrize("cfg_args", [(oracle.FMT_INT4, 32, 32, 0, 0), (oracle.FMT_INT4, 64, 64, 1, 0x5A5A5A5A),
                                      (oracle.FMT_MXFP4, 0, 32, 0, 0),
                                      (oracle.FMT_MXFP4, 128, 32, 0, (1 << 127) | 0xF0F0F)])
def test_variant_decode_equals_softmax_over_readback(cfg_args):
    """Decode over a variant's cache = softmax attention (scipy) over the
    stored bytes read back independently and brought back to the original
    basis with S R (numpy), per query head and its KV head (q / 4)."""
    cfg = oracle.qcfg(*cfg_args)
    P, hkv, hq = 16, 2, 8
    lens = [1, 40, 77]
    kp, vp, pt, cl, q, _, _ = _pool_case(cfg, lens, P, hkv, hq, seed=21)
    scale = 1 / math.sqrt(D)
    out = oracle.paged_decode_attn_cfg(q, kp, vp, pt, cl, hkv, P, cfg, scale)
    tb = oracle.tile_bytes_cfg(D, P, cfg)
    nsb = oracle.scale_bytes_per_vector(cfg)
    T = _rot(cfg.had_block) @ np.diag(_signs(int.from_bytes(bytes(cfg.sign_mask), "little")))   # R S
    for b, L in enumerate(lens):
        for h in range(hkv):
            K = np.zeros((L, D))
            V = np.zeros((L, D))
            for j in range(L):
                for pool, dst in ((kp, K), (vp, V)):
                    pg = pool[pt[b, j // P]].reshape(-1)
                    slot = j % P
                    c0 = (h * P + slot) * 64
                    s0 = hkv * P * 64 + (h * P + slot) * nsb
                    dst[j] = T.T @ _readback(pg[c0:c0 + 64], pg[s0:s0 + nsb], cfg)
            for g in range(hq // hkv):
                qh = h * (hq // hkv) + g
                want = _softmax_attention(q[b, qh].astype(np.float64), K, V, scale)
                assert np.max(np.abs(out[b, qh] - want)) < 1e-5
    assert tb == P * 64 + P * nsb


@pytest.mark.parametrize("fmt", [oracle.FMT_INT4, oracle.FMT_MXFP4])
def test_variant_decode_on_exactly_representable_cache_is_dense_attention(fmt):
    """Keys and values the variant stores exactly (INT4: x = S R y with
    integer codes y of absmax 7 per block of 64; MXFP4 without rotation: x =
    S y with y on the E2M1 grid and absmax 6 per group of 32), so decoding
    over the cache is dense softmax attention over the original fp16 K/V: the
    query rotated with R S and the output brought back with S R."""
    mask = 0x0123456789ABCDEF0FEDCBA987654321
    S = _signs(mask)
    if fmt == oracle.FMT_INT4:
        cfg = oracle.qcfg(fmt, 64, 64, 0, mask)
        H = _rot(64)

        def x_fn(r, shape):
            y = r.integers(-7, 8, size=shape).astype(np.float64)
            y[..., 0] = 7
            y[..., 64] = -7
            return (S * (y @ H.T)).astype(np.float16)
    else:
        cfg = oracle.qcfg(fmt, 0, 32, 0, mask)

        def x_fn(r, shape):
            y = E2M1[r.integers(0, 8, size=shape)] * np.where(r.random(shape) < 0.5, -1, 1)
            y[..., ::32] = 6.0
            return (S * y * 0.25).astype(np.float16)
    lens = [5, 64, 33]
    kp, vp, pt, cl, q, ks, vs = _pool_case(cfg, lens, 16, 2, 8, seed=33, x_fn=x_fn)
    scale = 1 / math.sqrt(D)
    out = oracle.paged_decode_attn_cfg(q, kp, vp, pt, cl, 2, 16, cfg, scale)
    for b in range(len(lens)):
        want = oracle.dense_decode_f64(q[b].astype(np.float64), ks[b].astype(np.float64),
                                       vs[b].astype(np.float64), scale)
        assert np.max(np.abs(out[b] - want)) < 1e-5

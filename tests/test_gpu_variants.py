"""GPU parity of the quantizer variants (kv_quant_append_cfg,
paged_decode_attn_cfg) with the oracle: per-group INT4 scales (with and
without scale search), the randomized Hadamard sign mask, and MXFP4.  Pools
are canary-filled and compared whole, byte for byte; attention within 2e-3
of the fp64 oracle on the same cache."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_kv_cache_quant_amd as kvq
import oracle
import workloads as wl
from gpu_util import ATOL, canary, say

pytestmark = pytest.mark.gpu
D = wl.HEAD_DIM
MASK = 0x9E3779B97F4A7C15F39CC0605CEDC834   # a fixed 128-bit sign mask

# (format, had_block, scale_group, scale_search, sign_mask)
APPEND_CFGS = [
    (0, 32, 32, 0, 0), (0, 64, 64, 0, 0), (0, 128, 32, 0, 0), (0, 0, 32, 0, 0), (0, 0, 64, 0, MASK),
    (0, 32, 32, 1, 0), (0, 64, 64, 1, MASK), (0, 128, 128, 1, 0), (0, 0, 32, 1, 0),
    (0, 32, 128, 0, MASK), (0, 64, 128, 0, MASK), (0, 128, 128, 0, MASK), (0, 0, 128, 0, MASK),
    (1, 0, 32, 0, 0), (1, 32, 32, 0, 0), (1, 64, 32, 0, MASK), (1, 128, 32, 0, 0),
]


def _ids(c):
    f, bh, g, s, m = c
    return f"{'mx' if f else 'int4'}-bh{bh}-g{g}{'-search' if s else ''}{'-signs' if m else ''}"


def _pools(w, cfg, dev, seed):
    tb = kvq.page_tile_bytes_cfg(D, w.page_size, kvq.quant_config(*cfg))
    assert tb == oracle.tile_bytes_cfg(D, w.page_size, oracle.qcfg(*cfg))
    shape = (w.num_pages, w.num_kv_heads, tb)
    return canary(shape, 500 + seed, dev), canary(shape, 600 + seed, dev)


def _special_rows(L, hkv, seed):
    """Rows that exercise the edges: zero vectors, tiny values (subnormal
    fp16 scales), large values, exact ties of the code grids, single spikes."""
    r = np.random.default_rng(seed)
    k = (r.standard_normal((L, hkv, D)) * 2).astype(np.float32)
    k[0] = 0
    k[1] *= 1e-5
    k[2] *= 300
    k[3] = r.integers(-28, 29, size=(hkv, D)) / 4.0           # quarter steps: many exact ties
    k[4] = 0
    k[4, :, 7] = 5.0                                          # one spike per vector
    k[5, :, :32] = 0                                          # an all-zero group
    k[6] = np.where(r.random((hkv, D)) < 0.5, -0.0, 0.0)      # signed zeros
    return k.astype(np.float16)


def _build(cfg, w, dev, seed, special=False):
    ocfg, gcfg = oracle.qcfg(*cfg), kvq.quant_config(*cfg)
    kp, vp = _pools(w, cfg, dev, seed)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    pt = w.table(0)
    pt_d = torch.as_tensor(pt, device=dev)
    for b in range(w.batch):
        L = int(w.prefill_lens[b])
        if L <= 0:
            continue
        k, v = w.rows(0, b, 0, L, dev)
        if special and b == 0 and L >= 8:
            sk = _special_rows(L, w.num_kv_heads, seed)
            k = torch.as_tensor(sk, device=dev)
            v = torch.as_tensor(sk[::-1].copy(), device=dev)
        seq = torch.full((L,), b, dtype=torch.int32, device=dev)
        pos = torch.arange(L, dtype=torch.int32, device=dev)
        kvq.kv_quant_append_cfg(k, v, seq, pos, pt_d, kp, vp, w.page_size, gcfg)
        oracle.kv_quant_append_cfg(k.cpu().numpy(), v.cpu().numpy(), seq.cpu().numpy(), pos.cpu().numpy(), pt,
                                   hk, hv, ocfg, w.page_size)
    torch.cuda.synchronize()
    return kp, vp, hk, hv


@pytest.mark.parametrize("cfg", APPEND_CFGS, ids=_ids)
@pytest.mark.parametrize("page_size", [16, 32])
def test_variant_append_bit_exact(dev, cfg, page_size):
    lens = [130, 1, 0, 77, 64]
    w = wl.small(len(lens), lens, cfg[1], page_size, cfg_id=400 + page_size)
    say(f"variant append {_ids(cfg)} P={page_size}")
    kp, vp, hk, hv = _build(cfg, w, dev, seed=cfg[1] + cfg[2] + page_size, special=True)
    assert np.array_equal(kp.cpu().numpy(), hk), "K pool differs from the oracle's"
    assert np.array_equal(vp.cpu().numpy(), hv), "V pool differs from the oracle's"


@pytest.mark.parametrize("cfg", [(0, 32, 32, 0, 0), (0, 128, 32, 1, MASK), (1, 64, 32, 0, 0)], ids=_ids)
@pytest.mark.parametrize("hkv", [1, 3, 6])
def test_variant_append_rows_over_kv_head_counts(dev, cfg, hkv):
    """Every token in one shuffled call, for 1, 3 and 6 KV heads, with a
    ragged last block of tokens: whole pools against the oracle."""
    lens = [45, 64, 2]
    w = wl.small(len(lens), lens, cfg[1], 16, cfg_id=430 + hkv, num_kv_heads=hkv, num_q_heads=4 * hkv)
    kp, vp = _pools(w, cfg, dev, hkv)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    seq = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(lens)])
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in lens])
    order = np.random.default_rng(7 + hkv).permutation(seq.size)
    seq, pos = seq[order], pos[order]
    k = _special_rows(seq.size, hkv, 50 + hkv)
    v = np.ascontiguousarray(k[::-1])
    say(f"variant append {_ids(cfg)} Hkv={hkv}")
    kvq.kv_quant_append_cfg(torch.as_tensor(k, device=dev), torch.as_tensor(v, device=dev),
                            torch.as_tensor(seq, device=dev), torch.as_tensor(pos, device=dev),
                            torch.as_tensor(w.table(0), device=dev), kp, vp, 16, kvq.quant_config(*cfg))
    torch.cuda.synchronize()
    oracle.kv_quant_append_cfg(k, v, seq, pos, w.table(0), hk, hv, oracle.qcfg(*cfg), 16)
    assert np.array_equal(kp.cpu().numpy(), hk), "K pool differs from the oracle's"
    assert np.array_equal(vp.cpu().numpy(), hv), "V pool differs from the oracle's"


def test_token_wise_config_is_the_plain_append(dev):
    """{INT4, Bh, 128, no search, no signs} through the variant entry point
    writes exactly what kv_quant_append writes."""
    lens = [200, 33]
    w = wl.small(len(lens), lens, 64, 16, cfg_id=420)
    kp1, vp1 = _pools(w, (0, 64, 128, 0, 0), dev, 1)
    kp2, vp2 = kp1.clone(), vp1.clone()
    pt_d = torch.as_tensor(w.table(0), device=dev)
    for b in range(w.batch):
        L = int(w.prefill_lens[b])
        k, v = w.rows(0, b, 0, L, dev)
        seq = torch.full((L,), b, dtype=torch.int32, device=dev)
        pos = torch.arange(L, dtype=torch.int32, device=dev)
        kvq.kv_quant_append(k, v, seq, pos, pt_d, kp1, vp1, 16, 64)
        kvq.kv_quant_append_cfg(k, v, seq, pos, pt_d, kp2, vp2, 16, kvq.quant_config(0, 64, 128, 0, 0))
    torch.cuda.synchronize()
    assert torch.equal(kp1, kp2) and torch.equal(vp1, vp2)


DECODE_CFGS = [
    (0, 32, 32, 0, 0), (0, 64, 64, 0, 0), (0, 128, 32, 0, 0), (0, 0, 32, 0, 0), (0, 32, 32, 1, MASK),
    (0, 64, 128, 0, MASK), (0, 0, 128, 0, MASK), (0, 128, 128, 1, MASK),
    (1, 0, 32, 0, 0), (1, 32, 32, 0, 0), (1, 128, 32, 0, MASK),
]


@pytest.mark.parametrize("cfg", DECODE_CFGS, ids=_ids)
@pytest.mark.parametrize("sched", ["split", "balanced"])
def test_variant_decode_against_oracle(dev, cfg, sched):
    """Ragged lengths (empty, one token, page and chunk tails); 5 sequences
    run the per-sequence split schedule, 21 the batch-wide one.  Page size
    16 for the split case, 32 for the batch-wide one."""
    if sched == "split":
        lens, P = [0, 1, 300, 65, 129], 16
    else:
        r = np.random.default_rng(31)
        lens, P = [int(x) for x in r.integers(0, 350, size=21)], 32
        lens[3] = 0
        lens[4] = 1
    w = wl.small(len(lens), lens, cfg[1], P, cfg_id=430 + P)
    say(f"variant decode {_ids(cfg)} {sched} B={w.batch} P={P}")
    kp, vp, hk, hv = _build(cfg, w, dev, seed=7)
    assert np.array_equal(kp.cpu().numpy(), hk) and np.array_equal(vp.cpu().numpy(), hv)
    q = w.query(0, dev)
    maxctx = int(max(lens))
    out = kvq.paged_decode_attn_cfg(q, kp, vp, torch.as_tensor(w.table(0), device=dev),
                                    torch.as_tensor(w.context_lens, device=dev), w.num_kv_heads, P,
                                    kvq.quant_config(*cfg), w.softmax_scale, maxctx)
    torch.cuda.synchronize()
    want = oracle.paged_decode_attn_cfg(q.cpu().numpy(), hk, hv, w.table(0), w.context_lens, w.num_kv_heads, P,
                                        oracle.qcfg(*cfg), w.softmax_scale)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    say(f"  max-abs error {err:.3e}")
    assert err <= ATOL
    assert np.all(got[lens.index(0)] == 0)


@pytest.mark.parametrize("cfg", [(0, 64, 32, 0, MASK), (1, 32, 32, 0, 0)], ids=_ids)
@pytest.mark.parametrize("group,lens", [(3, [0, 1, 300, 65, 129]), (6, [int(x) for x in np.random.default_rng(37).integers(0, 300, 19)])])
def test_variant_decode_odd_groups(dev, cfg, group, lens):
    """GQA groups that are not a power of two and leave the last head chunk
    of each KV head partly filled (6 = 4 + 2), in both schedules (5
    sequences: per-sequence splits; 19: batch-wide ranges)."""
    hkv = 8 if group == 3 else 2
    w = wl.small(len(lens), lens, cfg[1], 16, cfg_id=470 + group, num_kv_heads=hkv, num_q_heads=hkv * group)
    say(f"variant decode {_ids(cfg)} group {group} B={w.batch}")
    kp, vp, hk, hv = _build(cfg, w, dev, seed=11)
    assert np.array_equal(kp.cpu().numpy(), hk) and np.array_equal(vp.cpu().numpy(), hv)
    q = w.query(0, dev)
    out = kvq.paged_decode_attn_cfg(q, kp, vp, torch.as_tensor(w.table(0), device=dev),
                                    torch.as_tensor(w.context_lens, device=dev), w.num_kv_heads, 16,
                                    kvq.quant_config(*cfg), w.softmax_scale, int(max(lens)))
    torch.cuda.synchronize()
    want = oracle.paged_decode_attn_cfg(q.cpu().numpy(), hk, hv, w.table(0), w.context_lens, w.num_kv_heads, 16,
                                        oracle.qcfg(*cfg), w.softmax_scale)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    say(f"  max-abs error {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("cfg", [(0, 32, 32, 1, MASK), (1, 128, 32, 0, MASK)], ids=_ids)
@pytest.mark.parametrize("mult", [4.0])
def test_variant_decode_sharp_softmax(dev, cfg, mult):
    """Four times the softmax scale (a few keys carry most of the weight):
    the per-group score sums keep the 2e-3 bar."""
    lens = [300, 150, 40]
    w = wl.small(len(lens), lens, cfg[1], 16, cfg_id=440)
    kp, vp, hk, hv = _build(cfg, w, dev, seed=9)
    q = w.query(0, dev)
    scale = float(np.float32(mult * w.softmax_scale))
    out = kvq.paged_decode_attn_cfg(q, kp, vp, torch.as_tensor(w.table(0), device=dev),
                                    torch.as_tensor(w.context_lens, device=dev), w.num_kv_heads, 16,
                                    kvq.quant_config(*cfg), scale, 300)
    torch.cuda.synchronize()
    want = oracle.paged_decode_attn_cfg(q.cpu().numpy(), hk, hv, w.table(0), w.context_lens, w.num_kv_heads, 16,
                                        oracle.qcfg(*cfg), scale)
    err = float(np.max(np.abs(out.cpu().numpy() - want)))
    say(f"variant decode {_ids(cfg)} at {mult}x scale: max-abs {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("cfg", [(1, 32, 32, 0, 0), (1, 128, 32, 0, MASK)], ids=_ids)
@pytest.mark.parametrize("sched", ["split", "balanced"])
def test_mxfp4_decode_reads_negative_zero_as_zero(dev, cfg, sched):
    """E2M1 has two zeros; the append stores +0 only, but a cache may hold
    -0 (code 8).  Every +0 code of the written code rows rewritten as -0
    leaves the decode's output unchanged bit for bit (keys through the scaled
    FP4 instruction, values through the sign-mask byte conversion), and the
    oracle over the rewritten cache agrees."""
    lens = [300, 77, 5] if sched == "split" else [int(x) for x in np.random.default_rng(44).integers(1, 300, 20)]
    w = wl.small(len(lens), lens, cfg[1], 16, cfg_id=445)
    kp, vp, hk, hv = _build(cfg, w, dev, seed=45)
    q = w.query(0, dev)
    pt = torch.as_tensor(w.table(0), device=dev)
    cl = torch.as_tensor(w.context_lens, device=dev)
    gcfg = kvq.quant_config(*cfg)

    def decode(k_pool, v_pool):
        o = kvq.paged_decode_attn_cfg(q, k_pool, v_pool, pt, cl, w.num_kv_heads, 16, gcfg, w.softmax_scale,
                                      int(max(lens)))
        torch.cuda.synchronize()
        return o.clone()
    before = decode(kp, vp)
    ncode = w.num_kv_heads * 16 * (D // 2)   # code rows of every head come first in a page

    def negative_zeros(pool):
        flat = pool.reshape(pool.shape[0], -1).copy()
        c = flat[:, :ncode]
        lo, hi = c & 0x0F, c >> 4
        flat[:, :ncode] = (np.where(hi == 0, 8, hi) << 4) | np.where(lo == 0, 8, lo)
        return flat.reshape(pool.shape)
    hk2, hv2 = negative_zeros(hk), negative_zeros(hv)
    assert np.count_nonzero(hk2 != hk) > 0 and np.count_nonzero(hv2 != hv) > 0
    say(f"MXFP4 decode over -0 codes {_ids(cfg)} {sched}: {np.count_nonzero(hv2 != hv)} value bytes rewritten")
    after = decode(torch.as_tensor(hk2, device=dev), torch.as_tensor(hv2, device=dev))
    assert torch.equal(after, before)
    want = oracle.paged_decode_attn_cfg(q.cpu().numpy(), hk2, hv2, w.table(0), w.context_lens, w.num_kv_heads, 16,
                                        oracle.qcfg(*cfg), w.softmax_scale)
    assert float(np.max(np.abs(after.cpu().numpy() - want))) <= ATOL

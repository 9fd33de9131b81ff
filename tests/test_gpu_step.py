"""GPU parity of paged_decode_step_int4 (the fused decode step: each
sequence's new token is appended and attention runs over the context that
ends with it) with the oracle's two steps, kv_quant_append of the new tokens
then the fp64 decode: the whole pools byte for byte (canary-filled, so a
stray write shows) and every output row within 2e-3."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import bit_kv_cache_quant_amd as kvq
import oracle
import workloads as wl
from gpu_util import ATOL, int4_pools, prefill, prefill_batched, say

pytestmark = pytest.mark.gpu
D = wl.HEAD_DIM


def _step_case(dev, lens, bh, P, cfg_id, pages_per_split=0, hkv=8, hq=32, scale_mult=1.0, batched=False):
    """Cache positions 0 .. L_b - 2 of every sequence (GPU and oracle), then
    the fused step on the GPU against the oracle's append + decode."""
    lens = np.asarray(lens, np.int32)
    w = wl.small(len(lens), lens, bh, P, cfg_id, num_kv_heads=hkv, num_q_heads=hq)
    w = dataclasses.replace(w, prefill_lens=np.maximum(lens - 1, 0))
    kp, vp = int4_pools(w, dev, seed=cfg_id)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    say(f"fused step B={w.batch} bh={bh} P={P} pps={pages_per_split} lens[:8]={lens[:8].tolist()}")
    if batched:
        prefill_batched(w, 0, dev, kp, vp, bh, host_pools=(hk, hv))
    else:
        prefill(w, 0, dev, kp, vp, bh, host_pools=(hk, hv))
    assert np.array_equal(kp.cpu().numpy(), hk) and np.array_equal(vp.cpu().numpy(), hv)
    k_new = torch.zeros((w.batch, hkv, D), dtype=torch.float16)
    v_new = torch.zeros_like(k_new)
    live = [b for b in range(w.batch) if lens[b] > 0]
    if batched:   # seeded N(0, 1) rows from one generator
        g = torch.Generator()
        g.manual_seed(0x5EED1000 + cfg_id)
        k_new = torch.randn((w.batch, hkv, D), generator=g).to(torch.float16)
        v_new = torch.randn((w.batch, hkv, D), generator=g).to(torch.float16)
    else:
        for b in live:
            k, v = w.rows(0, b, int(lens[b]) - 1, 1)
            k_new[b], v_new[b] = k[0], v[0]
    pt = w.table(0)
    if live:
        sel = np.asarray(live)
        oracle.kv_quant_append(k_new.numpy()[sel], v_new.numpy()[sel], sel.astype(np.int32),
                               (lens[sel] - 1).astype(np.int32), pt, hk, hv, bh, P)
    q = w.query(0, dev)
    scale = w.softmax_scale * scale_mult
    maxctx = int(max(lens.max(), 0))
    out = kvq.paged_decode_step_int4(q, k_new.to(dev), v_new.to(dev), kp, vp, torch.as_tensor(pt, device=dev),
                                     torch.as_tensor(lens, device=dev), hkv, P, bh, scale, maxctx,
                                     pages_per_split=pages_per_split)
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), hk), "K pool differs from the oracle's append"
    assert np.array_equal(vp.cpu().numpy(), hv), "V pool differs from the oracle's append"
    want = oracle.paged_decode_attn_int4(q.cpu().numpy(), hk, hv, pt, lens, hkv, P, bh, scale)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got.astype(np.float64) - want))) if got.size else 0.0
    say(f"  max-abs error {err:.3e}")
    assert err <= ATOL
    for b in range(w.batch):
        if lens[b] <= 0:
            assert np.all(got[b] == 0), "a sequence with no context gets a zero row"
    return got


@pytest.mark.parametrize("page_size", [16, 32])
@pytest.mark.parametrize("had_block", [0, 32, 64, 128])
def test_step_ragged_split_mode(dev, had_block, page_size):
    """Fewer than 16 sequences (per-sequence ranges); lengths 0 (no new
    token), 1 (the new token alone), page and chunk boundaries."""
    lens = [0, 1, 2, 15, 16, 17, 63, 64, 65, 100, 333, 5]
    _step_case(dev, lens, had_block, page_size, cfg_id=300 + had_block + page_size)


@pytest.mark.parametrize("bh,P,pps", [(64, 16, 0), (64, 16, 3), (128, 32, 0), (0, 16, 1), (32, 32, 2)])
def test_step_balanced_mode(dev, bh, P, pps):
    """37 ragged sequences (batch-wide balanced ranges, which may cross
    sequences), some empty and some holding only the new token."""
    r = np.random.default_rng(7 + bh + P + pps)
    lens = [int(x) for x in r.integers(0, 300, size=37)]
    lens[2], lens[3], lens[11], lens[30] = 0, 1, 1, 0
    _step_case(dev, lens, bh, P, cfg_id=340 + bh + P + pps, pages_per_split=pps)


@pytest.mark.parametrize("lens,pps", [([20000], 4), ([3000, 2500], 4), ([1000], 4), ([1], 0), ([4097, 0, 1], 2)])
def test_step_many_ranges(dev, lens, pps):
    """Many ranges per sequence, so the merge shares a unit's partial states
    among 4 or 16 waves and folds the new token after their LDS merge."""
    _step_case(dev, lens, 128, 16, cfg_id=380 + len(lens) + pps, pages_per_split=pps)


@pytest.mark.parametrize("group", [1, 2, 3, 6, 8])
def test_step_gqa_groups(dev, group):
    """One writer per KV head whatever the group size."""
    hkv = 2
    _step_case(dev, [50, 200, 17, 1], 64, 16, cfg_id=390 + group, hkv=hkv, hq=hkv * group)


@pytest.mark.parametrize("batch", [15, 16, 4096, 4097])
def test_step_batch_schedule_edges(dev, batch):
    """The fused step at the edges of the decode schedules (15 / 16: split
    and batch-wide ranges; 4096: the largest batch-wide schedule; 4097:
    splits again), with empty and one-token sequences among them."""
    r = np.random.default_rng(600 + batch)
    hi = 300 if batch < 100 else 40
    lens = [int(x) for x in r.integers(0, hi, size=batch)]
    lens[1] = 0
    lens[2] = 1
    _step_case(dev, lens, 64, 16, cfg_id=600 + batch % 89, batched=True)


@pytest.mark.parametrize("mult", [2.0, 4.0])
def test_step_sharper_softmax(dev, mult):
    """2x and 4x the softmax scale: the new token's score, computed apart
    from the cached tokens', must still be consistent with theirs."""
    _step_case(dev, [300, 64, 1, 129], 64, 16, cfg_id=395 + int(mult), scale_mult=mult)


def test_step_matches_two_calls(dev):
    """The fused step and the two separate calls (append, then decode) on
    copies of the same cache: identical pools, outputs within fp32 reordering."""
    lens = np.asarray([700, 1500, 33, 1, 64, 65] * 4, np.int32)
    w = wl.small(len(lens), lens, 128, 16, cfg_id=398)
    w = dataclasses.replace(w, prefill_lens=np.maximum(lens - 1, 0))
    kp, vp = int4_pools(w, dev, seed=398)
    prefill(w, 0, dev, kp, vp, 128)
    kp2, vp2 = kp.clone(), vp.clone()
    k_new = torch.zeros((w.batch, 8, D), dtype=torch.float16)
    v_new = torch.zeros_like(k_new)
    for b in range(w.batch):
        k, v = w.rows(0, b, int(lens[b]) - 1, 1)
        k_new[b], v_new[b] = k[0], v[0]
    k_new, v_new = k_new.to(dev), v_new.to(dev)
    pt = torch.as_tensor(w.table(0), device=dev)
    cl = torch.as_tensor(lens, device=dev)
    q = w.query(0, dev)
    maxctx = int(lens.max())
    fused = kvq.paged_decode_step_int4(q, k_new, v_new, kp, vp, pt, cl, 8, 16, 128, w.softmax_scale, maxctx)
    seq = torch.arange(w.batch, dtype=torch.int32, device=dev)
    kvq.kv_quant_append(k_new, v_new, seq, cl - 1, pt, kp2, vp2, 16, 128)
    two = kvq.paged_decode_attn_int4(q, kp2, vp2, pt, cl, 8, 16, 128, w.softmax_scale, maxctx)
    torch.cuda.synchronize()
    assert torch.equal(kp, kp2) and torch.equal(vp, vp2)
    assert float((fused - two).abs().max()) <= 1e-5 * max(1.0, float(two.abs().max()))

"""GPU parity of paged_decode_attn_int4 / paged_decode_attn_fp16 with the
fp64 oracle: max-abs error <= 2e-3 on the same cache (the GPU cache is first
checked byte-for-byte against the oracle's own cache built from the same
inputs), plus split-count invariance and edge cases."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_kv_cache_quant_amd as kvq
import oracle
import workloads as wl
from gpu_util import ATOL, append_step, fp16_pools, int4_pools, prefill, prefill_batched, say

pytestmark = pytest.mark.gpu
D = wl.HEAD_DIM


def _int4_case(w: wl.Workload, dev, layer=0, had_block=None, pages_per_split=0, check_cache=True):
    bh = w.had_block if had_block is None else had_block
    kp, vp = int4_pools(w, dev)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    say(f"prefill {w.name} layer {layer} bh={bh}")
    prefill(w, layer, dev, kp, vp, bh, host_pools=(hk, hv))
    append_step(w, layer, dev, kp, vp, bh, host_pools=(hk, hv))
    if check_cache:
        assert np.array_equal(kp.cpu().numpy(), hk), "GPU K cache differs from the oracle's"
        assert np.array_equal(vp.cpu().numpy(), hv), "GPU V cache differs from the oracle's"
    q = w.query(layer, dev)
    pt = torch.as_tensor(w.table(layer), device=dev)
    cl = torch.as_tensor(w.context_lens, device=dev)
    maxctx = int(max(w.context_lens.max(), 0))
    say(f"decode {w.name} B={w.batch} maxctx={maxctx} pps={pages_per_split}")
    out = kvq.paged_decode_attn_int4(q, kp, vp, pt, cl, w.num_kv_heads, w.page_size, bh, w.softmax_scale,
                                     maxctx, pages_per_split=pages_per_split)
    torch.cuda.synchronize()
    want = oracle.paged_decode_attn_int4(q.cpu().numpy(), hk, hv, w.table(layer), w.context_lens,
                                         w.num_kv_heads, w.page_size, bh, w.softmax_scale)
    return out.cpu().numpy(), want, (kp, vp, q, pt, cl, maxctx, bh)


def _assert_close(got, want, atol=ATOL):
    err = np.max(np.abs(got.astype(np.float64) - want.astype(np.float64))) if got.size else 0.0
    assert np.all(np.isfinite(got))
    assert err <= atol, f"max-abs error {err:.3e} > {atol}"
    return err


def test_decode_c1(dev):
    w = wl.c1()
    got, want, _ = _int4_case(w, dev)
    _assert_close(got, want)


@pytest.mark.parametrize("page_size", [16, 32])
@pytest.mark.parametrize("had_block", [0, 32, 64, 128])
def test_decode_ragged_lengths(dev, had_block, page_size):
    lens = [0, 1, 15, 16, 17, 100, 333, 64, 5]
    w = wl.small(len(lens), lens, had_block, page_size, cfg_id=60 + had_block + page_size)
    got, want, _ = _int4_case(w, dev)
    _assert_close(got, want)
    assert np.all(got[0] == 0), "a zero-length sequence gives a zero row"


@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 6, 8])
def test_decode_gqa_groups(dev, group):
    lens = [50, 200, 17]
    w = wl.small(len(lens), lens, 64, 16, cfg_id=80 + group, num_kv_heads=2, num_q_heads=2 * group)
    got, want, _ = _int4_case(w, dev)
    _assert_close(got, want)


@pytest.mark.parametrize("pages_per_split,group", [(0, 4), (4, 4), (9, 4), (0, 1), (3, 8), (5, 2), (0, 3), (2, 6)])
def test_decode_ranges_cross_sequences(dev, pages_per_split, group):
    """Many short, ragged sequences (some empty): with batches of 16 or more
    the decode cuts the concatenated chunks of all sequences into equal
    ranges, so a range can end inside one sequence and run on into the next
    ones; small pages_per_split values force ranges of one or two chunks."""
    r = np.random.default_rng(123)
    lens = [int(x) for x in r.integers(0, 260, size=37)]
    lens[3] = 0
    lens[4] = 0
    lens[20] = 1
    hkv = 8 if group <= 4 else 2
    w = wl.small(len(lens), lens, 64, 16, cfg_id=150 + group, num_kv_heads=hkv, num_q_heads=hkv * group)
    got, want, _ = _int4_case(w, dev, pages_per_split=pages_per_split)
    _assert_close(got, want)
    assert np.all(got[3] == 0) and np.all(got[4] == 0)


def test_decode_split_invariance(dev):
    lens = [700, 1500, 33]
    w = wl.small(len(lens), lens, 128, 16, cfg_id=90)
    got, want, (kp, vp, q, pt, cl, maxctx, bh) = _int4_case(w, dev)
    _assert_close(got, want)
    outs = []
    for pps in (1, 3, 7, 64, 200):
        o = kvq.paged_decode_attn_int4(q, kp, vp, pt, cl, w.num_kv_heads, w.page_size, bh, w.softmax_scale,
                                       maxctx, pages_per_split=pps)
        outs.append(o.cpu().numpy())
    # Different splits only reorder fp32 sums: the differences scale with the
    # output's magnitude (|o| reaches ~20 with the x20 outlier channels).
    bound = 1e-5 * max(1.0, float(np.max(np.abs(got))))
    for o in outs:
        assert np.max(np.abs(o - got)) <= bound


def _fp16_case(w: wl.Workload, dev, layer=0, pages_per_split=0, poison=False):
    kp, vp = fp16_pools(w, dev, poison=poison)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    say(f"fp16 prefill {w.name} B={w.batch} P={w.page_size} poison={poison}")
    prefill(w, layer, dev, kp, vp, 0, fp16=True, host_pools=(hk, hv))
    append_step(w, layer, dev, kp, vp, 0, fp16=True, host_pools=(hk, hv))
    assert np.array_equal(kp.cpu().numpy().view(np.uint16), hk.view(np.uint16)), "fp16 K pool differs"
    assert np.array_equal(vp.cpu().numpy().view(np.uint16), hv.view(np.uint16)), "fp16 V pool differs"
    q = w.query(layer, dev)
    pt = torch.as_tensor(w.table(layer), device=dev)
    cl = torch.as_tensor(w.context_lens, device=dev)
    maxctx = int(max(w.context_lens.max(), 0))
    say(f"fp16 decode {w.name} B={w.batch} maxctx={maxctx} pps={pages_per_split}")
    out = kvq.paged_decode_attn_fp16(q, kp, vp, pt, cl, w.num_kv_heads, w.page_size, w.softmax_scale, maxctx,
                                     pages_per_split=pages_per_split)
    torch.cuda.synchronize()
    want = oracle.paged_decode_attn_fp16(q.cpu().numpy(), hk, hv, w.table(layer), w.context_lens,
                                         w.num_kv_heads, w.page_size, w.softmax_scale)
    return out.cpu().numpy(), want


@pytest.mark.parametrize("page_size", [16, 32])
def test_decode_fp16_baseline(dev, page_size):
    """Ragged lengths (empty, one token, tails of every kind) with unwritten
    slots poisoned with NaN keys and infinite values: masked tokens must not
    reach the result."""
    lens = [0, 1, 17, 300, 64, 31, 32, 33, 95]
    w = wl.small(len(lens), lens, 0, page_size, cfg_id=95 + page_size)
    got, want = _fp16_case(w, dev, poison=True)
    _assert_close(got, want)
    assert np.all(got[0] == 0), "a zero-length sequence gives a zero row"


@pytest.mark.parametrize("group", [1, 2, 3, 4, 6, 8])
def test_decode_fp16_gqa_groups(dev, group):
    lens = [50, 200, 17]
    w = wl.small(len(lens), lens, 0, 16, cfg_id=180 + group, num_kv_heads=2, num_q_heads=2 * group)
    got, want = _fp16_case(w, dev)
    _assert_close(got, want)


@pytest.mark.parametrize("pages_per_split,page_size", [(0, 16), (4, 16), (1, 16), (0, 32), (2, 32)])
def test_decode_fp16_ranges_cross_sequences(dev, pages_per_split, page_size):
    """Batches of 16 or more: the fp16 decode uses the INT4 kernel's batch-wide
    ranges, which run from one sequence into the next."""
    r = np.random.default_rng(321)
    lens = [int(x) for x in r.integers(0, 300, size=29)]
    lens[5] = 0
    lens[6] = 1
    w = wl.small(len(lens), lens, 0, page_size, cfg_id=190 + page_size + pages_per_split)
    got, want = _fp16_case(w, dev, pages_per_split=pages_per_split, poison=True)
    _assert_close(got, want)
    assert np.all(got[5] == 0)


def test_decode_fp16_split_invariance(dev):
    lens = [700, 1500, 33]
    w = wl.small(len(lens), lens, 0, 16, cfg_id=93)
    got, want = _fp16_case(w, dev)
    _assert_close(got, want)
    for pps in (1, 3, 7, 200):
        o, _ = _fp16_case(w, dev, pages_per_split=pps)
        bound = 1e-5 * max(1.0, float(np.max(np.abs(got))))
        assert np.max(np.abs(o - got)) <= bound


def test_decode_rotation_off_matches_naive_oracle(dev):
    """had_block = 0 is naive INT4: the same kernels with no rotation."""
    lens = [120, 47]
    w = wl.small(len(lens), lens, 0, 32, cfg_id=97)
    got, want, _ = _int4_case(w, dev, had_block=0)
    _assert_close(got, want)


@pytest.mark.parametrize("had_block", [0, 128])
@pytest.mark.parametrize("pages_per_split", [0, 2])
def test_decode_ranges_cross_sequences_page32(dev, had_block, pages_per_split):
    """The batch-wide ranges with 32-token pages: a 64-token chunk is two
    pages, so a range boundary falls on every other page; ragged lengths
    (empty, one token, half pages, whole chunks) over 21 sequences."""
    r = np.random.default_rng(77)
    lens = [int(x) for x in r.integers(0, 400, size=21)]
    lens[2] = 0
    lens[7] = 1
    lens[9] = 32
    lens[10] = 64
    lens[11] = 33
    w = wl.small(len(lens), lens, had_block, 32, cfg_id=160 + had_block + pages_per_split)
    got, want, _ = _int4_case(w, dev, pages_per_split=pages_per_split)
    _assert_close(got, want)
    assert np.all(got[2] == 0)


@pytest.mark.parametrize("lens", [[100, 300, 50], [int(x) for x in np.random.default_rng(5).integers(0, 300, 20)]])
def test_decode_context_len_above_max_is_clamped(dev, lens):
    """A context length above max_context_len (outside the contract) is read
    as max_context_len: the row is that of the shorter context, and nothing
    outside the buffers is touched.  Here every buffer is sized for the real
    lengths, so the call stays in bounds either way; the rows must equal the
    oracle's at the clamped lengths (split schedule for 3 sequences, the
    batch-wide one for 20)."""
    lens = list(lens)
    lens[1] = 300
    w = wl.small(len(lens), lens, 64, 16, cfg_id=170 + len(lens))
    kp, vp = int4_pools(w, dev)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    prefill(w, 0, dev, kp, vp, w.had_block, host_pools=(hk, hv))
    q = w.query(0, dev)
    maxctx = 200
    out = kvq.paged_decode_attn_int4(q, kp, vp, torch.as_tensor(w.table(0), device=dev),
                                     torch.as_tensor(w.context_lens, device=dev), w.num_kv_heads, w.page_size,
                                     w.had_block, w.softmax_scale, maxctx)
    torch.cuda.synchronize()
    clamped = np.minimum(w.context_lens, maxctx).astype(np.int32)
    want = oracle.paged_decode_attn_int4(q.cpu().numpy(), hk, hv, w.table(0), clamped, w.num_kv_heads,
                                         w.page_size, w.had_block, w.softmax_scale)
    _assert_close(out.cpu().numpy(), want)


@pytest.mark.parametrize("lens,page_size,had_block", [([2100, 700, 1], 16, 128), ([300] * 9, 32, 64),
                                                      ([4096], 16, 0)])
def test_decode_range_shared_by_waves(dev, lens, page_size, had_block, monkeypatch):
    """Split mode with few work items: a page range shared by 1, 2 or 4 waves
    of one block (their partial states merged in LDS) gives the oracle's
    result, and the three agree to fp32 reordering."""
    w = wl.small(len(lens), lens, had_block, page_size, cfg_id=180 + page_size + had_block)
    kp, vp = int4_pools(w, dev)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    prefill(w, 0, dev, kp, vp, had_block, host_pools=(hk, hv))
    q = w.query(0, dev)
    pt = torch.as_tensor(w.table(0), device=dev)
    cl = torch.as_tensor(w.context_lens, device=dev)
    want = oracle.paged_decode_attn_int4(q.cpu().numpy(), hk, hv, w.table(0), w.context_lens, w.num_kv_heads,
                                         page_size, had_block, w.softmax_scale)
    outs = {}
    for wpr in ("1", "2", "4"):
        monkeypatch.setenv("KVQ_RANGE_WAVES", wpr)
        say(f"range waves {wpr}: B={w.batch} P={page_size} bh={had_block}")
        o = kvq.paged_decode_attn_int4(q, kp, vp, pt, cl, w.num_kv_heads, page_size, had_block, w.softmax_scale,
                                       int(max(lens)))
        torch.cuda.synchronize()
        outs[wpr] = o.cpu().numpy()
        _assert_close(outs[wpr], want)
    bound = 1e-5 * max(1.0, float(np.max(np.abs(outs["1"]))))
    assert np.max(np.abs(outs["2"] - outs["1"])) <= bound
    assert np.max(np.abs(outs["4"] - outs["1"])) <= bound



@pytest.mark.parametrize("batch", [15, 16, 4096, 4097])
def test_decode_batch_schedule_edges(dev, batch):
    """Batches at the edges of the decode schedules: 15 (the largest batch
    of per-sequence splits below the batch-wide ranges), 16 (the smallest
    with them), 4096 (the largest: one block scans every context length)
    and 4097 (per-sequence splits again, over a grid of 4097 sequences).
    Every output row is compared."""
    r = np.random.default_rng(500 + batch)
    hi = 300 if batch < 100 else 40
    lens = [int(x) for x in r.integers(0, hi, size=batch)]
    lens[1] = 0
    lens[-1] = hi + 17
    w = wl.small(batch, lens, 64, 16, cfg_id=500 + batch % 97)
    kp, vp = int4_pools(w, dev)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    say(f"schedule edge B={batch}")
    prefill_batched(w, 0, dev, kp, vp, 64, host_pools=(hk, hv))
    assert np.array_equal(kp.cpu().numpy(), hk) and np.array_equal(vp.cpu().numpy(), hv)
    q = w.query(0, dev)
    out = kvq.paged_decode_attn_int4(q, kp, vp, torch.as_tensor(w.table(0), device=dev),
                                     torch.as_tensor(w.context_lens, device=dev), w.num_kv_heads, w.page_size, 64,
                                     w.softmax_scale, int(max(lens)))
    torch.cuda.synchronize()
    want = oracle.paged_decode_attn_int4(q.cpu().numpy(), hk, hv, w.table(0), w.context_lens, w.num_kv_heads,
                                         w.page_size, 64, w.softmax_scale)
    got = out.cpu().numpy()
    _assert_close(got, want)
    assert np.all(got[1] == 0)

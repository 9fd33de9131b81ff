"""Parity at the workloads' full sizes, in the launch configuration the
benchmark uses.  The whole cache is built on the GPU; the oracle rebuilds
the sampled sequences from the same inputs, the GPU tiles of those sequences
are compared byte for byte, and their decode outputs within 2e-3."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_kv_cache_quant_amd as kvq
import oracle
import workloads as wl
from gpu_util import ATOL, append_step, say

pytestmark = pytest.mark.gpu


def _zero_pools(w, dev):
    tb = kvq.page_tile_bytes(wl.HEAD_DIM, w.page_size)
    kp = torch.zeros((w.num_pages, w.num_kv_heads, tb), dtype=torch.uint8, device=dev)
    return kp, torch.zeros_like(kp), np.zeros((w.num_pages, w.num_kv_heads, tb), np.uint8), \
        np.zeros((w.num_pages, w.num_kv_heads, tb), np.uint8)


def _check_sampled(w, dev, layer, bh, sample):
    kp, vp, hk, hv = _zero_pools(w, dev)
    pt = w.table(layer)
    pt_d = torch.as_tensor(pt, device=dev)
    say(f"{w.name} layer {layer} bh {bh}: GPU prefill of {w.batch} sequences")
    for b in range(w.batch):
        L = int(w.prefill_lens[b])
        k, v = w.rows(layer, b, 0, L, dev)
        seq = torch.full((L,), b, dtype=torch.int32, device=dev)
        pos = torch.arange(L, dtype=torch.int32, device=dev)
        kvq.kv_quant_append(k, v, seq, pos, pt_d, kp, vp, w.page_size, bh)
        if b in sample:
            oracle.kv_quant_append(k.cpu().numpy(), v.cpu().numpy(), seq.cpu().numpy(), pos.cpu().numpy(),
                                   pt, hk, hv, bh, w.page_size)
    # the step's own appends (only sampled sequences mirrored on the host)
    if w.append_seq.size:
        k, v = w.append_rows(layer, dev)
        kvq.kv_quant_append(k, v, torch.as_tensor(w.append_seq, device=dev),
                            torch.as_tensor(w.append_pos, device=dev), pt_d, kp, vp, w.page_size, bh)
        m = np.isin(w.append_seq, np.array(sorted(sample)))
        oracle.kv_quant_append(k.cpu().numpy()[m], v.cpu().numpy()[m], w.append_seq[m], w.append_pos[m], pt,
                               hk, hv, bh, w.page_size)
    torch.cuda.synchronize()
    gk, gv = kp.cpu().numpy(), vp.cpu().numpy()
    for b in sample:
        pages = pt[b, :(int(w.context_lens[b]) + w.page_size - 1) // w.page_size]
        assert np.array_equal(gk[pages], hk[pages]), f"K tiles of sequence {b} differ"
        assert np.array_equal(gv[pages], hv[pages]), f"V tiles of sequence {b} differ"
    q = w.query(layer, dev)
    maxctx = int(w.context_lens.max())
    say(f"{w.name}: decode B={w.batch} maxctx={maxctx}")
    out = kvq.paged_decode_attn_int4(q, kp, vp, pt_d, torch.as_tensor(w.context_lens, device=dev),
                                     w.num_kv_heads, w.page_size, bh, w.softmax_scale, maxctx)
    torch.cuda.synchronize()
    idx = np.array(sorted(sample))
    want = oracle.paged_decode_attn_int4(q.cpu().numpy()[idx], hk, hv, pt[idx], w.context_lens[idx],
                                         w.num_kv_heads, w.page_size, bh, w.softmax_scale)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got[idx] - want)))
    say(f"{w.name}: max-abs error {err:.3e} over sequences {list(idx)}")
    assert err <= ATOL
    return got, (hk, hv, pt, idx)


@pytest.mark.parametrize("layer", [0, 35])
def test_c3_layer_full(dev, layer):
    """Batch 1, 32K context, Bh 128: every code byte and every output row."""
    w = wl.c3()
    _check_sampled(w, dev, layer, 128, sample={0})


def test_c4_decode_step_sampled(dev):
    """Batch 256, ctx U[1024, 8192]: append at ctx_b, decode over ctx_b + 1;
    oracle on the shortest, the longest and two seeded sequences."""
    w = wl.c4()
    r = np.random.default_rng(44)
    sample = {int(np.argmin(w.context_lens)), int(np.argmax(w.context_lens))} | set(
        int(x) for x in r.choice(w.batch, 2, replace=False))
    _check_sampled(w, dev, 0, 64, sample)


@pytest.mark.parametrize("bh", [128, 0])
def test_c5_long_context_sampled(dev, bh):
    """Batch 8 x 131,072, P 32, rotation on and off: two sequences checked."""
    w = wl.c5(had_block=bh)
    _check_sampled(w, dev, 0, bh, sample={0, 5})


def test_c4_fp16_decode_sampled(dev):
    """The fp16 baseline on the same batch-256 step: fp16 pools (4.8 GB),
    the balanced launch the benchmark times, the oracle on four sequences."""
    w = wl.c4()
    r = np.random.default_rng(45)
    sample = {int(np.argmin(w.context_lens)), int(np.argmax(w.context_lens))} | set(
        int(x) for x in r.choice(w.batch, 2, replace=False))
    shape = (w.num_pages, w.num_kv_heads, w.page_size, wl.HEAD_DIM)
    kp = torch.zeros(shape, dtype=torch.float16, device=dev)
    vp = torch.zeros_like(kp)
    hk = np.zeros(shape, np.float16)
    hv = np.zeros(shape, np.float16)
    pt = w.table(0)
    pt_d = torch.as_tensor(pt, device=dev)
    say(f"{w.name} fp16: GPU prefill of {w.batch} sequences")
    for b in range(w.batch):
        L = int(w.prefill_lens[b])
        k, v = w.rows(0, b, 0, L, dev)
        seq = torch.full((L,), b, dtype=torch.int32, device=dev)
        pos = torch.arange(L, dtype=torch.int32, device=dev)
        kvq.kv_append_fp16(k, v, seq, pos, pt_d, kp, vp, w.page_size)
        if b in sample:
            oracle.kv_append_fp16(k.cpu().numpy(), v.cpu().numpy(), seq.cpu().numpy(), pos.cpu().numpy(),
                                  pt, hk, hv, w.page_size)
    k, v = w.append_rows(0, dev)
    kvq.kv_append_fp16(k, v, torch.as_tensor(w.append_seq, device=dev), torch.as_tensor(w.append_pos, device=dev),
                       pt_d, kp, vp, w.page_size)
    m = np.isin(w.append_seq, np.array(sorted(sample)))
    oracle.kv_append_fp16(k.cpu().numpy()[m], v.cpu().numpy()[m], w.append_seq[m], w.append_pos[m], pt, hk, hv,
                          w.page_size)
    torch.cuda.synchronize()
    q = w.query(0, dev)
    maxctx = int(w.context_lens.max())
    say(f"{w.name} fp16: decode B={w.batch} maxctx={maxctx}")
    out = kvq.paged_decode_attn_fp16(q, kp, vp, pt_d, torch.as_tensor(w.context_lens, device=dev),
                                     w.num_kv_heads, w.page_size, w.softmax_scale, maxctx)
    torch.cuda.synchronize()
    idx = np.array(sorted(sample))
    gk = kp.cpu().numpy()
    gv = vp.cpu().numpy()
    for b in idx:
        pages = pt[b, :(int(w.context_lens[b]) + w.page_size - 1) // w.page_size]
        assert np.array_equal(gk[pages].view(np.uint16), hk[pages].view(np.uint16)), f"K rows of {b} differ"
        assert np.array_equal(gv[pages].view(np.uint16), hv[pages].view(np.uint16)), f"V rows of {b} differ"
    want = oracle.paged_decode_attn_fp16(q.cpu().numpy()[idx], hk, hv, pt[idx], w.context_lens[idx],
                                         w.num_kv_heads, w.page_size, w.softmax_scale)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got[idx] - want)))
    say(f"{w.name} fp16: max-abs error {err:.3e} over sequences {list(idx)}")
    assert err <= ATOL

"""Parity at the workloads' full sizes, in the launch configuration the
benchmark uses.  The whole cache is built on the GPU, and the oracle builds
the whole cache again on the host from the very same inputs (copied back
from the GPU sequence by sequence); the two pools are compared byte for byte
in full, and every output row of the decode within 2e-3 of the oracle's."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_kv_cache_quant_amd as kvq
import oracle
import workloads as wl
from gpu_util import ATOL, say

pytestmark = pytest.mark.gpu


def _build_both(w, dev, layer, bh, fp16=False, gpu_append=True):
    """GPU pools built through the C ABI and host pools built by the oracle,
    both from zero, from the same rows: every sequence's prefill, then the
    workload's own append step (on the host only, if not gpu_append)."""
    if fp16:
        shape = (w.num_pages, w.num_kv_heads, w.page_size, wl.HEAD_DIM)
        kp = torch.zeros(shape, dtype=torch.float16, device=dev)
        hk, hv = np.zeros(shape, np.float16), np.zeros(shape, np.float16)
    else:
        shape = (w.num_pages, w.num_kv_heads, kvq.page_tile_bytes(wl.HEAD_DIM, w.page_size))
        kp = torch.zeros(shape, dtype=torch.uint8, device=dev)
        hk, hv = np.zeros(shape, np.uint8), np.zeros(shape, np.uint8)
    vp = torch.zeros_like(kp)
    pt = w.table(layer)
    pt_d = torch.as_tensor(pt, device=dev)

    def both(k, v, seq, pos, gpu=True):
        if not gpu:
            oracle.kv_quant_append(k.cpu().numpy(), v.cpu().numpy(), seq.cpu().numpy(), pos.cpu().numpy(), pt,
                                   hk, hv, bh, w.page_size)
        elif fp16:
            kvq.kv_append_fp16(k, v, seq, pos, pt_d, kp, vp, w.page_size)
            oracle.kv_append_fp16(k.cpu().numpy(), v.cpu().numpy(), seq.cpu().numpy(), pos.cpu().numpy(), pt,
                                  hk, hv, w.page_size)
        else:
            kvq.kv_quant_append(k, v, seq, pos, pt_d, kp, vp, w.page_size, bh)
            oracle.kv_quant_append(k.cpu().numpy(), v.cpu().numpy(), seq.cpu().numpy(), pos.cpu().numpy(), pt,
                                   hk, hv, bh, w.page_size)

    say(f"{w.name} layer {layer} bh {bh} fp16={fp16}: prefill of {w.batch} sequences on GPU and oracle")
    for b in range(w.batch):
        L = int(w.prefill_lens[b])
        if L <= 0:
            continue
        k, v = w.rows(layer, b, 0, L, dev)
        both(k, v, torch.full((L,), b, dtype=torch.int32, device=dev),
             torch.arange(L, dtype=torch.int32, device=dev))
    if w.append_seq.size:
        k, v = w.append_rows(layer, dev)
        both(k, v, torch.as_tensor(w.append_seq, device=dev), torch.as_tensor(w.append_pos, device=dev),
             gpu=gpu_append)
    torch.cuda.synchronize()
    return kp, vp, hk, hv, pt, pt_d


def _compare_pools(kp, vp, hk, hv, fp16):
    gk, gv = kp.cpu().numpy(), vp.cpu().numpy()
    if fp16:
        gk, gv, hk, hv = gk.view(np.uint16), gv.view(np.uint16), hk.view(np.uint16), hv.view(np.uint16)
    assert np.array_equal(gk, hk), "GPU K pool differs from the oracle's"
    assert np.array_equal(gv, hv), "GPU V pool differs from the oracle's"


def _check_full(w, dev, layer, bh, fp16=False):
    kp, vp, hk, hv, pt, pt_d = _build_both(w, dev, layer, bh, fp16)
    _compare_pools(kp, vp, hk, hv, fp16)
    q = w.query(layer, dev)
    maxctx = int(w.context_lens.max())
    cl = torch.as_tensor(w.context_lens, device=dev)
    say(f"{w.name}: decode B={w.batch} maxctx={maxctx} fp16={fp16}")
    if fp16:
        out = kvq.paged_decode_attn_fp16(q, kp, vp, pt_d, cl, w.num_kv_heads, w.page_size, w.softmax_scale,
                                         maxctx)
    else:
        out = kvq.paged_decode_attn_int4(q, kp, vp, pt_d, cl, w.num_kv_heads, w.page_size, bh, w.softmax_scale,
                                         maxctx)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del kp, vp
    torch.cuda.empty_cache()
    say(f"{w.name}: oracle decode of all {w.batch} sequences")
    if fp16:
        want = oracle.paged_decode_attn_fp16(q.cpu().numpy(), hk, hv, pt, w.context_lens, w.num_kv_heads,
                                             w.page_size, w.softmax_scale)
    else:
        want = oracle.paged_decode_attn_int4(q.cpu().numpy(), hk, hv, pt, w.context_lens, w.num_kv_heads,
                                             w.page_size, bh, w.softmax_scale)
    assert np.all(np.isfinite(got))
    err_rows = np.max(np.abs(got.astype(np.float64) - want), axis=(1, 2))
    say(f"{w.name}: max-abs error {float(err_rows.max()):.3e} over all {w.batch} sequences "
        f"(worst sequence {int(err_rows.argmax())})")
    assert float(err_rows.max()) <= ATOL
    return got


@pytest.mark.parametrize("layer", [0, 35])
def test_c3_layer_full(dev, layer):
    """Batch 1, 32K context, Bh 128: the whole pool and every output row."""
    _check_full(wl.c3(), dev, layer, 128)


def test_c4_decode_step_full(dev):
    """Batch 256, ctx U[1024, 8192]: append at ctx_b, decode over ctx_b + 1,
    in the batch-wide balanced schedule the benchmark times; all 256
    sequences' tiles and output rows."""
    _check_full(wl.c4(), dev, 0, 64)


def test_c4_fused_step_full(dev):
    """The fused step (paged_decode_step_int4) as the benchmark times it, on
    the batch-256 workload: the GPU pools hold the prefill only, the
    oracle's also the step's append; after the step both pools must match
    byte for byte and all 256 output rows lie within 2e-3."""
    w = wl.c4()
    kp, vp, hk, hv, pt, pt_d = _build_both(w, dev, 0, 64, gpu_append=False)
    assert np.array_equal(w.append_seq, np.arange(w.batch)) and np.array_equal(w.append_pos, w.context_lens - 1)
    k_new, v_new = w.append_rows(0, dev)       # row b: sequence b's new token
    q = w.query(0, dev)
    maxctx = int(w.context_lens.max())
    cl = torch.as_tensor(w.context_lens, device=dev)
    say(f"{w.name}: fused step B={w.batch} maxctx={maxctx}")
    out = kvq.paged_decode_step_int4(q, k_new, v_new, kp, vp, pt_d, cl, w.num_kv_heads, w.page_size, 64,
                                     w.softmax_scale, maxctx)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    _compare_pools(kp, vp, hk, hv, False)
    del kp, vp
    torch.cuda.empty_cache()
    say(f"{w.name}: oracle decode of all {w.batch} sequences")
    want = oracle.paged_decode_attn_int4(q.cpu().numpy(), hk, hv, pt, w.context_lens, w.num_kv_heads,
                                         w.page_size, 64, w.softmax_scale)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got.astype(np.float64) - want)))
    say(f"{w.name}: fused step max-abs error {err:.3e} over all {w.batch} sequences")
    assert err <= ATOL


@pytest.mark.parametrize("bh", [128, 0])
def test_c5_long_context_full(dev, bh):
    """Batch 8 x 131,072, P 32, rotation on and off: all 8 sequences."""
    _check_full(wl.c5(had_block=bh), dev, 0, bh)


def test_c4_fp16_decode_full(dev):
    """The fp16 baseline on the same batch-256 step (fp16 pools, 4.8 GB):
    the whole pool and all 256 output rows."""
    _check_full(wl.c4(), dev, 0, 0, fp16=True)

"""The optional host-side index checks (environment variable KVQ_CHECK=1):
with valid indices the checked calls give exactly the unchecked results; a
page-table entry outside the declared pool, a position past the declared
page table and a context length above max_context_len are rejected with
KVQ_ERR_INVALID_ARG before anything is launched.

Every invalid index here still points into memory the test owns (the pools
are passed as views that declare one page fewer than they hold, the page
table as a view without its last row), so even an unchecked call would stay
inside its buffers."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_kv_cache_quant_amd as kvq
import workloads as wl
from gpu_util import int4_pools, prefill, say

pytestmark = pytest.mark.gpu

LENS = [40, 17, 100]
BH, P = 64, 16


def _setup(dev):
    w = wl.small(len(LENS), LENS, BH, P, cfg_id=610)
    kp, vp = int4_pools(w, dev, seed=61)
    prefill(w, 0, dev, kp, vp, BH)
    q = w.query(0, dev)
    pt = torch.as_tensor(w.table(0), device=dev)
    cl = torch.as_tensor(w.context_lens, device=dev)
    return w, kp, vp, q, pt, cl


def _decode(w, q, kp, vp, pt, cl, maxctx=None):
    out = kvq.paged_decode_attn_int4(q, kp, vp, pt, cl, w.num_kv_heads, P, BH, w.softmax_scale,
                                     int(max(LENS)) if maxctx is None else maxctx)
    torch.cuda.synchronize()
    return out


def test_checked_calls_match_unchecked(dev, monkeypatch):
    w, kp, vp, q, pt, cl = _setup(dev)
    monkeypatch.delenv("KVQ_CHECK", raising=False)
    plain = _decode(w, q, kp, vp, pt, cl).clone()
    k, v = w.rows(0, 2, 0, LENS[2], dev)
    seq = torch.full((LENS[2],), 2, dtype=torch.int32, device=dev)
    pos = torch.arange(LENS[2], dtype=torch.int32, device=dev)
    kp2, vp2 = kp.clone(), vp.clone()
    kvq.kv_quant_append(k, v, seq, pos, pt, kp2, vp2, P, BH)
    monkeypatch.setenv("KVQ_CHECK", "1")
    say("KVQ_CHECK=1: decode and append with valid indices")
    checked = _decode(w, q, kp, vp, pt, cl)
    assert torch.equal(checked, plain)
    kp3, vp3 = kp.clone(), vp.clone()
    kvq.kv_quant_append(k, v, seq, pos, pt, kp3, vp3, P, BH)
    torch.cuda.synchronize()
    assert torch.equal(kp3, kp2) and torch.equal(vp3, vp2)


def test_checked_decode_rejects_page_outside_the_pool(dev, monkeypatch):
    w, kp, vp, q, pt, cl = _setup(dev)
    n = kp.shape[0]
    bad = pt.clone()
    bad[0, 0] = n - 1                       # held by the tensors, beyond the declared n - 1 pages
    monkeypatch.setenv("KVQ_CHECK", "1")
    say("KVQ_CHECK=1: decode with a page-table entry past the declared pool")
    with pytest.raises(kvq.KVQError) as e:
        _decode(w, q, kp[:n - 1], vp[:n - 1], bad, cl)
    assert e.value.status == kvq.KVQ_ERR_INVALID_ARG


def test_checked_decode_rejects_length_above_max(dev, monkeypatch):
    w, kp, vp, q, pt, cl = _setup(dev)
    monkeypatch.setenv("KVQ_CHECK", "1")
    say("KVQ_CHECK=1: decode with a context length above max_context_len")
    with pytest.raises(kvq.KVQError) as e:
        _decode(w, q, kp, vp, pt, cl, maxctx=max(LENS) - 1)   # (the device would clamp it)
    assert e.value.status == kvq.KVQ_ERR_INVALID_ARG


def test_checked_append_rejects_page_outside_the_pool(dev, monkeypatch):
    w, kp, vp, q, pt, cl = _setup(dev)
    n = kp.shape[0]
    bad = pt.clone()
    bad[1, 0] = n - 1
    k, v = w.rows(0, 1, 0, 1, dev)
    one = torch.ones(1, dtype=torch.int32, device=dev)
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    monkeypatch.setenv("KVQ_CHECK", "1")
    say("KVQ_CHECK=1: append into a page past the declared pool")
    with pytest.raises(kvq.KVQError) as e:
        kvq.kv_quant_append(k, v, one, zero, bad, kp[:n - 1], vp[:n - 1], P, BH)
    assert e.value.status == kvq.KVQ_ERR_INVALID_ARG


def test_checked_append_rejects_position_past_the_table(dev, monkeypatch):
    w, kp, vp, q, pt, cl = _setup(dev)
    B, maxp = pt.shape
    # a table with one more row than declared: a position one page past the
    # last sequence's row would read that row's first entry, a real page
    full = torch.cat([pt, torch.zeros((1, maxp), dtype=torch.int32, device=dev)]).contiguous()
    table = full[:B]
    k, v = w.rows(0, B - 1, 0, 1, dev)
    seq = torch.full((1,), B - 1, dtype=torch.int32, device=dev)
    pos = torch.full((1,), maxp * P, dtype=torch.int32, device=dev)
    monkeypatch.setenv("KVQ_CHECK", "1")
    say("KVQ_CHECK=1: append at a position past max_pages_per_seq pages")
    with pytest.raises(kvq.KVQError) as e:
        kvq.kv_quant_append(k, v, seq, pos, table, kp, vp, P, BH)
    assert e.value.status == kvq.KVQ_ERR_INVALID_ARG
    assert table.data_ptr() == full.data_ptr() and np.array_equal(table.cpu().numpy(), pt.cpu().numpy())


def test_checked_prefill(dev, monkeypatch):
    """The prefill under KVQ_CHECK=1: valid indices give the unchecked result
    bit for bit; a page outside the declared pool is rejected."""
    w, kp, vp, q, pt, cl = _setup(dev)
    qlens = [40, 5, 33]
    qs = torch.as_tensor(np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32), device=dev)
    g = torch.Generator(device="cpu")
    g.manual_seed(620)
    qp = torch.randn((int(sum(qlens)), w.num_q_heads, wl.HEAD_DIM), generator=g).to(torch.float16).to(dev)

    def run(kpool, vpool, table):
        out = kvq.paged_prefill_attn_int4(qp, qs, kpool, vpool, table, cl, w.num_kv_heads, P, BH, w.softmax_scale)
        torch.cuda.synchronize()
        return out
    monkeypatch.delenv("KVQ_CHECK", raising=False)
    plain = run(kp, vp, pt).clone()
    monkeypatch.setenv("KVQ_CHECK", "1")
    say("KVQ_CHECK=1: prefill with valid indices, then with a page past the declared pool")
    assert torch.equal(run(kp, vp, pt), plain)
    n = kp.shape[0]
    bad = pt.clone()
    bad[2, 3] = n - 1
    with pytest.raises(kvq.KVQError) as e:
        run(kp[:n - 1], vp[:n - 1], bad)
    assert e.value.status == kvq.KVQ_ERR_INVALID_ARG

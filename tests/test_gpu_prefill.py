"""GPU parity of paged_prefill_attn_int4 (causal prefill attention over the
INT4 cache) with the oracle: query row i of a prompt must equal the decode
oracle at context length position(i) + 1 -- the definition of causal
attention -- within 2e-3, on the same cache (checked byte for byte against
the oracle's own cache first)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_kv_cache_quant_amd as kvq
import oracle
import workloads as wl
from gpu_util import ATOL, int4_pools, prefill, say

pytestmark = pytest.mark.gpu
D = wl.HEAD_DIM


def _queries(nq, hq, seed, dev):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn((nq, hq, D), generator=g).to(torch.float16).to(dev)


def _check(w, dev, qlens, sample=None, scale=None):
    bh = w.had_block
    scale = w.softmax_scale if scale is None else scale
    kp, vp = int4_pools(w, dev)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    say(f"prefill cache {w.name} B={w.batch} bh={bh} P={w.page_size}")
    prefill(w, 0, dev, kp, vp, bh, host_pools=(hk, hv))
    assert np.array_equal(kp.cpu().numpy(), hk), "GPU K cache differs from the oracle's"
    assert np.array_equal(vp.cpu().numpy(), hv), "GPU V cache differs from the oracle's"
    lens = [int(x) for x in w.context_lens]
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    nq = int(qs[-1])
    q = _queries(nq, w.num_q_heads, 1000 + w.cfg_id, dev)
    say(f"prefill attention nq={nq}")
    out = kvq.paged_prefill_attn_int4(q, torch.as_tensor(qs, device=dev), kp, vp,
                                      torch.as_tensor(w.table(0), device=dev),
                                      torch.as_tensor(w.context_lens, device=dev), w.num_kv_heads, w.page_size,
                                      bh, scale)
    torch.cuda.synchronize()
    rows_seq = np.repeat(np.arange(w.batch), qlens)
    rows_pos = np.concatenate([np.arange(L - ql, L) for L, ql in zip(lens, qlens)]).astype(np.int64)
    idx = np.arange(nq) if sample is None else np.array(sorted(sample))
    # one decode per query row: a pseudo-batch with context length position + 1
    want = oracle.paged_decode_attn_int4(q.cpu().numpy()[idx], hk, hv, w.table(0)[rows_seq[idx]],
                                         (rows_pos[idx] + 1).astype(np.int32), w.num_kv_heads, w.page_size, bh,
                                         scale)
    got = out.cpu().numpy()[idx]
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    say(f"prefill max-abs error {err:.3e} over {idx.size} rows")
    assert err <= ATOL
    return out


@pytest.mark.parametrize("bh,P", [(64, 16), (0, 16), (128, 32), (32, 32)])
def test_prefill_whole_prompt(dev, bh, P):
    w = wl.small(1, [200], bh, P, cfg_id=240 + bh + P)
    _check(w, dev, [200])


@pytest.mark.parametrize("bh,P", [(64, 16), (0, 32)])
def test_prefill_ragged_batch_tails_and_empty(dev, bh, P):
    """Several sequences, query counts that are not multiples of the 16-row
    tile, a sequence with no queries and an empty one; queries are each
    sequence's last positions (chunked prefill)."""
    lens = [130, 17, 64, 0, 5, 300]
    qlens = [130, 5, 33, 0, 5, 1]
    w = wl.small(len(lens), lens, bh, P, cfg_id=250 + P)
    _check(w, dev, qlens)


def test_prefill_more_queries_than_context_gives_zero_rows(dev):
    """Out of contract, handled on the device: a sequence claiming more query
    positions than cached tokens gets zero rows (none of its pages is read);
    the other sequences are unaffected."""
    w = wl.small(2, [40, 5], 64, 16, cfg_id=290)
    kp, vp = int4_pools(w, dev)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    prefill(w, 0, dev, kp, vp, w.had_block, host_pools=(hk, hv))
    qlens = [3, 8]
    qs = torch.as_tensor(np.array([0, 3, 11], np.int32), device=dev)
    q = _queries(11, w.num_q_heads, 1000 + w.cfg_id, dev)
    out = kvq.paged_prefill_attn_int4(q, qs, kp, vp, torch.as_tensor(w.table(0), device=dev),
                                      torch.as_tensor(w.context_lens, device=dev), w.num_kv_heads, w.page_size,
                                      w.had_block, w.softmax_scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[3:] == 0.0)
    want = oracle.paged_decode_attn_int4(q.cpu().numpy()[:3], hk, hv, np.repeat(w.table(0)[:1], 3, axis=0),
                                         np.array([38, 39, 40], np.int32), w.num_kv_heads, w.page_size,
                                         w.had_block, w.softmax_scale)
    assert float(np.max(np.abs(got[:3] - want))) <= ATOL


def test_prefill_graph_replay(dev):
    """The prefill call enqueues one kernel and allocates nothing, so it can
    be captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, gives the eager result bit for bit."""
    w = wl.small(2, [200, 77], 64, 16, cfg_id=280)
    kp, vp = int4_pools(w, dev)
    prefill(w, 0, dev, kp, vp, w.had_block)
    qlens = [200, 20]
    qs = torch.as_tensor(np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32), device=dev)
    q = _queries(int(sum(qlens)), w.num_q_heads, 1000 + w.cfg_id, dev)
    pt = torch.as_tensor(w.table(0), device=dev)
    cl = torch.as_tensor(w.context_lens, device=dev)
    out = torch.empty((int(sum(qlens)), w.num_q_heads, D), dtype=torch.float32, device=dev)
    call = lambda: kvq.paged_prefill_attn_int4(q, qs, kp, vp, pt, cl, w.num_kv_heads, w.page_size, w.had_block,
                                               w.softmax_scale, out=out)
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        call()
        torch.cuda.synchronize()
    say("prefill graph: 3 replays equal to the eager call")


@pytest.mark.parametrize("group", [1, 2, 3, 6, 8])
def test_prefill_gqa_groups(dev, group):
    lens = [70, 40]
    w = wl.small(len(lens), lens, 32, 16, cfg_id=260 + group, num_kv_heads=2, num_q_heads=2 * group)
    _check(w, dev, [70, 12])


def test_prefill_32k_prompt_sampled(dev):
    """Batch 1, a 32,768-token prompt (Bh 128, P 16, shuffled pages): every
    position attends causally; the oracle checks rows at tile edges, chunk
    edges and the ends."""
    w = wl.c3(layers=1)
    L = int(w.context_lens[0])
    rows = [0, 1, 15, 16, 17, 63, 64, 65, 1000, 4095, 4096, 16383, 25000, L - 2, L - 1]
    _check(w, dev, [L], sample=rows)

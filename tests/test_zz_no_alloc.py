"""The allocation-free decode (paged_decode_attn_int4_noalloc, static
per-GPU scratch instead of a workspace) against the workspace entry point
(paged_decode_attn_int4) on the same inputs: two calls in a row, the second
with a smaller input, each equal to the workspace call's output bit for bit
(the same kernels and schedule) and within 2e-3 of the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_kv_cache_quant_amd as kvq
import oracle
import workloads as wl
from gpu_util import ATOL, int4_pools, prefill, say

pytestmark = pytest.mark.gpu


def _case(dev, lens, bh, P, cfg_id):
    w = wl.small(len(lens), lens, bh, P, cfg_id=cfg_id)
    kp, vp = int4_pools(w, dev)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    prefill(w, 0, dev, kp, vp, bh, host_pools=(hk, hv))
    return w, kp, vp, hk, hv


def test_noalloc_decode_matches_workspace_decode_on_two_calls(dev):
    r = np.random.default_rng(11)
    big = [int(x) for x in r.integers(0, 900, size=24)]     # batch-wide ranges
    small = [300, 17, 64]                                    # per-sequence splits, fewer partial states
    for step, (lens, bh, P) in enumerate([(big, 64, 16), (small, 128, 32)]):
        w, kp, vp, hk, hv = _case(dev, lens, bh, P, 300 + step)
        q = w.query(0, dev)
        pt = torch.as_tensor(w.table(0), device=dev)
        cl = torch.as_tensor(w.context_lens, device=dev)
        maxctx = int(max(lens))
        assert kvq.workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, maxctx, P) <= kvq.SCRATCH_BYTES
        say(f"no-alloc decode call {step}: B={w.batch} maxctx={maxctx} bh={bh} P={P}")
        out_na = torch.full((w.batch, w.num_q_heads, wl.HEAD_DIM), float("nan"), device=dev)
        kvq.paged_decode_attn_int4_noalloc(q, kp, vp, pt, cl, w.num_kv_heads, P, bh, w.softmax_scale, maxctx,
                                           out=out_na)
        out_ws = kvq.paged_decode_attn_int4(q, kp, vp, pt, cl, w.num_kv_heads, P, bh, w.softmax_scale, maxctx)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws), "the allocation-free call differs from the workspace call"
        want = oracle.paged_decode_attn_int4(q.cpu().numpy(), hk, hv, w.table(0), w.context_lens, w.num_kv_heads,
                                             P, bh, w.softmax_scale)
        err = float(np.max(np.abs(out_na.cpu().numpy() - want)))
        say(f"no-alloc decode call {step}: equal to the workspace call, max-abs vs oracle {err:.3e}")
        assert err <= ATOL


def test_noalloc_decode_rejects_a_request_beyond_the_scratch(dev):
    """Batch 4096 x 8192 context needs 260 MiB of partial states: refused on
    the host with KVQ_ERR_TOO_LARGE, nothing launched."""
    q = torch.zeros((4096, 32, 128), dtype=torch.float16, device=dev)
    pool = torch.zeros((1, 8, 1056), dtype=torch.uint8, device=dev)
    pt = torch.zeros((4096, 512), dtype=torch.int32, device=dev)
    cl = torch.zeros(4096, dtype=torch.int32, device=dev)
    out = torch.zeros((4096, 32, 128), dtype=torch.float32, device=dev)
    with pytest.raises(kvq.KVQError) as e:
        kvq.paged_decode_attn_int4_noalloc(q, pool, pool, pt, cl, 8, 16, 64, 0.088, 8192, out=out)
    assert e.value.status == kvq.KVQ_ERR_TOO_LARGE


def test_noalloc_decode_replays_under_hip_graph(dev):
    """Callers that cannot allocate capture it: a captured call replays to the
    eager output, with eager calls of another shape between replays (they
    overwrite the shared static scratch, which each call fully rewrites
    before reading)."""
    r = np.random.default_rng(12)
    lens = [int(x) for x in r.integers(0, 700, size=20)]    # batch-wide ranges
    w, kp, vp, _, _ = _case(dev, lens, 64, 16, 320)
    w2, kp2, vp2, _, _ = _case(dev, [300, 17, 64], 128, 32, 321)   # per-sequence splits

    def args(wk, k, v):
        return (wk.query(0, dev), k, v, torch.as_tensor(wk.table(0), device=dev),
                torch.as_tensor(wk.context_lens, device=dev), wk.num_kv_heads, wk.page_size, wk.had_block,
                wk.softmax_scale, int(max(wk.context_lens)))

    a1, a2 = args(w, kp, vp), args(w2, kp2, vp2)
    out1 = torch.empty((w.batch, w.num_q_heads, wl.HEAD_DIM), dtype=torch.float32, device=dev)
    out2 = torch.empty((w2.batch, w2.num_q_heads, wl.HEAD_DIM), dtype=torch.float32, device=dev)
    say(f"no-alloc decode under graph capture: B={w.batch}, eager B={w2.batch} between replays")
    kvq.paged_decode_attn_int4_noalloc(*a1, out=out1)
    kvq.paged_decode_attn_int4_noalloc(*a2, out=out2)
    torch.cuda.synchronize()
    eager1, eager2 = out1.clone(), out2.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kvq.paged_decode_attn_int4_noalloc(*a1, out=out1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kvq.paged_decode_attn_int4_noalloc(*a1, out=out1)
    for rep in range(4):
        out1.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out1, eager1), f"replay {rep} differs from the eager call"
        out2.fill_(float("nan"))
        kvq.paged_decode_attn_int4_noalloc(*a2, out=out2)   # eager work on the same scratch
        torch.cuda.synchronize()
        assert torch.equal(out2, eager2), f"the eager call after replay {rep} changed"
    del graph

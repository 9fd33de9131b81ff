"""The hot path under HIP graph capture: the append and the decode calls
enqueue only kernels (no allocation, no host synchronisation, no memset), so
a captured step replays to exactly the eager step's results.  Every replay
is checked, with eager work and synchronisations between replays."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_kv_cache_quant_amd as kvq
import workloads as wl
from gpu_util import fp16_pools, int4_pools, prefill, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lens,fp16", [([300, 17, 1, 0, 129], False),                       # split mode
                                       ([int(x) for x in np.random.default_rng(7).integers(0, 400, 24)], False),
                                       ([int(x) for x in np.random.default_rng(8).integers(0, 400, 24)], True)])
def test_step_replays_under_hip_graph(dev, lens, fp16):
    w = wl.small(len(lens), lens, 0 if fp16 else 64, 16, cfg_id=210 + len(lens) + int(fp16))
    kp, vp = fp16_pools(w, dev) if fp16 else int4_pools(w, dev)
    say(f"graph case B={w.batch} fp16={fp16}")
    prefill(w, 0, dev, kp, vp, w.had_block, fp16=fp16)
    # the step: re-append every sequence's last token (same bytes) + decode
    live = [b for b in range(w.batch) if lens[b] > 0]
    seq = torch.as_tensor(np.array(live, np.int32), device=dev)
    pos = torch.as_tensor(np.array([lens[b] - 1 for b in live], np.int32), device=dev)
    k_new = torch.stack([w.rows(0, b, lens[b] - 1, 1, dev)[0][0] for b in live])
    v_new = torch.stack([w.rows(0, b, lens[b] - 1, 1, dev)[1][0] for b in live])
    pt = torch.as_tensor(w.table(0), device=dev)
    cl = torch.as_tensor(w.context_lens, device=dev)
    q = w.query(0, dev)
    maxctx = int(max(lens))
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, maxctx, w.page_size),
                     dtype=torch.uint8, device=dev)

    def step():
        if fp16:
            kvq.kv_append_fp16(k_new, v_new, seq, pos, pt, kp, vp, w.page_size)
            kvq.paged_decode_attn_fp16(q, kp, vp, pt, cl, w.num_kv_heads, w.page_size, w.softmax_scale, maxctx,
                                       out=out, workspace=ws)
        else:
            kvq.kv_quant_append(k_new, v_new, seq, pos, pt, kp, vp, w.page_size, w.had_block)
            kvq.paged_decode_attn_int4(q, kp, vp, pt, cl, w.num_kv_heads, w.page_size, w.had_block,
                                       w.softmax_scale, maxctx, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    pools = (kp.clone(), vp.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager step"
        assert torch.equal(kp, pools[0]) and torch.equal(vp, pools[1]), f"replay {r} changed other cache bytes"
        step()   # eager work between replays
        torch.cuda.synchronize()
    del graph


@pytest.mark.parametrize("lens", [[300, 17, 1, 0, 129, 2],                                      # split mode
                                  [int(x) for x in np.random.default_rng(9).integers(0, 400, 24)]])  # balanced
def test_fused_step_replays_under_hip_graph(dev, lens):
    """paged_decode_step_int4 captured in a graph: every replay rewrites the
    same new-token bytes and gives the eager output exactly."""
    w = wl.small(len(lens), lens, 128, 16, cfg_id=230 + len(lens))
    kp, vp = int4_pools(w, dev)
    prefill(w, 0, dev, kp, vp, w.had_block)
    k_new = torch.zeros((w.batch, w.num_kv_heads, w.head_dim), dtype=torch.float16, device=dev)
    v_new = torch.zeros_like(k_new)
    for b in range(w.batch):
        if lens[b] > 0:
            k, v = w.rows(0, b, lens[b] - 1, 1, dev)
            k_new[b], v_new[b] = k[0], v[0]
    pt = torch.as_tensor(w.table(0), device=dev)
    cl = torch.as_tensor(w.context_lens, device=dev)
    q = w.query(0, dev)
    maxctx = int(max(lens))
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, maxctx, w.page_size),
                     dtype=torch.uint8, device=dev)

    def step():
        kvq.paged_decode_step_int4(q, k_new, v_new, kp, vp, pt, cl, w.num_kv_heads, w.page_size, w.had_block,
                                   w.softmax_scale, maxctx, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    pools = (kp.clone(), vp.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager step"
        assert torch.equal(kp, pools[0]) and torch.equal(vp, pools[1]), f"replay {r} changed other cache bytes"
        step()
        torch.cuda.synchronize()
    del graph


@pytest.mark.parametrize("cfg", [(0, 32, 32, 1, 0xFFFF0000_00000000_12345678_0F0F0F0F),   # INT4 per block + search
                                 (1, 32, 32, 0, 0)],                                           # MXFP4
                         ids=["int4-g32-search-signs", "mxfp4-bh32"])
@pytest.mark.parametrize("lens", [[300, 17, 1, 0, 129],                                       # split mode
                                  [int(x) for x in np.random.default_rng(11).integers(0, 300, 21)]])  # balanced
def test_variant_step_replays_under_hip_graph(dev, cfg, lens):
    """A quantizer variant's append of each sequence's last token and its
    decode, captured in a graph: every replay rewrites the same bytes and
    gives the eager output exactly."""
    fmt, bh, g, search, mask = cfg
    qc = kvq.quant_config(fmt, bh, g, search, mask)
    w = wl.small(len(lens), lens, bh, 16, cfg_id=240 + len(lens) + fmt)
    tb = kvq.page_tile_bytes_cfg(w.head_dim, w.page_size, qc)
    kp = torch.zeros((w.num_pages, w.num_kv_heads, tb), dtype=torch.uint8, device=dev)
    vp = torch.zeros_like(kp)
    pt = torch.as_tensor(w.table(0), device=dev)
    for b in range(w.batch):
        L = int(lens[b])
        if L <= 1:
            continue
        k, v = w.rows(0, b, 0, L - 1, dev)
        kvq.kv_quant_append_cfg(k, v, torch.full((L - 1,), b, dtype=torch.int32, device=dev),
                                torch.arange(L - 1, dtype=torch.int32, device=dev), pt, kp, vp, w.page_size, qc)
    live = [b for b in range(w.batch) if lens[b] > 0]
    seq = torch.as_tensor(np.array(live, np.int32), device=dev)
    pos = torch.as_tensor(np.array([lens[b] - 1 for b in live], np.int32), device=dev)
    k_new = torch.stack([w.rows(0, b, lens[b] - 1, 1, dev)[0][0] for b in live])
    v_new = torch.stack([w.rows(0, b, lens[b] - 1, 1, dev)[1][0] for b in live])
    cl = torch.as_tensor(w.context_lens, device=dev)
    q = w.query(0, dev)
    maxctx = int(max(lens))
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, maxctx, w.page_size),
                     dtype=torch.uint8, device=dev)
    say(f"variant graph case fmt={fmt} G={g} B={w.batch}")

    def step():
        kvq.kv_quant_append_cfg(k_new, v_new, seq, pos, pt, kp, vp, w.page_size, qc)
        kvq.paged_decode_attn_cfg(q, kp, vp, pt, cl, w.num_kv_heads, w.page_size, qc, w.softmax_scale, maxctx,
                                  out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    pools = (kp.clone(), vp.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager step"
        assert torch.equal(kp, pools[0]) and torch.equal(vp, pools[1]), f"replay {r} changed other cache bytes"
        step()
        torch.cuda.synchronize()
    del graph

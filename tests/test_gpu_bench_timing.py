"""The measurement helpers of bench.py on the device: each returns a positive,
finite GPU time for a small append call and leaves the call's results as an
untimed call leaves them (the cache flush reads another buffer and writes
nothing the call reads)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import bench
import bit_kv_cache_quant_amd as kvq
import workloads as wl
from gpu_util import int4_pools, say

pytestmark = pytest.mark.gpu


def _append_call(dev):
    w = wl.small(4, [40, 17, 64, 3], 64, 16, cfg_id=331)
    kp, vp = int4_pools(w, dev)
    rows = [w.rows(0, b, 0, int(w.context_lens[b]), dev) for b in range(w.batch)]
    k = torch.cat([r[0] for r in rows])
    v = torch.cat([r[1] for r in rows])
    seq = torch.as_tensor(np.repeat(np.arange(w.batch, dtype=np.int32), w.context_lens), device=dev)
    pos = torch.as_tensor(np.concatenate([np.arange(L, dtype=np.int32) for L in w.context_lens]), device=dev)
    pt = torch.as_tensor(w.page_table, device=dev)

    def fn():
        kvq.kv_quant_append(k, v, seq, pos, pt, kp, vp, w.page_size, w.had_block)
    return fn, kp, vp


def test_timing_helpers_give_positive_times_and_keep_results(dev):
    fn, kp, vp = _append_call(dev)
    say("bench timing helpers on a 124-token append")
    fn()
    torch.cuda.synchronize()
    k_ref, v_ref = kp.clone(), vp.clone()
    spent = bench.settle(fn, 1.0)
    mean, median = bench.time_calls(fn, 5, 1)
    cold = bench.time_calls_cold(fn, 3, dev, flush_bytes=64 << 20)
    for t in (spent, mean, median, cold):
        assert math.isfinite(t) and t > 0.0
    assert torch.equal(kp, k_ref) and torch.equal(vp, v_ref)

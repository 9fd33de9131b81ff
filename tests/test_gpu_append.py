"""GPU parity of kv_quant_append / kv_append_fp16 with the oracle: INT4 codes,
scales and placement bit-exact, every other pool byte untouched."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_kv_cache_quant_amd as kvq
import oracle
import workloads as wl
from gpu_util import canary, int4_pools, say

pytestmark = pytest.mark.gpu
D = wl.HEAD_DIM


def _run_append(w: wl.Workload, dev, layer=0, had_block=None, k=None, v=None):
    bh = w.had_block if had_block is None else had_block
    if k is None:
        k, v = w.append_rows(layer, dev)
    kp, vp = int4_pools(w, dev)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    seq = torch.as_tensor(w.append_seq, device=dev)
    pos = torch.as_tensor(w.append_pos, device=dev)
    pt = torch.as_tensor(w.table(layer), device=dev)
    say(f"append {w.name} T={seq.numel()} bh={bh} P={w.page_size}")
    kvq.kv_quant_append(k, v, seq, pos, pt, kp, vp, w.page_size, bh)
    torch.cuda.synchronize()
    oracle.kv_quant_append(k.cpu().numpy(), v.cpu().numpy(), w.append_seq, w.append_pos,
                           w.table(layer), hk, hv, bh, w.page_size)
    return kp.cpu().numpy(), vp.cpu().numpy(), hk, hv


def _assert_pools_equal(got, want, what):
    if not np.array_equal(got, want):
        diff = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
        raise AssertionError(f"{what}: {diff.size} bytes differ, first at flat offsets {diff[:8]}")


def test_append_c1_bit_exact(dev):
    gk, gv, hk, hv = _run_append(wl.c1(), dev)
    _assert_pools_equal(gk, hk, "K pool")
    _assert_pools_equal(gv, hv, "V pool")


def test_append_c2_bit_exact(dev):
    gk, gv, hk, hv = _run_append(wl.c2(), dev)
    _assert_pools_equal(gk, hk, "K pool")
    _assert_pools_equal(gv, hv, "V pool")


def test_append_c2_stream_bit_exact(dev):
    gk, gv, hk, hv = _run_append(wl.c2_stream(), dev)
    _assert_pools_equal(gk, hk, "K pool")
    _assert_pools_equal(gv, hv, "V pool")


def _edge_rows(T, hkv, seed):
    """Rows that exercise every branch of the quantizer: zeros, fp16
    subnormal scales (the clamp), values up to 1024, exact ties under the
    Bh=64 rotation, one-hot channels, outlier channels."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, hkv, D))
    kinds = r.integers(0, 7, size=(T, hkv))
    H64 = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(64)] for i in range(64)])
    for t in range(T):
        for h in range(hkv):
            kd = kinds[t, h]
            if kd == 0:
                x[t, h] = 0
            elif kd == 1:
                x[t, h] = r.integers(-12, 13, D) * 2.0 ** -24          # subnormal range
            elif kd == 2:
                x[t, h] = np.clip(r.standard_normal(D) * 300, -1024, 1024)
            elif kd == 3:
                y = np.clip(r.integers(-14, 15, D) / 2.0, -7, 7)
                y[r.integers(0, D)] = 7.0
                x[t, h] = np.concatenate([H64 @ y[:64], H64 @ y[64:]]) / 8.0
            elif kd == 4:
                x[t, h] = 0
                x[t, h, r.integers(0, D)] = r.choice([-1, 1]) * 2.0 ** r.integers(-20, 10)
            elif kd == 5:
                x[t, h, r.choice(D, 4, replace=False)] *= 20
            else:
                x[t, h] *= 10.0 ** r.uniform(-6, 2)
    return x.astype(np.float16)


@pytest.mark.parametrize("page_size", [16, 32])
@pytest.mark.parametrize("had_block", [0, 32, 64, 128])
def test_append_edge_values_all_block_sizes(dev, had_block, page_size):
    w = wl.small(3, [37, 64, 5], had_block, page_size, cfg_id=40 + page_size + had_block, num_kv_heads=4,
                 num_q_heads=16)
    # every cached token of every sequence appended in one call, in shuffled order
    seq = np.concatenate([np.full(int(n), b, np.int32) for b, n in enumerate(w.context_lens)])
    pos = np.concatenate([np.arange(int(n), dtype=np.int32) for n in w.context_lens])
    order = np.random.default_rng(1).permutation(seq.size)
    w.append_seq, w.append_pos = seq[order], pos[order]
    k = torch.as_tensor(_edge_rows(seq.size, 4, 10 + had_block), device=dev)
    v = torch.as_tensor(_edge_rows(seq.size, 4, 20 + had_block), device=dev)
    gk, gv, hk, hv = _run_append(w, dev, k=k, v=v)
    _assert_pools_equal(gk, hk, "K pool")
    _assert_pools_equal(gv, hv, "V pool")


@pytest.mark.parametrize("hkv,bh", [(1, 128), (2, 64), (3, 32), (5, 128), (6, 0), (7, 64), (12, 32), (16, 128)])
def test_append_rows_over_kv_head_counts(dev, hkv, bh):
    # Every token in one shuffled call, for KV-head counts from 1 to 16
    # (powers of two and not), token counts that leave a ragged last block,
    # and each block size: whole canary-filled pools against the oracle.
    lens = [29, 64, 3, 50]
    w = wl.small(len(lens), lens, bh, 16, cfg_id=90 + hkv, num_kv_heads=hkv, num_q_heads=4 * hkv)
    seq = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(lens)])
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in lens])
    order = np.random.default_rng(hkv).permutation(seq.size)
    w.append_seq, w.append_pos = seq[order], pos[order]
    k = torch.as_tensor(_edge_rows(seq.size, hkv, 30 + hkv), device=dev)
    v = torch.as_tensor(_edge_rows(seq.size, hkv, 40 + hkv), device=dev)
    gk, gv, hk, hv = _run_append(w, dev, k=k, v=v)
    _assert_pools_equal(gk, hk, f"K pool (Hkv {hkv})")
    _assert_pools_equal(gv, hv, f"V pool (Hkv {hkv})")


def test_append_zero_tokens_is_a_noop(dev):
    w = wl.c1()
    kp, vp = int4_pools(w, dev)
    before = kp.clone()
    empty = torch.zeros((0, 8, D), dtype=torch.float16, device=dev)
    none = torch.zeros(0, dtype=torch.int32, device=dev)
    kvq.kv_quant_append(empty, empty, none, none, torch.as_tensor(w.page_table, device=dev), kp, vp, 16, 32)
    torch.cuda.synchronize()
    assert torch.equal(kp, before)


def test_append_fp16_places_rows(dev):
    w = wl.c2()
    k, v = w.append_rows(0, dev)
    shape = (w.num_pages, w.num_kv_heads, w.page_size, D)
    kp = canary(shape, 5, dev, torch.float16)
    vp = canary(shape, 6, dev, torch.float16)
    hk, hv = kp.cpu().numpy(), vp.cpu().numpy()
    say("append_fp16 c2")
    kvq.kv_append_fp16(k, v, torch.as_tensor(w.append_seq, device=dev), torch.as_tensor(w.append_pos, device=dev),
                       torch.as_tensor(w.page_table, device=dev), kp, vp, w.page_size)
    torch.cuda.synchronize()
    oracle.kv_append_fp16(k.cpu().numpy(), v.cpu().numpy(), w.append_seq, w.append_pos, w.page_table, hk, hv,
                          w.page_size)
    _assert_pools_equal(kp.cpu().numpy().view(np.uint16), hk.view(np.uint16), "fp16 K pool")
    _assert_pools_equal(vp.cpu().numpy().view(np.uint16), hv.view(np.uint16), "fp16 V pool")

"""Shared helpers for the GPU parity tests: build the same cache on the GPU
(through the C ABI) and in the oracle (on the host) from the same seeded
inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

import bit_kv_cache_quant_amd as kvq
import oracle
import workloads as wl

ATOL = 2e-3   # decode-attention tolerance, max-abs against the fp64 oracle


def say(msg: str) -> None:
    print(msg, flush=True)


def canary(shape, seed: int, device, dtype=torch.uint8):
    """Random bytes filling a tensor of exactly `shape` and `dtype`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    width = torch.empty((), dtype=dtype).element_size()
    raw_shape = tuple(shape[:-1]) + (shape[-1] * width,)
    x = torch.randint(0, 256, raw_shape, dtype=torch.uint8, device=device, generator=g)
    out = x if dtype == torch.uint8 else x.view(dtype)
    assert tuple(out.shape) == tuple(shape)
    return out


def int4_pools(w: wl.Workload, device, seed: int = 0):
    tb = kvq.page_tile_bytes(wl.HEAD_DIM, w.page_size)
    shape = (w.num_pages, w.num_kv_heads, tb)
    return canary(shape, 100 + seed, device), canary(shape, 200 + seed, device)


def fp16_pools(w: wl.Workload, device, poison: bool = False):
    """fp16 pools, zero, or (poison) every element a NaN / infinity bit
    pattern, so that slots no append writes hold values a decode must never
    let into its result."""
    shape = (w.num_pages, w.num_kv_heads, w.page_size, wl.HEAD_DIM)
    k = torch.zeros(shape, dtype=torch.float16, device=device)
    v = torch.zeros_like(k)
    if poison:
        k.view(torch.int16).fill_(0x7E00)          # quiet NaN
        v.view(torch.int16).fill_(0x7C00)          # +infinity
    return k, v


def prefill(w: wl.Workload, layer: int, device, kp, vp, had_block: int, fp16: bool = False,
            host_pools=None, host_seqs=None):
    """Append every sequence's prefill tokens on the GPU; optionally mirror the
    same appends for the sequences in host_seqs into host (oracle) pools."""
    pt = w.table(layer)
    pt_d = torch.as_tensor(pt, device=device)
    for b in range(w.batch):
        L = int(w.prefill_lens[b])
        if L <= 0:
            continue
        k, v = w.rows(layer, b, 0, L, device)
        seq = torch.full((L,), b, dtype=torch.int32, device=device)
        pos = torch.arange(L, dtype=torch.int32, device=device)
        if fp16:
            kvq.kv_append_fp16(k, v, seq, pos, pt_d, kp, vp, w.page_size)
        else:
            kvq.kv_quant_append(k, v, seq, pos, pt_d, kp, vp, w.page_size, had_block)
        if host_pools is not None and (host_seqs is None or b in host_seqs):
            hk, hv = host_pools
            kk, vv = k.cpu().numpy(), v.cpu().numpy()
            s_, p_ = seq.cpu().numpy(), pos.cpu().numpy()
            if fp16:
                oracle.kv_append_fp16(kk, vv, s_, p_, pt, hk, hv, w.page_size)
            else:
                oracle.kv_quant_append(kk, vv, s_, p_, pt, hk, hv, had_block, w.page_size)
    torch.cuda.synchronize()


def prefill_batched(w: wl.Workload, layer: int, device, kp, vp, had_block: int, host_pools=None, seed: int = 0):
    """prefill() for large batches: every sequence's prefill tokens in one
    INT4 append call (and one oracle call on host_pools).  The rows are
    seeded N(0, 1) fp16 from one generator for the whole batch (the
    per-sequence generators of the workload recipe cost ~15 ms per sequence
    on the host)."""
    lens = np.maximum(np.asarray(w.prefill_lens, np.int64), 0)
    T = int(lens.sum())
    if T == 0:
        return
    g = torch.Generator()
    g.manual_seed(0x5EED0000 + 1009 * w.cfg_id + seed)
    k = torch.randn((T, w.num_kv_heads, w.head_dim), generator=g).to(torch.float16)
    v = torch.randn((T, w.num_kv_heads, w.head_dim), generator=g).to(torch.float16)
    seq = np.repeat(np.arange(w.batch, dtype=np.int32), lens)
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    pt = w.table(layer)
    kvq.kv_quant_append(k.to(device), v.to(device), torch.as_tensor(seq, device=device),
                        torch.as_tensor(pos, device=device), torch.as_tensor(pt, device=device), kp, vp,
                        w.page_size, had_block)
    if host_pools is not None:
        oracle.kv_quant_append(k.numpy(), v.numpy(), seq, pos, pt, host_pools[0], host_pools[1], had_block,
                               w.page_size)
    torch.cuda.synchronize()


def append_step(w: wl.Workload, layer: int, device, kp, vp, had_block: int, fp16: bool = False,
                host_pools=None):
    """The workload's own append (its new tokens), on the GPU and mirrored on
    the host pools when given."""
    T = int(w.append_seq.size)
    if T == 0:
        return
    k, v = w.append_rows(layer, device)
    seq = torch.as_tensor(w.append_seq, device=device)
    pos = torch.as_tensor(w.append_pos, device=device)
    pt = w.table(layer)
    pt_d = torch.as_tensor(pt, device=device)
    if fp16:
        kvq.kv_append_fp16(k, v, seq, pos, pt_d, kp, vp, w.page_size)
    else:
        kvq.kv_quant_append(k, v, seq, pos, pt_d, kp, vp, w.page_size, had_block)
    if host_pools is not None:
        hk, hv = host_pools
        if fp16:
            oracle.kv_append_fp16(k.cpu().numpy(), v.cpu().numpy(), w.append_seq, w.append_pos, pt, hk, hv,
                                  w.page_size)
        else:
            oracle.kv_quant_append(k.cpu().numpy(), v.cpu().numpy(), w.append_seq, w.append_pos, pt, hk, hv,
                                   had_block, w.page_size)
    torch.cuda.synchronize()


def tiles_of(pool_np: np.ndarray, page_table: np.ndarray, b: int, L: int, page_size: int):
    """Physical pages holding the first L tokens of sequence b."""
    n = (L + page_size - 1) // page_size
    return [int(p) for p in page_table[b, :n]]

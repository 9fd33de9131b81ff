"""Seeded synthetic workloads for the INT4 KV-cache hot path.

This module only draws random inputs and builds page tables: it holds none of
the method's arithmetic (no rotation, no quantization, no attention).  Both
the CPU oracle and the HIP library are fed from it, always with the very same
arrays.

Shapes follow a Qwen3-4B-like attention layer: 8 KV heads of dimension 128,
32 query heads (GQA 4:1).  Real activations are not available, so K/V rows
are standard normal with a few fixed "outlier" channels per head scaled up,
the structure that makes naive per-token INT4 lose accuracy.

Recipe (stated once, used everywhere):
  * structure (outlier channels, page permutations, lengths, positions) comes
    from numpy ``Generator(PCG64(SeedSequence([1000 + cfg_id, *key])))``;
  * values come from ``torch.randn`` (float32) on the requested device with a
    ``torch.Generator`` seeded from the same SeedSequence, generated in chunks
    of ``CHUNK`` positions per (layer, sequence, tensor) so that any range of
    positions can be regenerated alone; outlier channels are multiplied, then
    the tensor is rounded to fp16;
  * queries are standard normal fp16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CHUNK = 1024          # positions per value chunk
HEAD_DIM = 128
NUM_KV_HEADS = 8
NUM_Q_HEADS = 32


def _seq(cfg_id: int, *key: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([1000 + cfg_id, *[int(k) for k in key]])


def np_rng(cfg_id: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_seq(cfg_id, *key)))


def torch_seed(cfg_id: int, *key: int) -> int:
    return int(_seq(cfg_id, *key).generate_state(1, np.uint64)[0] & np.uint64(2**62 - 1))


# key tags (first element of every key)
_OUTLIER, _VALUE, _QUERY, _PAGES, _LENS = 1, 2, 3, 4, 5
K_TENSOR, V_TENSOR = 0, 1


@dataclasses.dataclass
class Workload:
    name: str
    cfg_id: int
    batch: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    had_block: int
    page_size: int
    num_pages: int                   # pool size (pages) per layer
    page_table: np.ndarray           # int32 [batch][max_pages_per_seq]
    prefill_lens: np.ndarray         # int32 [batch]: tokens cached before the step
    append_seq: np.ndarray           # int32 [T]: the step's new tokens
    append_pos: np.ndarray           # int32 [T]
    context_lens: np.ndarray         # int32 [batch]: decode length after the append
    layers: int = 1
    k_outliers: int = 4
    k_mult: float = 20.0
    v_outliers: int = 4
    v_mult: float = 20.0
    description: str = ""
    per_layer_page_tables: Optional[list] = None

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    def table(self, layer: int = 0) -> np.ndarray:
        if self.per_layer_page_tables is not None:
            return self.per_layer_page_tables[layer]
        return self.page_table

    # -- values ----------------------------------------------------------
    def outlier_channels(self, layer: int, tensor: int) -> np.ndarray:
        """int64 [Hkv][n] distinct channels per head (empty if none)."""
        n = self.k_outliers if tensor == K_TENSOR else self.v_outliers
        r = np_rng(self.cfg_id, _OUTLIER, layer, tensor)
        out = np.zeros((self.num_kv_heads, n), np.int64)
        for h in range(self.num_kv_heads):
            out[h] = r.choice(self.head_dim, size=n, replace=False)
        return out

    def rows(self, layer: int, seq: int, pos0: int, count: int, device="cpu"):
        """fp16 (K, V) rows for positions [pos0, pos0+count) of one sequence:
        torch tensors [count][Hkv][D] on ``device``."""
        import torch
        res = []
        for tensor in (K_TENSOR, V_TENSOR):
            mult = self.k_mult if tensor == K_TENSOR else self.v_mult
            ch = self.outlier_channels(layer, tensor)
            gain = torch.ones(self.num_kv_heads, self.head_dim, dtype=torch.float32)
            for h in range(self.num_kv_heads):
                gain[h, torch.as_tensor(ch[h])] = float(mult)
            gain = gain.to(device)
            parts = []
            c0, c1 = pos0 // CHUNK, (pos0 + count - 1) // CHUNK if count > 0 else pos0 // CHUNK - 1
            for c in range(c0, c1 + 1):
                g = torch.Generator(device=device)
                g.manual_seed(torch_seed(self.cfg_id, _VALUE, layer, tensor, seq, c))
                vals = torch.randn((CHUNK, self.num_kv_heads, self.head_dim), generator=g,
                                   device=device, dtype=torch.float32)
                lo = max(pos0, c * CHUNK) - c * CHUNK
                hi = min(pos0 + count, (c + 1) * CHUNK) - c * CHUNK
                parts.append(vals[lo:hi])
            if parts:
                x = torch.cat(parts, 0)
            else:
                x = torch.zeros((0, self.num_kv_heads, self.head_dim), device=device)
            res.append((x * gain).to(torch.float16))
        return res[0], res[1]

    def append_rows(self, layer: int = 0, device="cpu"):
        """The step's new tokens (append_seq, append_pos) as fp16 (K, V) [T][Hkv][D]."""
        import torch
        T = int(self.append_seq.size)
        k = torch.empty((T, self.num_kv_heads, self.head_dim), dtype=torch.float16, device=device)
        v = torch.empty_like(k)
        # group consecutive runs of the same sequence with consecutive positions
        i = 0
        while i < T:
            j = i + 1
            while (j < T and self.append_seq[j] == self.append_seq[i]
                   and self.append_pos[j] == self.append_pos[j - 1] + 1):
                j += 1
            kk, vv = self.rows(layer, int(self.append_seq[i]), int(self.append_pos[i]), j - i, device)
            k[i:j], v[i:j] = kk, vv
            i = j
        return k, v

    def query(self, layer: int = 0, device="cpu"):
        import torch
        g = torch.Generator(device=device)
        g.manual_seed(torch_seed(self.cfg_id, _QUERY, layer))
        q = torch.randn((self.batch, self.num_q_heads, self.head_dim), generator=g,
                        device=device, dtype=torch.float32)
        return q.to(torch.float16)


def _identity_table(batch: int, pages_per_seq: int) -> np.ndarray:
    return np.arange(batch * pages_per_seq, dtype=np.int32).reshape(batch, pages_per_seq)


def c1() -> Workload:
    """One sequence, 256 tokens appended at positions 0..255, then one decode
    step over all 256 with 32 query heads; Bh 32, page size 16, identity
    page table."""
    T = 256
    return Workload(
        name="c1", cfg_id=1, batch=1, num_kv_heads=NUM_KV_HEADS, num_q_heads=NUM_Q_HEADS,
        head_dim=HEAD_DIM, had_block=32, page_size=16, num_pages=16,
        page_table=_identity_table(1, 16), prefill_lens=np.zeros(1, np.int32),
        append_seq=np.zeros(T, np.int32), append_pos=np.arange(T, dtype=np.int32),
        context_lens=np.full(1, T, np.int32),
        description="1 seq x 256 tokens, Hkv 8 x D 128, Hq 32, Bh 32, P 16, identity pages")


def _c2_table(cfg_id: int):
    r = np_rng(cfg_id, _PAGES, 0)
    perm = r.permutation(65536).astype(np.int32)
    return perm.reshape(256, 256)


def c2() -> Workload:
    """256 sequences each appending one decode token into a 1M-token page pool
    (65,536 pages of 16) through a seeded random permutation; Bh 64."""
    pt = _c2_table(2)
    lens = np_rng(2, _LENS, 0).integers(0, 4096, size=256).astype(np.int32)
    return Workload(
        name="c2", cfg_id=2, batch=256, num_kv_heads=NUM_KV_HEADS, num_q_heads=NUM_Q_HEADS,
        head_dim=HEAD_DIM, had_block=64, page_size=16, num_pages=65536, page_table=pt,
        prefill_lens=lens, append_seq=np.arange(256, dtype=np.int32), append_pos=lens.copy(),
        context_lens=lens + 1,
        description="append-only: 256 seqs x 1 token, Bh 64, P 16, 65,536-page pool, random permutation")


def c2_stream(tokens_per_seq: int = 256) -> Workload:
    """Same layout as c2, but each sequence appends ``tokens_per_seq``
    consecutive tokens, so one call moves enough bytes to measure bandwidth."""
    pt = _c2_table(2)
    start = np_rng(2, _LENS, 1).integers(0, 4096 - tokens_per_seq + 1, size=256).astype(np.int32)
    seq = np.repeat(np.arange(256, dtype=np.int32), tokens_per_seq)
    pos = (start[:, None] + np.arange(tokens_per_seq, dtype=np.int32)[None, :]).reshape(-1)
    return Workload(
        name="c2_stream", cfg_id=2, batch=256, num_kv_heads=NUM_KV_HEADS, num_q_heads=NUM_Q_HEADS,
        head_dim=HEAD_DIM, had_block=64, page_size=16, num_pages=65536, page_table=pt,
        prefill_lens=start, append_seq=seq, append_pos=pos.astype(np.int32),
        context_lens=start + tokens_per_seq,
        description=f"append: 256 seqs x {tokens_per_seq} consecutive tokens, Bh 64, P 16, 65,536-page pool")


def c3(layers: int = 36) -> Workload:
    """Batch 1, context 32,768, 36 layers each with its own 2048-page pool and
    random page permutation; Bh 128, P 16."""
    ctx = 32768
    tables = [np_rng(3, _PAGES, l).permutation(2048).astype(np.int32).reshape(1, 2048)
              for l in range(layers)]
    return Workload(
        name="c3", cfg_id=3, batch=1, num_kv_heads=NUM_KV_HEADS, num_q_heads=NUM_Q_HEADS,
        head_dim=HEAD_DIM, had_block=128, page_size=16, num_pages=2048, page_table=tables[0],
        prefill_lens=np.full(1, ctx, np.int32), append_seq=np.zeros(0, np.int32),
        append_pos=np.zeros(0, np.int32), context_lens=np.full(1, ctx, np.int32), layers=layers,
        per_layer_page_tables=tables,
        description="batch 1, ctx 32768, 36 layers, Hkv 8 x D 128, Hq 32, Bh 128, P 16, scattered pages")


def c4(batch: int = 256, lo: int = 1024, hi: int = 8192, cfg_id: int = 4) -> Workload:
    """Batch of sequences with context lengths uniform in [lo, hi]; the step
    appends one token at position ctx_b and decodes over ctx_b + 1.  Pages are
    one global permutation split by sequence; Bh 64, P 16."""
    P = 16
    ctx = np_rng(cfg_id, _LENS, 0).integers(lo, hi + 1, size=batch).astype(np.int32)
    need = (ctx + 1 + P - 1) // P
    total = int(need.sum())
    perm = np_rng(cfg_id, _PAGES, 0).permutation(total).astype(np.int32)
    maxp = int(need.max())
    pt = np.full((batch, maxp), -1, np.int32)
    off = 0
    for b in range(batch):
        pt[b, :need[b]] = perm[off:off + need[b]]
        off += int(need[b])
    return Workload(
        name="c4" if cfg_id == 4 else f"c4_{batch}_{lo}_{hi}", cfg_id=cfg_id, batch=batch,
        num_kv_heads=NUM_KV_HEADS, num_q_heads=NUM_Q_HEADS, head_dim=HEAD_DIM, had_block=64,
        page_size=P, num_pages=total, page_table=pt, prefill_lens=ctx,
        append_seq=np.arange(batch, dtype=np.int32), append_pos=ctx.copy(),
        context_lens=ctx + 1,
        description=f"decode+append: batch {batch}, ctx U[{lo},{hi}], Hkv 8 x D 128, Hq 32, Bh 64, P 16")


def c5(batch: int = 8, ctx: int = 131072, had_block: int = 128, cfg_id: int = 5) -> Workload:
    """Long context: batch 8 x 131,072 tokens, P 32, scattered pages; K with
    8 outlier channels x50 per head, V plain normal."""
    P = 32
    per = ctx // P
    total = batch * per
    perm = np_rng(cfg_id, _PAGES, 0).permutation(total).astype(np.int32)
    return Workload(
        name="c5" if had_block == 128 else f"c5_bh{had_block}", cfg_id=cfg_id, batch=batch,
        num_kv_heads=NUM_KV_HEADS, num_q_heads=NUM_Q_HEADS, head_dim=HEAD_DIM,
        had_block=had_block, page_size=P, num_pages=total, page_table=perm.reshape(batch, per),
        prefill_lens=np.full(batch, ctx, np.int32), append_seq=np.zeros(0, np.int32),
        append_pos=np.zeros(0, np.int32), context_lens=np.full(batch, ctx, np.int32),
        k_outliers=8, k_mult=50.0, v_outliers=0, v_mult=1.0,
        description=f"long context: batch {batch} x {ctx}, Bh {had_block}, P 32, K 8 outliers x50")


def small(batch: int, lens, had_block: int, page_size: int, cfg_id: int,
          num_kv_heads: int = NUM_KV_HEADS, num_q_heads: int = NUM_Q_HEADS,
          spare_pages: int = 3) -> Workload:
    """A small decode workload (oracle-sized) with arbitrary context lengths,
    a shuffled page pool and a few spare pages never referenced."""
    lens = np.asarray(lens, np.int32)
    P = page_size
    need = np.maximum((lens + P - 1) // P, 1)
    total = int(need.sum()) + spare_pages
    perm = np_rng(cfg_id, _PAGES, 0).permutation(total).astype(np.int32)
    maxp = int(need.max())
    pt = np.full((batch, maxp), -1, np.int32)
    off = 0
    for b in range(batch):
        pt[b, :need[b]] = perm[off:off + need[b]]
        off += int(need[b])
    return Workload(
        name=f"small{cfg_id}", cfg_id=cfg_id, batch=batch, num_kv_heads=num_kv_heads,
        num_q_heads=num_q_heads, head_dim=HEAD_DIM, had_block=had_block, page_size=P,
        num_pages=total, page_table=pt, prefill_lens=np.maximum(lens, 0),
        append_seq=np.zeros(0, np.int32), append_pos=np.zeros(0, np.int32),
        context_lens=lens, description="small decode case")


def prefill_tokens(w: Workload, b: int):
    """(seq, pos) arrays for the tokens already cached in sequence b."""
    n = int(max(w.prefill_lens[b], 0))
    return np.full(n, b, np.int32), np.arange(n, dtype=np.int32)

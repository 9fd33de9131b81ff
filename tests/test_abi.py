"""C-ABI checks that need no GPU: the library loads, exports every function
include/kvq.h declares, and rejects bad arguments on the host before any
launch.  No call here reaches a kernel."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import bit_kv_cache_quant_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_expected_entry_points():
    names = _declared_functions()
    for must in ("kv_quant_append", "paged_decode_attn_int4", "paged_prefill_attn_int4", "kv_append_fp16",
                 "paged_decode_attn_fp16", "paged_decode_attn_workspace_bytes",
                 "kvq_page_tile_bytes", "kvq_status_string"):
        assert must in names
    assert set(names) == set(kvq.SIGNATURES), "binding signatures must cover the header exactly"


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kvq.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_tile_bytes():
    assert kvq.status_string(kvq.KVQ_OK) == "ok"
    assert "workspace" in kvq.status_string(kvq.KVQ_ERR_WORKSPACE)
    assert kvq.page_tile_bytes(128, 16) == 1056
    assert kvq.page_tile_bytes(128, 32) == 2112
    assert kvq.page_tile_bytes(64, 16) == 0
    assert kvq.page_tile_bytes(128, 8) == 0


def _split_bytes(batch, hq, hkv, ctx, P, pps=0):
    """Split-mode workspace (batches below 16 or above 4096)."""
    npages = max(1, -(-ctx // P))
    chunks = -(-(hq // hkv) // 4)
    if pps <= 0:
        items = batch * hkv * chunks
        want = 1 if items >= 1024 else -(-1024 // items)
        pps = -(-npages // want)
    pps = max(1, min(pps, 2048 // P))
    cp = 64 // P
    pps = -(-pps // cp) * cp
    return batch * hq * (-(-npages // pps)) * 130 * 4


def _balanced_bytes(batch, hq, hkv, ctx, P, pps=0):
    """Balanced decode workspace (16 <= batch <= 4096): quads x (groups +
    batch) x 16 partial states of 130 floats, then batch + 1 int32 prefix sums
    (16-byte padded)."""
    if batch < 16 or batch > 4096:
        return 0
    quads = -(-(hkv * -(-(hq // hkv) // 4)) // 4)
    tot_max = max(1, batch * (-(-ctx // 64)))
    if pps <= 0:
        gmax = max(1, 1024 // quads)
        gmin = max(1, gmax // 2)
    else:
        cpr = max(1, -(-(pps * P) // 64))
        gmax = gmin = -(-tot_max // cpr)
    g = min(max(-(-tot_max // 32), gmin), gmax)       # ranges of ~32 chunks within [gmin, gmax]
    groups = max(1, min(max(g, -(-tot_max // 64)), tot_max))
    units = quads * (groups + batch) * 16
    return units * 130 * 4 + -(-((batch + 1) * 4) // 16) * 16


def test_workspace_query():
    # the larger of the two layouts (one workspace serves INT4 and fp16 calls)
    for args, pps in [((1, 32, 8, 256, 16), 0), ((1, 32, 8, 256, 16), 4), ((1, 32, 8, 256, 16), 1),
                      ((1, 32, 8, 256, 32), 1), ((256, 32, 8, 8193, 16), 0), ((256, 32, 8, 8193, 16), 1000),
                      ((8, 32, 8, 131072, 32), 0), ((3, 32, 8, 129, 16), 0), ((1, 8, 8, 300, 16), 0),
                      ((2, 32, 8, 256, 16), 4), ((16, 32, 8, 256, 16), 4), ((4096, 32, 8, 64, 16), 0),
                      ((4097, 32, 8, 64, 16), 0)]:
        want = max(_split_bytes(*args, pps), _balanced_bytes(*args, pps))
        assert kvq.workspace_bytes(*args, pages_per_split=pps) == want, (args, pps)
    # hand-checked values: ctx 256 at P 16 is 4 chunks
    assert _split_bytes(1, 32, 8, 256, 16) == 1 * 32 * 4 * 130 * 4
    assert _balanced_bytes(16, 32, 8, 256, 16, 4) == 2 * (64 + 16) * 16 * 130 * 4 + 80
    # long sequences: split mode caps a split at 2048 tokens
    assert _split_bytes(256, 32, 8, 8193, 16) == 256 * 32 * 5 * 130 * 4
    assert kvq.workspace_bytes(0, 32, 8, 256, 16) == 0
    assert kvq.workspace_bytes(1, 30, 8, 256, 16) == 0      # Hq not a multiple of Hkv


FAKE = 0x1000  # an aligned, never-dereferenced address


def _append(**kw):
    a = dict(k=FAKE, v=FAKE, seq=FAKE, pos=FAKE, T=4, pt=FAKE, maxp=4, kp=FAKE, vp=FAKE, npages=8,
             hkv=8, d=128, P=16, bh=64, stream=None)
    a.update(kw)
    return kvq.lib().kv_quant_append(a["k"], a["v"], a["seq"], a["pos"], a["T"], a["pt"], a["maxp"],
                                     a["kp"], a["vp"], a["npages"], a["hkv"], a["d"], a["P"], a["bh"],
                                     a["stream"])


def test_append_host_validation_rejects_before_launch():
    assert _append(d=64) == kvq.KVQ_ERR_UNSUPPORTED
    assert _append(P=8) == kvq.KVQ_ERR_UNSUPPORTED
    assert _append(bh=16) == kvq.KVQ_ERR_UNSUPPORTED
    assert _append(bh=256) == kvq.KVQ_ERR_UNSUPPORTED
    assert _append(k=None) == kvq.KVQ_ERR_INVALID_ARG
    assert _append(kp=FAKE + 4) == kvq.KVQ_ERR_INVALID_ARG    # misaligned pool
    assert _append(T=-1) == kvq.KVQ_ERR_INVALID_ARG
    assert _append(hkv=0) == kvq.KVQ_ERR_INVALID_ARG
    assert _append(T=0, k=None, v=None) == kvq.KVQ_OK          # empty call: no-op
    assert _append(T=1, hkv=1 << 30) == kvq.KVQ_ERR_UNSUPPORTED  # 2^31 blocks: beyond one grid dimension


def _decode(**kw):
    a = dict(q=FAKE, kp=FAKE, vp=FAKE, npages=8, pt=FAKE, maxp=4, cl=FAKE, B=2, maxctx=64, hq=32, hkv=8,
             d=128, P=16, bh=64, scale=0.088, out=FAKE, ws=FAKE, wsb=1 << 20, pps=0, ev=None, stream=None)
    a.update(kw)
    return kvq.lib().paged_decode_attn_int4(a["q"], a["kp"], a["vp"], a["npages"], a["pt"], a["maxp"],
                                            a["cl"], a["B"], a["maxctx"], a["hq"], a["hkv"], a["d"], a["P"],
                                            a["bh"], a["scale"], a["out"], a["ws"], a["wsb"], a["pps"],
                                            a["ev"], a["stream"])


def test_decode_host_validation_rejects_before_launch():
    assert _decode(d=256) == kvq.KVQ_ERR_UNSUPPORTED
    assert _decode(P=64) == kvq.KVQ_ERR_UNSUPPORTED
    assert _decode(bh=48) == kvq.KVQ_ERR_UNSUPPORTED
    assert _decode(hq=30) == kvq.KVQ_ERR_INVALID_ARG
    assert _decode(maxctx=65) == kvq.KVQ_ERR_INVALID_ARG      # exceeds max_pages * P
    assert _decode(q=None) == kvq.KVQ_ERR_INVALID_ARG
    assert _decode(out=FAKE + 8) == kvq.KVQ_ERR_INVALID_ARG
    assert _decode(ws=None) == kvq.KVQ_ERR_WORKSPACE
    assert _decode(wsb=100) == kvq.KVQ_ERR_WORKSPACE
    assert _decode(pps=-1) == kvq.KVQ_ERR_INVALID_ARG
    assert _decode(B=0, q=None, out=None) == kvq.KVQ_OK       # empty batch: no-op


def _step(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kp=FAKE, vp=FAKE, npages=8, pt=FAKE, maxp=4, cl=FAKE, B=2, maxctx=64,
             hq=32, hkv=8, d=128, P=16, bh=64, scale=0.088, out=FAKE, ws=FAKE, wsb=1 << 20, pps=0, ev=None,
             stream=None)
    a.update(kw)
    return kvq.lib().paged_decode_step_int4(a["q"], a["kn"], a["vn"], a["kp"], a["vp"], a["npages"], a["pt"],
                                            a["maxp"], a["cl"], a["B"], a["maxctx"], a["hq"], a["hkv"], a["d"],
                                            a["P"], a["bh"], a["scale"], a["out"], a["ws"], a["wsb"], a["pps"],
                                            a["ev"], a["stream"])


def test_fused_step_host_validation_rejects_before_launch():
    """The fused step checks its new-token rows and then everything the
    decode checks."""
    assert _step(kn=None) == kvq.KVQ_ERR_INVALID_ARG
    assert _step(vn=None) == kvq.KVQ_ERR_INVALID_ARG
    assert _step(kn=FAKE + 2) == kvq.KVQ_ERR_INVALID_ARG       # misaligned rows
    assert _step(bh=48) == kvq.KVQ_ERR_UNSUPPORTED
    assert _step(P=64) == kvq.KVQ_ERR_UNSUPPORTED
    assert _step(maxctx=65) == kvq.KVQ_ERR_INVALID_ARG
    assert _step(ws=None) == kvq.KVQ_ERR_WORKSPACE
    assert _step(B=0, q=None, out=None) == kvq.KVQ_OK           # empty batch: no-op


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kvq, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(kvq, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        kvq.lib()


def test_binding_rejects_mis_shaped_pools_before_launch():
    """A pool smaller than [num_pages][Hkv][tile] (or [num_pages][Hkv][P][D]
    for fp16) is refused on the host, before any pointer reaches a kernel."""
    import torch
    k = torch.zeros((2, 8, 128), dtype=torch.float16)
    idx = torch.zeros(2, dtype=torch.int32)
    pt = torch.zeros((1, 4), dtype=torch.int32)
    half_pool = torch.zeros((4, 8, 16, 64), dtype=torch.float16)     # last dim halved
    with pytest.raises(ValueError, match="pools must"):
        kvq.kv_append_fp16(k, k, idx, idx, pt, half_pool, half_pool, 16)
    short_tile = torch.zeros((4, 8, 1024), dtype=torch.uint8)
    with pytest.raises(ValueError, match="pools must"):
        kvq.kv_quant_append(k, k, idx, idx, pt, short_tile, short_tile, 16, 64)
    q = torch.zeros((1, 32, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="pools must"):
        kvq.paged_decode_attn_int4(q, short_tile, short_tile, pt, torch.zeros(1, dtype=torch.int32), 8, 16, 64,
                                   0.088, 64)


def test_binding_rejects_a_host_workspace_before_launch():
    """The workspace is checked like every other tensor: a CPU tensor (or a
    non-contiguous view) never reaches the kernels as a device pointer."""
    import torch
    pool = torch.zeros((4, 8, 1056), dtype=torch.uint8)
    q = torch.zeros((1, 32, 128), dtype=torch.float16)
    pt = torch.zeros((1, 4), dtype=torch.int32)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    # the workspace is checked before the other tensors are marshalled
    with pytest.raises(ValueError, match="workspace must be a GPU tensor"):
        kvq.paged_decode_attn_int4(q, pool, pool, pt, torch.zeros(1, dtype=torch.int32), 8, 16, 64, 0.088, 64,
                                   workspace=ws)


def _prefill(**kw):
    a = dict(q=FAKE, qs=FAKE, nq=32, kp=FAKE, vp=FAKE, npages=8, pt=FAKE, maxp=4, cl=FAKE, B=1, hq=32, hkv=8,
             d=128, P=16, bh=64, scale=0.088, out=FAKE, stream=None)
    a.update(kw)
    return kvq.lib().paged_prefill_attn_int4(a["q"], a["qs"], a["nq"], a["kp"], a["vp"], a["npages"], a["pt"],
                                             a["maxp"], a["cl"], a["B"], a["hq"], a["hkv"], a["d"], a["P"],
                                             a["bh"], a["scale"], a["out"], a["stream"])


def test_prefill_host_validation():
    """Rejected on the host before any launch (no pointer is dereferenced)."""
    assert _prefill(d=64) == kvq.KVQ_ERR_UNSUPPORTED
    assert _prefill(P=8) == kvq.KVQ_ERR_UNSUPPORTED
    assert _prefill(bh=16) == kvq.KVQ_ERR_UNSUPPORTED
    assert _prefill(hq=30) == kvq.KVQ_ERR_INVALID_ARG
    assert _prefill(nq=-1) == kvq.KVQ_ERR_INVALID_ARG
    assert _prefill(q=None) == kvq.KVQ_ERR_INVALID_ARG
    assert _prefill(qs=None) == kvq.KVQ_ERR_INVALID_ARG
    assert _prefill(out=FAKE + 4) == kvq.KVQ_ERR_INVALID_ARG     # misaligned
    assert _prefill(scale=0.0) == kvq.KVQ_ERR_INVALID_ARG        # the scale must be positive
    assert _prefill(scale=-0.088) == kvq.KVQ_ERR_INVALID_ARG
    assert _prefill(scale=float("nan")) == kvq.KVQ_ERR_INVALID_ARG
    assert _prefill(nq=0) == kvq.KVQ_OK                           # no-op
    assert _prefill(B=0) == kvq.KVQ_OK


def test_noalloc_decode_rejects_requests_beyond_the_scratch_on_the_host():
    """The allocation-free decode refuses, before touching the device, a call
    whose partial states need more than its static scratch (here batch 4096 x
    8192 context: 260 MiB against 32 MiB); a call that fits is checked the
    same way as the workspace entry point."""
    lib = kvq.lib()
    need = kvq.workspace_bytes(4096, 32, 8, 8192, 16)
    assert need > kvq.SCRATCH_BYTES
    rc = lib.paged_decode_attn_int4_noalloc(FAKE, FAKE, FAKE, 1 << 20, FAKE, 512, FAKE, 4096, 8192, 32, 8, 128,
                                            16, 64, 0.088, FAKE, 0, None, None)
    assert rc == kvq.KVQ_ERR_TOO_LARGE
    assert "scratch" in kvq.status_string(kvq.KVQ_ERR_TOO_LARGE)
    # argument errors come first, as in the workspace entry point
    assert lib.paged_decode_attn_int4_noalloc(FAKE, FAKE, FAKE, 8, FAKE, 4, FAKE, 2, 64, 32, 8, 256, 16, 64, 0.088,
                                              FAKE, 0, None, None) == kvq.KVQ_ERR_UNSUPPORTED
    assert lib.paged_decode_attn_int4_noalloc(None, FAKE, FAKE, 8, FAKE, 4, FAKE, 0, 64, 32, 8, 128, 16, 64, 0.088,
                                              None, 0, None, None) == kvq.KVQ_OK

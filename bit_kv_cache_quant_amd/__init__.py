"""Python binding of the MI355X INT4 KV-cache library (``libkvq.so``).

Argument marshalling only: every function checks shapes, dtypes, devices and
contiguity of torch tensors, then calls the C entry point of the same name
with raw device pointers and the current HIP stream.  All computation happens
in the HIP kernels.  If the library has not been built, importing the
functions raises ``RuntimeError``; there is no fallback.

The computation and the layouts are documented in ``include/kvq.h``.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

KVQ_OK = 0
KVQ_ERR_INVALID_ARG = -1
KVQ_ERR_UNSUPPORTED = -2
KVQ_ERR_WORKSPACE = -3
KVQ_ERR_HIP = -4
KVQ_ERR_TOO_LARGE = -5
SCRATCH_BYTES = 32 << 20     # KVQ_SCRATCH_BYTES: the allocation-free decode's static scratch

HEAD_DIM = 128

FORMAT_INT4 = 0
FORMAT_MXFP4 = 1


class QuantConfig(ctypes.Structure):
    """kvq_quant_config: quantizer variant (format, had_block, scale_group,
    scale_search, sign_mask as four 32-bit words; see include/kvq.h)."""
    _fields_ = [("format", ctypes.c_int32), ("had_block", ctypes.c_int32), ("scale_group", ctypes.c_int32),
                ("scale_search", ctypes.c_int32), ("sign_mask", ctypes.c_uint32 * 4)]


def quant_config(format: int = FORMAT_INT4, had_block: int = 0, scale_group: int = 128, scale_search: int = 0,
                 sign_mask: int = 0) -> QuantConfig:
    """A configuration; sign_mask is a 128-bit integer (bit i negates channel i)."""
    c = QuantConfig()
    c.format, c.had_block, c.scale_group, c.scale_search = int(format), int(had_block), int(scale_group), \
        int(scale_search)
    for w in range(4):
        c.sign_mask[w] = (int(sign_mask) >> (32 * w)) & 0xFFFFFFFF
    return c


# Every symbol include/kvq.h declares, with its ctypes signature.
_P, _I32, _I64, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_CFG = ctypes.POINTER(QuantConfig)
SIGNATURES = {
    "kvq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvq_page_tile_bytes": (_SZ, [_I32, _I32]),
    "kv_quant_append": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _I32, _P, _P, _I64, _I32, _I32, _I32, _I32, _P]),
    "paged_decode_attn_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "paged_decode_attn_int4": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32,
                                              _I32, _I32, _F32, _P, _P, _SZ, _I32, _P, _P]),
    "paged_decode_step_int4": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _I32, _I32,
                                              _I32, _I32, _I32, _F32, _P, _P, _SZ, _I32, _P, _P]),
    "paged_prefill_attn_int4": (ctypes.c_int, [_P, _P, _I32, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _I32, _I32,
                                               _I32, _I32, _F32, _P, _P]),
    "kvq_page_tile_bytes_cfg": (_SZ, [_I32, _I32, _CFG]),
    "kv_quant_append_cfg": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _I32, _P, _P, _I64, _I32, _I32, _I32, _CFG,
                                           _P]),
    "paged_decode_attn_cfg": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                             _CFG, _F32, _P, _P, _SZ, _I32, _P, _P]),
    "kv_append_fp16": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _I32, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "paged_decode_attn_int4_noalloc": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _I32, _I32,
                                                      _I32, _I32, _I32, _F32, _P, _I32, _P, _P]),
    "paged_decode_attn_fp16": (ctypes.c_int, [_P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32,
                                              _I32, _F32, _P, _P, _SZ, _I32, _P, _P]),
}

_lib = None


class KVQError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: status {status} ({status_string(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libkvq.so (built by ``python -m bit_kv_cache_quant_amd._build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run python -m bit_kv_cache_quant_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kvq_status_string(int(status)).decode()


_tile_bytes_cache: dict = {}


def page_tile_bytes(head_dim: int, page_size: int) -> int:
    key = (int(head_dim), int(page_size))
    v = _tile_bytes_cache.get(key)
    if v is None:
        v = _tile_bytes_cache[key] = int(lib().kvq_page_tile_bytes(key[0], key[1]))
    return v


def workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, max_context_len: int,
                    page_size: int, pages_per_split: int = 0, head_dim: int = HEAD_DIM) -> int:
    return int(lib().paged_decode_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                       max_context_len, page_size, pages_per_split))


# --------------------------------------------------------------------------
def _stream(t) -> int:
    """The raw handle of the current stream of t's GPU (torch's own accessor
    for it when present: building a Stream object costs ~3 us per call)."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return int(raw(t.get_device()))
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t, dtype, name: str, ndim: int | None = None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    return t.data_ptr()


def _check(rc: int, what: str) -> None:
    if rc != KVQ_OK:
        raise KVQError(rc, what)


def kv_quant_append(k_new, v_new, token_seq, token_pos, page_table, k_pool, v_pool,
                    page_size: int, had_block: int) -> None:
    """Rotate, quantize and append new tokens into INT4 pools (in place).

    k_new, v_new: fp16 [T][Hkv][D]; token_seq, token_pos: int32 [T];
    page_table: int32 [B][max_pages]; k_pool, v_pool: uint8 [num_pages][Hkv][tile].
    """
    import torch
    T, hkv, d = k_new.shape
    if tuple(v_new.shape) != (T, hkv, d):
        raise ValueError("k_new and v_new shapes differ")
    tile = page_tile_bytes(d, int(page_size))
    if (k_pool.dim() != 3 or tuple(v_pool.shape) != tuple(k_pool.shape)
            or tuple(k_pool.shape[1:]) != (hkv, tile)):
        raise ValueError(f"pools must both be [num_pages][{hkv}][{tile}], got {tuple(k_pool.shape)} "
                         f"and {tuple(v_pool.shape)}")
    if token_seq.numel() != T or token_pos.numel() != T:
        raise ValueError("token_seq/token_pos must have one entry per token")
    rc = lib().kv_quant_append(
        _dev(k_new, torch.float16, "k_new", 3), _dev(v_new, torch.float16, "v_new", 3),
        _dev(token_seq, torch.int32, "token_seq"), _dev(token_pos, torch.int32, "token_pos"), T,
        _dev(page_table, torch.int32, "page_table", 2), page_table.shape[1],
        _dev(k_pool, torch.uint8, "k_pool"), _dev(v_pool, torch.uint8, "v_pool"), k_pool.shape[0],
        hkv, d, int(page_size), int(had_block), _stream(k_new))
    _check(rc, "kv_quant_append")


def page_tile_bytes_cfg(head_dim: int, page_size: int, cfg: QuantConfig) -> int:
    return int(lib().kvq_page_tile_bytes_cfg(head_dim, page_size, ctypes.byref(cfg)))


def kv_quant_append_cfg(k_new, v_new, token_seq, token_pos, page_table, k_pool, v_pool,
                        page_size: int, cfg: QuantConfig) -> None:
    """kv_quant_append under a quantizer configuration; pools uint8
    [num_pages][Hkv][page_tile_bytes_cfg(...)]."""
    import torch
    T, hkv, d = k_new.shape
    if tuple(v_new.shape) != (T, hkv, d):
        raise ValueError("k_new and v_new shapes differ")
    tile = page_tile_bytes_cfg(d, int(page_size), cfg)
    if tile == 0:
        raise KVQError(KVQ_ERR_UNSUPPORTED, "kv_quant_append_cfg")
    if (k_pool.dim() != 3 or tuple(v_pool.shape) != tuple(k_pool.shape)
            or tuple(k_pool.shape[1:]) != (hkv, tile)):
        raise ValueError(f"pools must both be [num_pages][{hkv}][{tile}], got {tuple(k_pool.shape)} "
                         f"and {tuple(v_pool.shape)}")
    if token_seq.numel() != T or token_pos.numel() != T:
        raise ValueError("token_seq/token_pos must have one entry per token")
    rc = lib().kv_quant_append_cfg(
        _dev(k_new, torch.float16, "k_new", 3), _dev(v_new, torch.float16, "v_new", 3),
        _dev(token_seq, torch.int32, "token_seq"), _dev(token_pos, torch.int32, "token_pos"), T,
        _dev(page_table, torch.int32, "page_table", 2), page_table.shape[1],
        _dev(k_pool, torch.uint8, "k_pool"), _dev(v_pool, torch.uint8, "v_pool"), k_pool.shape[0],
        hkv, d, int(page_size), ctypes.byref(cfg), _stream(k_new))
    _check(rc, "kv_quant_append_cfg")


def kv_append_fp16(k_new, v_new, token_seq, token_pos, page_table, k_pool, v_pool,
                   page_size: int) -> None:
    """Baseline: copy new tokens into fp16 pools [num_pages][Hkv][P][D] (in place)."""
    import torch
    T, hkv, d = k_new.shape
    if tuple(v_new.shape) != (T, hkv, d):
        raise ValueError("k_new and v_new shapes differ")
    if (k_pool.dim() != 4 or tuple(v_pool.shape) != tuple(k_pool.shape)
            or tuple(k_pool.shape[1:]) != (hkv, int(page_size), d)):
        raise ValueError(f"pools must both be [num_pages][{hkv}][{page_size}][{d}], got "
                         f"{tuple(k_pool.shape)} and {tuple(v_pool.shape)}")
    if token_seq.numel() != T or token_pos.numel() != T:
        raise ValueError("token_seq/token_pos must have one entry per token")
    rc = lib().kv_append_fp16(
        _dev(k_new, torch.float16, "k_new", 3), _dev(v_new, torch.float16, "v_new", 3),
        _dev(token_seq, torch.int32, "token_seq"), _dev(token_pos, torch.int32, "token_pos"), T,
        _dev(page_table, torch.int32, "page_table", 2), page_table.shape[1],
        _dev(k_pool, torch.float16, "k_pool"), _dev(v_pool, torch.float16, "v_pool"), k_pool.shape[0],
        hkv, d, int(page_size), _stream(k_new))
    _check(rc, "kv_append_fp16")


def _event_handle(event):
    """hipEvent_t of a torch.cuda.Event (which must have been recorded once, so
    that it exists), or None."""
    return None if event is None else event.cuda_event


def _decode(int4: bool, q, k_pool, v_pool, page_table, context_lens, num_kv_heads: int,
            page_size: int, had_block: int, softmax_scale: float, max_context_len: int,
            out=None, workspace=None, pages_per_split: int = 0, phase_event=None, cfg=None,
            k_new=None, v_new=None):
    import torch
    B, hq, d = q.shape
    if k_new is not None:
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if t is None or tuple(t.shape) != (B, int(num_kv_heads), d):
                raise ValueError(f"{name} must be [{B}][{num_kv_heads}][{d}]")
    if cfg is not None:
        want = (int(num_kv_heads), page_tile_bytes_cfg(d, int(page_size), cfg))
    elif int4:
        want = (int(num_kv_heads), page_tile_bytes(d, int(page_size)))
    else:
        want = (int(num_kv_heads), int(page_size), d)
    if (tuple(k_pool.shape[1:]) != want or tuple(v_pool.shape) != tuple(k_pool.shape)):
        raise ValueError(f"pools must both be [num_pages]{list(want)}, got {tuple(k_pool.shape)} "
                         f"and {tuple(v_pool.shape)}")
    if context_lens.numel() != B or page_table.dim() != 2 or page_table.shape[0] < B:
        raise ValueError("context_lens must have one entry per sequence and page_table one row each")
    if out is not None and tuple(out.shape) != (B, hq, d):
        raise ValueError(f"out must be [{B}][{hq}][{d}]")
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:   # (a caller's workspace is checked against the need by the library)
        need = workspace_bytes(B, hq, num_kv_heads, max_context_len, page_size, pages_per_split, d) if B else 0
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, torch.uint8, "workspace")
    if workspace.device != q.device:
        raise ValueError(f"workspace must be on {q.device}, got {workspace.device}")
    ws_bytes = workspace.numel()
    pool_dtype = torch.uint8 if int4 else torch.float16
    args = [_dev(q, torch.float16, "q", 3)]
    if k_new is not None:
        args += [_dev(k_new, torch.float16, "k_new", 3), _dev(v_new, torch.float16, "v_new", 3)]
    args += [_dev(k_pool, pool_dtype, "k_pool"),
            _dev(v_pool, pool_dtype, "v_pool"), k_pool.shape[0],
            _dev(page_table, torch.int32, "page_table", 2), page_table.shape[1],
            _dev(context_lens, torch.int32, "context_lens", 1), B, int(max_context_len), hq,
            int(num_kv_heads), d, int(page_size)]
    if cfg is not None:
        args.append(ctypes.byref(cfg))
    elif int4:
        args.append(int(had_block))
    args += [float(softmax_scale), _dev(out, torch.float32, "out", 3), ws_ptr, ws_bytes,
             int(pages_per_split), _event_handle(phase_event), _stream(q)]
    if k_new is not None:
        name = "paged_decode_step_int4"
    else:
        name = "paged_decode_attn_cfg" if cfg is not None else ("paged_decode_attn_int4" if int4
                                                                else "paged_decode_attn_fp16")
    _check(getattr(lib(), name)(*args), name)
    return out


def paged_decode_attn_cfg(q, k_pool, v_pool, page_table, context_lens, num_kv_heads: int, page_size: int,
                          cfg: QuantConfig, softmax_scale: float, max_context_len: int, out=None, workspace=None,
                          pages_per_split: int = 0, phase_event=None):
    """One decode step over a cache written by kv_quant_append_cfg with the
    same configuration; returns fp32 [B][Hq][D]."""
    return _decode(True, q, k_pool, v_pool, page_table, context_lens, num_kv_heads, page_size, 0,
                   softmax_scale, max_context_len, out, workspace, pages_per_split, phase_event, cfg)


def paged_prefill_attn_int4(q, q_start, k_pool, v_pool, page_table, context_lens, num_kv_heads: int,
                            page_size: int, had_block: int, softmax_scale: float, out=None):
    """Causal prefill attention over the INT4 cache: rows q_start[b] ..
    q_start[b+1]-1 of q (fp16 [num_q][Hq][D]) are the last positions of
    sequence b; returns fp32 [num_q][Hq][D]."""
    import torch
    nq, hq, d = q.shape
    B = context_lens.numel()
    want = (int(num_kv_heads), page_tile_bytes(d, int(page_size)))
    if tuple(k_pool.shape[1:]) != want or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError(f"pools must both be [num_pages]{list(want)}")
    if q_start.numel() != B + 1 or page_table.dim() != 2 or page_table.shape[0] < B:
        raise ValueError("q_start must have batch + 1 entries and page_table one row per sequence")
    if out is None:
        out = torch.empty((nq, hq, d), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (nq, hq, d):
        raise ValueError(f"out must be [{nq}][{hq}][{d}]")
    _check(lib().paged_prefill_attn_int4(
        _dev(q, torch.float16, "q", 3), _dev(q_start, torch.int32, "q_start", 1), nq,
        _dev(k_pool, torch.uint8, "k_pool"), _dev(v_pool, torch.uint8, "v_pool"), k_pool.shape[0],
        _dev(page_table, torch.int32, "page_table", 2), page_table.shape[1],
        _dev(context_lens, torch.int32, "context_lens", 1), B, hq, int(num_kv_heads), d, int(page_size),
        int(had_block), float(softmax_scale), _dev(out, torch.float32, "out", 3), _stream(q)),
        "paged_prefill_attn_int4")
    return out


def paged_decode_attn_int4(q, k_pool, v_pool, page_table, context_lens, num_kv_heads: int,
                           page_size: int, had_block: int, softmax_scale: float,
                           max_context_len: int, out=None, workspace=None, pages_per_split: int = 0,
                           phase_event=None):
    """One decode step over the INT4 cache; returns fp32 [B][Hq][D].
    ``phase_event`` (a torch.cuda.Event recorded once before, or None) is
    recorded between the split-K partial kernel and the merge."""
    return _decode(True, q, k_pool, v_pool, page_table, context_lens, num_kv_heads, page_size,
                   had_block, softmax_scale, max_context_len, out, workspace, pages_per_split, phase_event)


def paged_decode_step_int4(q, k_new, v_new, k_pool, v_pool, page_table, context_lens, num_kv_heads: int,
                           page_size: int, had_block: int, softmax_scale: float, max_context_len: int,
                           out=None, workspace=None, pages_per_split: int = 0, phase_event=None):
    """One decode step with its append: the new token of sequence b
    (k_new[b], v_new[b], fp16 [B][Hkv][D]) goes into the INT4 pools at
    position context_lens[b] - 1, and attention runs over positions
    0 .. context_lens[b] - 1; returns fp32 [B][Hq][D]."""
    return _decode(True, q, k_pool, v_pool, page_table, context_lens, num_kv_heads, page_size,
                   had_block, softmax_scale, max_context_len, out, workspace, pages_per_split, phase_event,
                   k_new=k_new, v_new=v_new)


def paged_decode_attn_fp16(q, k_pool, v_pool, page_table, context_lens, num_kv_heads: int,
                           page_size: int, softmax_scale: float, max_context_len: int,
                           out=None, workspace=None, pages_per_split: int = 0, phase_event=None):
    """Baseline decode over fp16 pools; returns fp32 [B][Hq][D]."""
    return _decode(False, q, k_pool, v_pool, page_table, context_lens, num_kv_heads, page_size,
                   0, softmax_scale, max_context_len, out, workspace, pages_per_split, phase_event)


def paged_decode_attn_int4_noalloc(q, k_pool, v_pool, page_table, context_lens, num_kv_heads: int,
                                   page_size: int, had_block: int, softmax_scale: float,
                                   max_context_len: int, out, pages_per_split: int = 0, phase_event=None):
    """paged_decode_attn_int4 without a workspace: the library's static
    per-GPU scratch holds the partial states, and nothing is allocated (the
    caller passes ``out``, fp32 [B][Hq][D]).  Calls that overlap on one GPU
    race on that scratch."""
    import torch
    B, hq, d = q.shape
    want = (int(num_kv_heads), page_tile_bytes(d, int(page_size)))
    if tuple(k_pool.shape[1:]) != want or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError(f"pools must both be [num_pages]{list(want)}, got {tuple(k_pool.shape)} "
                         f"and {tuple(v_pool.shape)}")
    if context_lens.numel() != B or page_table.dim() != 2 or page_table.shape[0] < B:
        raise ValueError("context_lens must have one entry per sequence and page_table one row each")
    if out is None or tuple(out.shape) != (B, hq, d):
        raise ValueError(f"out must be given, [{B}][{hq}][{d}]")
    _check(lib().paged_decode_attn_int4_noalloc(
        _dev(q, torch.float16, "q", 3), _dev(k_pool, torch.uint8, "k_pool"), _dev(v_pool, torch.uint8, "v_pool"),
        k_pool.shape[0], _dev(page_table, torch.int32, "page_table", 2), page_table.shape[1],
        _dev(context_lens, torch.int32, "context_lens", 1), B, int(max_context_len), hq, int(num_kv_heads), d,
        int(page_size), int(had_block), float(softmax_scale), _dev(out, torch.float32, "out", 3),
        int(pages_per_split), _event_handle(phase_event), _stream(q)), "paged_decode_attn_int4_noalloc")
    return out

"""CPU oracle (ctypes wrapper around ``oracle.c``).

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path never imports this
package, and this package never imports the product package.

Arguments are NumPy arrays in host memory with the same layouts as the HIP
library's device buffers.  Every function raises ``RuntimeError`` when the C
routine reports a bad argument.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add may appear that the written
# arithmetic does not contain.  No -ffast-math, no -march (keeps SSE2 IEEE).
BUILD_CMD = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
             "-fopenmp", "-fPIC", "-shared", _SRC, "-o", _LIB_PATH, "-lm"]


def build() -> str:
    """Compile the oracle library in place and return its path."""
    subprocess.run(BUILD_CMD, check=True)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.kvq_oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.kvq_oracle_f16_to_f32.restype = f32
        L.kvq_oracle_f32_to_f16.argtypes = [f32]
        L.kvq_oracle_f32_to_f16.restype = ctypes.c_uint16
        L.kvq_oracle_hadamard_scale.argtypes = [ctypes.c_int]
        L.kvq_oracle_hadamard_scale.restype = f32
        L.kvq_oracle_fwht_f32.argtypes = [P, ctypes.c_int, ctypes.c_int]
        L.kvq_oracle_fwht_f32.restype = None
        L.kvq_oracle_rotate_f64.argtypes = [P, ctypes.c_int, ctypes.c_int]
        L.kvq_oracle_rotate_f64.restype = None
        L.kvq_oracle_quantize_vector.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P]
        L.kvq_oracle_quantize_vector.restype = ctypes.c_int
        L.kvq_oracle_tile_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        L.kvq_oracle_tile_bytes.restype = i64
        L.kvq_oracle_kv_quant_append.argtypes = [P, P, P, P, i32, P, i32, P, P, i64, i32, i32, i32, i32]
        L.kvq_oracle_kv_quant_append.restype = ctypes.c_int
        L.kvq_oracle_kv_append_fp16.argtypes = [P, P, P, P, i32, P, i32, P, P, i64, i32, i32, i32]
        L.kvq_oracle_kv_append_fp16.restype = ctypes.c_int
        L.kvq_oracle_paged_decode_attn_int4.argtypes = [P, P, P, i64, P, i32, P, i32, i32, i32, i32, i32, i32, f32, P]
        L.kvq_oracle_paged_decode_attn_int4.restype = ctypes.c_int
        L.kvq_oracle_paged_decode_attn_fp16.argtypes = [P, P, P, i64, P, i32, P, i32, i32, i32, i32, i32, f32, P]
        L.kvq_oracle_paged_decode_attn_fp16.restype = ctypes.c_int
        L.kvq_oracle_dense_decode_f64.argtypes = [P, P, P, i32, i32, i32, i32, f64, P]
        L.kvq_oracle_dense_decode_f64.restype = ctypes.c_int
        L.kvq_oracle_tile_bytes_cfg.argtypes = [ctypes.c_int, ctypes.c_int, P]
        L.kvq_oracle_tile_bytes_cfg.restype = i64
        L.kvq_oracle_quantize_vector_cfg.argtypes = [P, ctypes.c_int, P, P, P]
        L.kvq_oracle_quantize_vector_cfg.restype = ctypes.c_int
        L.kvq_oracle_reconstruct_cfg.argtypes = [P, ctypes.c_int, P, P]
        L.kvq_oracle_reconstruct_cfg.restype = ctypes.c_int
        L.kvq_oracle_kv_quant_append_cfg.argtypes = [P, P, P, P, i32, P, i32, P, P, i64, i32, i32, i32, P]
        L.kvq_oracle_kv_quant_append_cfg.restype = ctypes.c_int
        L.kvq_oracle_paged_decode_attn_cfg.argtypes = [P, P, P, i64, P, i32, P, i32, i32, i32, i32, i32, P, f32, P]
        L.kvq_oracle_paged_decode_attn_cfg.restype = ctypes.c_int
        L.kvq_oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.kvq_oracle_e2m1_value.restype = f32
        L.kvq_oracle_num_threads.argtypes = []
        L.kvq_oracle_num_threads.restype = ctypes.c_int
        L.kvq_oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.kvq_oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle {what} rejected its arguments (rc={rc})")


def _as(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def num_threads() -> int:
    return lib().kvq_oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only; results do not
    depend on it)."""
    lib().kvq_oracle_set_num_threads(int(n))


def f16_bits_to_f32(h: int) -> float:
    return lib().kvq_oracle_f16_to_f32(int(h))


def f32_to_f16_bits(x: float) -> int:
    return lib().kvq_oracle_f32_to_f16(float(np.float32(x)))


def hadamard_scale(bh: int) -> np.float32:
    return np.float32(lib().kvq_oracle_hadamard_scale(int(bh)))


def fwht_f32(y, bh: int) -> np.ndarray:
    """Unnormalised block FWHT of a float32 vector (returns a copy)."""
    a = _as(y, np.float32).copy()
    lib().kvq_oracle_fwht_f32(_ptr(a), a.size, int(bh))
    return a


def rotate_f64(x, bh: int) -> np.ndarray:
    """R.x in fp64 (block FWHT divided by sqrt(Bh)) on the last axis."""
    a = _as(x, np.float64).copy()
    d = a.shape[-1]
    flat = a.reshape(-1, d)
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        lib().kvq_oracle_rotate_f64(_ptr(row), d, int(bh))
        flat[r] = row
    return flat.reshape(a.shape)


def quantize_vector(x_f16, bh: int):
    """One vector of fp16 values -> (packed uint8 codes [D/2], fp16 scale bits)."""
    x = _as(x_f16, np.float16).view(np.uint16)
    d = x.size
    codes = np.zeros(d // 2, np.uint8)
    scale = np.zeros(1, np.uint16)
    _check(lib().kvq_oracle_quantize_vector(_ptr(x), d, int(bh), _ptr(codes), _ptr(scale)),
           "quantize_vector")
    return codes, int(scale[0])


def tile_bytes(head_dim: int, page_size: int) -> int:
    return int(lib().kvq_oracle_tile_bytes(head_dim, page_size))


def kv_quant_append(k_new, v_new, token_seq, token_pos, page_table, k_pool, v_pool,
                    had_block: int, page_size: int) -> None:
    """In-place append into uint8 pools [num_pages][Hkv][tile] (Hkv * tile bytes
    per page: the code rows of every head, then every head's scales)."""
    k = _as(k_new, np.float16).view(np.uint16)
    v = _as(v_new, np.float16).view(np.uint16)
    T, hkv, d = k.shape
    ts, tp = _as(token_seq, np.int32), _as(token_pos, np.int32)
    pt = _as(page_table, np.int32)
    assert k_pool.dtype == np.uint8 and v_pool.dtype == np.uint8
    num_pages = k_pool.shape[0]
    _check(lib().kvq_oracle_kv_quant_append(_ptr(k), _ptr(v), _ptr(ts), _ptr(tp), T, _ptr(pt),
                                            pt.shape[1], _ptr(k_pool), _ptr(v_pool), num_pages,
                                            hkv, d, int(page_size), int(had_block)),
           "kv_quant_append")


def kv_append_fp16(k_new, v_new, token_seq, token_pos, page_table, k_pool, v_pool,
                   page_size: int) -> None:
    """In-place copy into fp16 pools [num_pages][Hkv][P][D]."""
    k = _as(k_new, np.float16).view(np.uint16)
    v = _as(v_new, np.float16).view(np.uint16)
    T, hkv, d = k.shape
    ts, tp = _as(token_seq, np.int32), _as(token_pos, np.int32)
    pt = _as(page_table, np.int32)
    assert k_pool.dtype == np.float16 and v_pool.dtype == np.float16
    _check(lib().kvq_oracle_kv_append_fp16(_ptr(k), _ptr(v), _ptr(ts), _ptr(tp), T, _ptr(pt),
                                           pt.shape[1], _ptr(k_pool), _ptr(v_pool),
                                           k_pool.shape[0], hkv, d, int(page_size)),
           "kv_append_fp16")


def paged_decode_attn_int4(q, k_pool, v_pool, page_table, context_lens, num_kv_heads: int,
                           page_size: int, had_block: int, softmax_scale: float) -> np.ndarray:
    qq = _as(q, np.float16).view(np.uint16)
    B, hq, d = qq.shape
    pt, cl = _as(page_table, np.int32), _as(context_lens, np.int32)
    out = np.zeros((B, hq, d), np.float32)
    _check(lib().kvq_oracle_paged_decode_attn_int4(_ptr(qq), _ptr(k_pool), _ptr(v_pool),
                                                   k_pool.shape[0], _ptr(pt), pt.shape[1],
                                                   _ptr(cl), B, hq, int(num_kv_heads), d,
                                                   int(page_size), int(had_block),
                                                   float(softmax_scale), _ptr(out)),
           "paged_decode_attn_int4")
    return out


def paged_decode_attn_fp16(q, k_pool, v_pool, page_table, context_lens, num_kv_heads: int,
                           page_size: int, softmax_scale: float) -> np.ndarray:
    qq = _as(q, np.float16).view(np.uint16)
    B, hq, d = qq.shape
    pt, cl = _as(page_table, np.int32), _as(context_lens, np.int32)
    kp = np.ascontiguousarray(k_pool).view(np.uint16)
    vp = np.ascontiguousarray(v_pool).view(np.uint16)
    out = np.zeros((B, hq, d), np.float32)
    _check(lib().kvq_oracle_paged_decode_attn_fp16(_ptr(qq), _ptr(kp), _ptr(vp), kp.shape[0],
                                                   _ptr(pt), pt.shape[1], _ptr(cl), B, hq,
                                                   int(num_kv_heads), d, int(page_size),
                                                   float(softmax_scale), _ptr(out)),
           "paged_decode_attn_fp16")
    return out


def dense_decode_f64(q, k, v, softmax_scale: float) -> np.ndarray:
    """q [Hq][D], k/v [L][Hkv][D] (any real dtype) -> fp64 [Hq][D]."""
    qq = _as(q, np.float64)
    kk, vv = _as(k, np.float64), _as(v, np.float64)
    hq, d = qq.shape
    L, hkv, _ = kk.shape
    out = np.zeros((hq, d), np.float64)
    _check(lib().kvq_oracle_dense_decode_f64(_ptr(qq), _ptr(kk), _ptr(vv), L, hq, hkv, d,
                                             float(softmax_scale), _ptr(out)),
           "dense_decode_f64")
    return out


def dequantize_pool(pool: np.ndarray, page_table, context_len: int, seq: int, head: int,
                    head_dim: int, page_size: int) -> np.ndarray:
    """Read back the dequantized (still rotated) vectors of one (sequence, KV head)
    by decoding the stored nibbles and scales: float64 [L][D]."""
    pt = _as(page_table, np.int32)
    out = np.zeros((context_len, head_dim), np.float64)
    half = head_dim // 2
    hkv = pool.shape[1]
    for j in range(context_len):
        page = int(pt[seq, j // page_size])
        slot = j % page_size
        pg = pool[page].reshape(-1)       # codes of heads 0..hkv-1, then their scales
        c0 = (head * page_size + slot) * half
        row = pg[c0:c0 + half]
        lo = (row & 0xF).astype(np.int32)
        hi = (row >> 4).astype(np.int32)
        codes = np.empty(head_dim, np.int32)
        codes[0::2] = np.where(lo >= 8, lo - 16, lo)
        codes[1::2] = np.where(hi >= 8, hi - 16, hi)
        s0 = hkv * page_size * half + (head * page_size + slot) * 2
        sb = pg[s0:s0 + 2]
        s = float(np.frombuffer(bytes(sb), dtype="<f2")[0])
        out[j] = codes * s
    return out


# --------------------------------------------------------------------------
# Quantizer variants (per-group scales, scale search, randomized Hadamard,
# MXFP4).  A configuration is (format, had_block, scale_group, scale_search,
# sign_mask): format 0 = INT4 codes with fp16 scales, 1 = MXFP4 (E2M1 codes,
# E8M0 scales, groups of 32); sign_mask is a 128-bit integer (bit i: channel
# i negated before the rotation).
FMT_INT4 = 0
FMT_MXFP4 = 1


class QCfg(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("had_block", ctypes.c_int32), ("scale_group", ctypes.c_int32),
                ("scale_search", ctypes.c_int32), ("sign_mask", ctypes.c_uint32 * 4)]


def qcfg(fmt: int = FMT_INT4, had_block: int = 0, scale_group: int = 128, scale_search: int = 0,
         sign_mask: int = 0) -> QCfg:
    c = QCfg()
    c.format, c.had_block, c.scale_group, c.scale_search = int(fmt), int(had_block), int(scale_group), \
        int(scale_search)
    for w in range(4):
        c.sign_mask[w] = (int(sign_mask) >> (32 * w)) & 0xFFFFFFFF
    return c


def scale_bytes_per_vector(cfg: QCfg, head_dim: int = 128) -> int:
    return (head_dim // cfg.scale_group) * (1 if cfg.format == FMT_MXFP4 else 2)


def tile_bytes_cfg(head_dim: int, page_size: int, cfg: QCfg) -> int:
    n = int(lib().kvq_oracle_tile_bytes_cfg(head_dim, page_size, ctypes.byref(cfg)))
    if n < 0:
        raise RuntimeError("oracle tile_bytes_cfg rejected its arguments")
    return n


def quantize_vector_cfg(x_f16, cfg: QCfg):
    """One vector of fp16 values -> (packed uint8 codes [D/2], scale bytes)."""
    x = _as(x_f16, np.float16).view(np.uint16)
    d = x.size
    codes = np.zeros(d // 2, np.uint8)
    scales = np.zeros(scale_bytes_per_vector(cfg, d), np.uint8)
    _check(lib().kvq_oracle_quantize_vector_cfg(_ptr(x), d, ctypes.byref(cfg), _ptr(codes), _ptr(scales)),
           "quantize_vector_cfg")
    return codes, scales


def reconstruct_cfg(x_f16, cfg: QCfg) -> np.ndarray:
    """Quantize one fp16 vector and bring it back to the original basis (fp64)."""
    x = _as(x_f16, np.float16).view(np.uint16)
    out = np.zeros(x.size, np.float64)
    _check(lib().kvq_oracle_reconstruct_cfg(_ptr(x), x.size, ctypes.byref(cfg), _ptr(out)), "reconstruct_cfg")
    return out


def e2m1_value(code: int) -> float:
    return float(lib().kvq_oracle_e2m1_value(int(code)))


def kv_quant_append_cfg(k_new, v_new, token_seq, token_pos, page_table, k_pool, v_pool, cfg: QCfg,
                        page_size: int) -> None:
    k = _as(k_new, np.float16).view(np.uint16)
    v = _as(v_new, np.float16).view(np.uint16)
    T, hkv, d = k.shape
    ts, tp = _as(token_seq, np.int32), _as(token_pos, np.int32)
    pt = _as(page_table, np.int32)
    assert k_pool.dtype == np.uint8 and v_pool.dtype == np.uint8
    _check(lib().kvq_oracle_kv_quant_append_cfg(_ptr(k), _ptr(v), _ptr(ts), _ptr(tp), T, _ptr(pt), pt.shape[1],
                                                _ptr(k_pool), _ptr(v_pool), k_pool.shape[0], hkv, d,
                                                int(page_size), ctypes.byref(cfg)),
           "kv_quant_append_cfg")


def paged_decode_attn_cfg(q, k_pool, v_pool, page_table, context_lens, num_kv_heads: int, page_size: int,
                          cfg: QCfg, softmax_scale: float) -> np.ndarray:
    qq = _as(q, np.float16).view(np.uint16)
    B, hq, d = qq.shape
    pt, cl = _as(page_table, np.int32), _as(context_lens, np.int32)
    out = np.zeros((B, hq, d), np.float32)
    _check(lib().kvq_oracle_paged_decode_attn_cfg(_ptr(qq), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
                                                  _ptr(pt), pt.shape[1], _ptr(cl), B, hq, int(num_kv_heads), d,
                                                  int(page_size), ctypes.byref(cfg), float(softmax_scale),
                                                  _ptr(out)),
           "paged_decode_attn_cfg")
    return out

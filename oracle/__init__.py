"""ctypes front end of the fp64 CPU oracle (``pa_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this module; the product package never does.  It shares no
code with the GPU library.  Every function takes host numpy arrays holding the exact bytes
the GPU side uses (bf16 and fp16 tensors as ``uint16`` bit patterns, fp32 as ``float32``) and
returns fp64 results.

Citations for what each function computes live in the header comment of ``pa_oracle.c``
(aphrodite-engine "xformers.py" and vLLM "cpu_attn" pages of the reference).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "libpa_oracle.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_F16 = 2
KV_CACHE_AUTO = 0        # the cache holds elements of the layer dtype
KV_CACHE_FP8_E4M3 = 1    # the cache holds FP8 E4M3 codes (uint8), scaled by k_scale / v_scale


def build(force: bool = True) -> str:
    """Compile ``pa_oracle.c`` into ``libpa_oracle.so`` with gcc (plain -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Layer(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("alibi_slopes", ctypes.c_void_p),
        ("sliding_window", ctypes.c_int32),
        ("logits_soft_cap", ctypes.c_float),
        ("sinks", ctypes.c_void_p),
        ("kv_cache_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.orc_cache_write.argtypes = [ctypes.POINTER(_Layer), P, P, ctypes.c_int64, ctypes.c_int64, P, P]
        lib.orc_cache_write.restype = ctypes.c_int
        lib.orc_decode.argtypes = [ctypes.POINTER(_Layer), P, P, ctypes.c_int64, P, P, ctypes.c_int32,
                                   P, ctypes.c_int32, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        lib.orc_decode.restype = ctypes.c_int
        lib.orc_decode_multi.argtypes = [ctypes.POINTER(_Layer), P, P, ctypes.c_int64, P, P, ctypes.c_int32,
                                         P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        lib.orc_decode_multi.restype = ctypes.c_int
        lib.orc_prefill.argtypes = [ctypes.POINTER(_Layer), P, P, ctypes.c_int64, P, P, ctypes.c_int64, P,
                                    P, ctypes.c_int32, P, P, ctypes.c_int32, P, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_int)]
        lib.orc_prefill.restype = ctypes.c_int
        lib.orc_copy_blocks.argtypes = [ctypes.POINTER(_Layer), P, ctypes.c_int32, P, ctypes.c_int64]
        lib.orc_copy_blocks.restype = ctypes.c_int
        lib.orc_swap_blocks.argtypes = [ctypes.POINTER(_Layer), P, ctypes.c_int64, P, ctypes.c_int64, P,
                                        ctypes.c_int64]
        lib.orc_swap_blocks.restype = ctypes.c_int
        _lib = lib
    return _lib


@dataclass
class OracleLayer:
    """Geometry of one attention layer, as the oracle needs it."""
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    dtype: int                       # DTYPE_F32, DTYPE_BF16 or DTYPE_F16
    scale: float
    alibi_slopes: Optional[np.ndarray] = None   # float32 [num_heads]
    sliding_window: int = 0
    logits_soft_cap: float = 0.0               # <= 0: off
    sinks: Optional[np.ndarray] = None          # float32 [num_heads] sink logits
    kv_cache_dtype: int = KV_CACHE_AUTO
    k_scale: float = 1.0                        # fp8 cache scales (fp32)
    v_scale: float = 1.0

    def _c(self):
        def f32_heads(a):
            if a is None:
                return None
            a = np.ascontiguousarray(a, dtype=np.float32)
            assert a.shape == (self.num_heads,)
            return a
        slopes, sinks = f32_heads(self.alibi_slopes), f32_heads(self.sinks)
        c = _Layer(self.num_heads, self.num_kv_heads, self.head_size, self.block_size,
                   self.num_blocks, self.dtype, float(np.float32(self.scale)),
                   slopes.ctypes.data if slopes is not None else None,
                   int(self.sliding_window), float(np.float32(self.logits_soft_cap)),
                   sinks.ctypes.data if sinks is not None else None, int(self.kv_cache_dtype),
                   float(np.float32(self.k_scale)), float(np.float32(self.v_scale)))
        return c, (slopes, sinks)   # keep the arrays alive while c is used


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _check(status: int, what: str):
    if status != 0:
        raise RuntimeError(f"oracle {what} failed with status {status}")


def _elt_dtype(layer: OracleLayer):
    return np.float32 if layer.dtype == DTYPE_F32 else np.uint16


def cache_dtype(layer: OracleLayer):
    """numpy dtype of the paged cache's elements (uint8 codes for an fp8 cache)."""
    return np.uint8 if layer.kv_cache_dtype == KV_CACHE_FP8_E4M3 else _elt_dtype(layer)


def cache_write(layer: OracleLayer, key: np.ndarray, value: np.ndarray, slot_mapping: np.ndarray,
                kv_cache: np.ndarray) -> None:
    """In place: scatter key/value rows [T, Hkv*D] into kv_cache through slot_mapping."""
    et = _elt_dtype(layer)
    assert key.dtype == et and value.dtype == et and kv_cache.dtype == cache_dtype(layer)
    assert key.shape == value.shape and key.ndim == 2
    if key.shape[0] == 0:
        return
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    assert kv_cache.flags.c_contiguous
    slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    assert slot_mapping.shape == (key.shape[0],)
    c, keep = layer._c()
    st = _load().orc_cache_write(ctypes.byref(c), _ptr(key), _ptr(value), key.shape[1],
                                 key.shape[0], _ptr(slot_mapping), _ptr(kv_cache))
    _check(st, "cache_write")


def copy_blocks(layer: OracleLayer, kv_caches, block_pairs: np.ndarray) -> None:
    """In place, every cache of the list: block src -> block dst for each (src, dst) pair
    (both planes; pairs outside [0, num_blocks) skipped; applied in order)."""
    et = cache_dtype(layer)
    pairs = np.ascontiguousarray(block_pairs, dtype=np.int64).reshape(-1, 2)
    for c in kv_caches:
        assert c.dtype == et and c.flags.c_contiguous
    ptrs = (ctypes.c_void_p * max(1, len(kv_caches)))(*[c.ctypes.data for c in kv_caches])
    c, keep = layer._c()
    st = _load().orc_copy_blocks(ctypes.byref(c), ptrs, len(kv_caches), _ptr(pairs), pairs.shape[0])
    _check(st, "copy_blocks")


def swap_blocks(layer: OracleLayer, src_cache: np.ndarray, dst_cache: np.ndarray, block_pairs: np.ndarray) -> None:
    """In place: block src of src_cache -> block dst of dst_cache, both planes, for each pair.
    The caches are [2, n_blocks, block elements] with their own block counts."""
    et = cache_dtype(layer)
    assert src_cache.dtype == et and dst_cache.dtype == et and dst_cache.flags.c_contiguous
    src_cache = np.ascontiguousarray(src_cache)
    pairs = np.ascontiguousarray(block_pairs, dtype=np.int64).reshape(-1, 2)
    c, keep = layer._c()
    st = _load().orc_swap_blocks(ctypes.byref(c), _ptr(src_cache), src_cache.shape[1], _ptr(dst_cache),
                                 dst_cache.shape[1], _ptr(pairs), pairs.shape[0])
    _check(st, "swap_blocks")


def decode(layer: OracleLayer, query: np.ndarray, kv_cache: np.ndarray, block_tables: np.ndarray,
           seq_lens: np.ndarray, num_threads: int = 0, return_threads: bool = False):
    """fp64 [B, H, D] decode output (see ``orc_decode`` in pa_oracle.c)."""
    et = _elt_dtype(layer)
    assert query.dtype == et and kv_cache.dtype == cache_dtype(layer) and kv_cache.flags.c_contiguous
    assert query.ndim == 2
    query = np.ascontiguousarray(query)
    B = query.shape[0]
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    assert block_tables.ndim == 2 and block_tables.shape[0] == B and seq_lens.shape == (B,)
    out = np.empty((B, layer.num_heads, layer.head_size), dtype=np.float64)
    c, keep = layer._c()
    used = ctypes.c_int(0)
    st = _load().orc_decode(ctypes.byref(c), _ptr(out), _ptr(query), query.shape[1],
                            _ptr(kv_cache), _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), B,
                            num_threads, ctypes.byref(used))
    _check(st, "decode")
    return (out, used.value) if return_threads else out


def decode_multi(layer: OracleLayer, query: np.ndarray, kv_cache: np.ndarray, block_tables: np.ndarray,
                 seq_lens: np.ndarray, query_len: int, num_threads: int = 0):
    """fp64 [B * query_len, H, D] multi-token decode output (see ``orc_decode_multi``)."""
    et = _elt_dtype(layer)
    assert query.dtype == et and kv_cache.dtype == cache_dtype(layer) and kv_cache.flags.c_contiguous
    query = np.ascontiguousarray(query)
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = seq_lens.shape[0]
    assert query.shape[0] == B * query_len and block_tables.shape[0] == B
    out = np.empty((B * query_len, layer.num_heads, layer.head_size), dtype=np.float64)
    c, keep = layer._c()
    used = ctypes.c_int(0)
    st = _load().orc_decode_multi(ctypes.byref(c), _ptr(out), _ptr(query), query.shape[1], _ptr(kv_cache),
                                  _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), B, int(query_len),
                                  num_threads, ctypes.byref(used))
    _check(st, "decode_multi")
    return out


def prefill(layer: OracleLayer, query: np.ndarray, key: np.ndarray, value: np.ndarray,
            kv_cache: Optional[np.ndarray], block_tables: Optional[np.ndarray],
            context_lens: Optional[np.ndarray], cu_subquery: np.ndarray,
            row_select: Optional[np.ndarray] = None, num_threads: int = 0,
            return_threads: bool = False):
    """fp64 [T, H, D] prefill output (see ``orc_prefill`` in pa_oracle.c).

    Rows not selected by ``row_select`` (bool [T]) are returned as NaN.
    """
    et = _elt_dtype(layer)
    assert query.dtype == et and key.dtype == et and value.dtype == et
    assert query.ndim == 2 and key.ndim == 2 and key.shape == value.shape
    query = np.ascontiguousarray(query)
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    T = query.shape[0]
    assert key.shape[0] == T
    cu = np.ascontiguousarray(cu_subquery, dtype=np.int32)
    N = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == T
    if context_lens is not None:
        context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
        assert context_lens.shape == (N,)
    maxb = 0
    if block_tables is not None:
        block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
        assert block_tables.ndim == 2 and block_tables.shape[0] == N
        maxb = block_tables.shape[1]
    if kv_cache is not None:
        assert kv_cache.dtype == cache_dtype(layer) and kv_cache.flags.c_contiguous
    sel = None
    if row_select is not None:
        sel = np.ascontiguousarray(row_select, dtype=np.uint8)
        assert sel.shape == (T,)
    out = np.full((T, layer.num_heads, layer.head_size), np.nan, dtype=np.float64)
    c, keep = layer._c()
    used = ctypes.c_int(0)
    st = _load().orc_prefill(ctypes.byref(c), _ptr(out), _ptr(query), query.shape[1],
                             _ptr(key), _ptr(value), key.shape[1], _ptr(kv_cache),
                             _ptr(block_tables), maxb, _ptr(context_lens), _ptr(cu), N, _ptr(sel),
                             num_threads, ctypes.byref(used))
    _check(st, "prefill")
    return (out, used.value) if return_threads else out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of IEEE binary16 bit patterns (uint16) as float64."""
    b = bits.astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 31
    f = (b & 1023).astype(np.float64)
    v = np.where(e == 0, np.ldexp(f, -24), np.ldexp(1024.0 + f, (e - 25).astype(np.int32)))
    v = np.where(e == 31, np.where(f != 0, np.nan, np.inf), v)
    return sign * v


def bits_to_f64(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Exact value of stored elements of the given oracle dtype as float64."""
    if dtype == DTYPE_F32:
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    return f16_bits_to_f64(bits) if dtype == DTYPE_F16 else bf16_bits_to_f64(bits)

"""Python binding of libpa: attention over a paged KV cache on AMD MI355X (gfx950).

Argument marshalling only.  Every function takes torch tensors that already live on the GPU,
checks shapes and dtypes, and hands raw device pointers, sizes and torch's current HIP stream
to the C ABI declared in ``include/pa.h``; all computation happens in libpa's HIP kernels.
torch supplies device memory (outputs and the decode workspace are allocated with torch when
the caller does not pass them) and streams, nothing else.  There is no CPU path: importing
this package without a built ``libpa.so`` raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARGUMENT = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_WORKSPACE = 3
PA_ERR_HIP = 4

PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
PA_DTYPE_F16 = 2
PA_KV_CACHE_AUTO = 0
PA_KV_CACHE_FP8_E4M3 = 1

EXPORTED = ("pa_cache_write", "pa_decode", "pa_decode_workspace_size", "pa_decode_noalloc", "pa_decode_multi",
            "pa_decode_multi_workspace_size",
            "pa_prefill_varlen", "pa_copy_blocks", "pa_swap_blocks", "pa_status_string", "pa_last_error_message",
            "pa_version")


class PaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class _CLayer(ctypes.Structure):
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


def _load_library(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"libpa.so is not built ({path} missing); run `python -m paged_kv_cache_242_amd.build` "
                          "or __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    LP = ctypes.POINTER(_CLayer)
    lib.pa_cache_write.argtypes = [LP, P, P, I64, I64, P, P, P]
    lib.pa_cache_write.restype = ctypes.c_int
    lib.pa_decode_workspace_size.argtypes = [LP, I32, I32]
    lib.pa_decode_workspace_size.restype = SZ
    lib.pa_decode.argtypes = [LP, P, P, I64, P, P, I32, P, I32, I32, P, SZ, P]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [LP, P, P, I64, P, P, I32, P, I32, I32, P]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_multi_workspace_size.argtypes = [LP, I32, I32, I32]
    lib.pa_decode_multi_workspace_size.restype = SZ
    lib.pa_decode_multi.argtypes = [LP, P, P, I64, P, P, I32, P, I32, I32, I32, P, SZ, P]
    lib.pa_decode_multi.restype = ctypes.c_int
    lib.pa_prefill_varlen.argtypes = [LP, P, P, I64, P, P, I64, P, P, I32, P, P, I32, I64, I32, I32, P]
    lib.pa_prefill_varlen.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [LP, P, I32, P, I64, P]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_swap_blocks.argtypes = [LP, P, I64, P, I64, P, I64, P]
    lib.pa_swap_blocks.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error_message.argtypes = []
    lib.pa_last_error_message.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_char_p
    return lib


_lib = _load_library()


def library() -> ctypes.CDLL:
    return _lib


def version() -> str:
    return _lib.pa_version().decode()


def _check(status: int):
    if status != PA_OK:
        name = _lib.pa_status_string(status).decode()
        raise PaError(status, f"{name}: {_lib.pa_last_error_message().decode()}")


@dataclass
class Layer:
    """Geometry of one attention layer (mirrors ``pa_layer``)."""
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    dtype: torch.dtype                               # torch.float32, torch.bfloat16 or torch.float16
    scale: float
    alibi_slopes: Optional[torch.Tensor] = None      # fp32 [num_heads] on the GPU
    sliding_window: int = 0                          # <= 0: off
    logits_soft_cap: float = 0.0                     # <= 0: off
    sinks: Optional[torch.Tensor] = None             # fp32 [num_heads] sink logits on the GPU
    kv_cache_dtype: str = "auto"                     # "auto" (the layer dtype) or "fp8_e4m3"
    k_scale: float = 1.0                             # fp8 cache scales
    v_scale: float = 1.0

    @property
    def cache_dtype(self) -> torch.dtype:
        """torch dtype of the paged cache tensor (uint8 codes for an fp8 cache)."""
        return torch.uint8 if self.kv_cache_dtype == "fp8_e4m3" else self.dtype

    def _c(self) -> _CLayer:
        dt = {torch.float32: PA_DTYPE_F32, torch.bfloat16: PA_DTYPE_BF16, torch.float16: PA_DTYPE_F16}.get(self.dtype)
        if dt is None:
            raise PaError(PA_ERR_UNSUPPORTED, f"dtype {self.dtype} is not supported (float32, bfloat16, float16)")
        def heads_ptr(t, name):
            if t is None:
                return None
            if t.dtype != torch.float32 or not t.is_cuda or t.numel() != self.num_heads or not t.is_contiguous():
                raise PaError(PA_ERR_INVALID_ARGUMENT, f"{name} must be a contiguous fp32 GPU tensor [num_heads]")
            return t.data_ptr()
        kvd = {"auto": PA_KV_CACHE_AUTO, "fp8_e4m3": PA_KV_CACHE_FP8_E4M3}.get(self.kv_cache_dtype)
        if kvd is None:
            raise PaError(PA_ERR_UNSUPPORTED, f"kv_cache_dtype {self.kv_cache_dtype!r} is not supported "
                                              "('auto', 'fp8_e4m3')")
        return _CLayer(self.num_heads, self.num_kv_heads, self.head_size, self.block_size, self.num_blocks, dt,
                       float(self.scale), heads_ptr(self.alibi_slopes, "alibi_slopes"), int(self.sliding_window or 0),
                       float(self.logits_soft_cap or 0.0), heads_ptr(self.sinks, "sinks"), kvd,
                       float(self.k_scale), float(self.v_scale))


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _rows(t: torch.Tensor, name: str, width: int, dtype: torch.dtype) -> int:
    """Validate a [rows, >= width] GPU tensor with unit inner stride; return its row stride."""
    if not t.is_cuda:
        raise PaError(PA_ERR_INVALID_ARGUMENT, f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise PaError(PA_ERR_INVALID_ARGUMENT, f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.dim() != 2 or t.shape[1] != width or (t.shape[1] > 1 and t.stride(1) != 1):
        raise PaError(PA_ERR_INVALID_ARGUMENT, f"{name} must be [rows, {width}] with unit inner stride, got "
                                               f"{tuple(t.shape)} strides {t.stride()}")
    return t.stride(0) if t.shape[0] > 1 else width


def _index(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape=None):
    if t is None:
        return None
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise PaError(PA_ERR_INVALID_ARGUMENT, f"{name} must be a contiguous {dtype} GPU tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise PaError(PA_ERR_INVALID_ARGUMENT, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _cache(kv_cache: torch.Tensor, layer: Layer):
    want = (2, layer.num_blocks, layer.block_size * layer.num_kv_heads * layer.head_size)
    if tuple(kv_cache.shape) != want or not kv_cache.is_contiguous() or kv_cache.dtype != layer.cache_dtype \
            or not kv_cache.is_cuda:
        raise PaError(PA_ERR_INVALID_ARGUMENT, f"kv_cache must be a contiguous {layer.cache_dtype} GPU tensor {want}, "
                                               f"got {tuple(kv_cache.shape)} {kv_cache.dtype}")
    return kv_cache.data_ptr()


def cache_write(key: torch.Tensor, value: torch.Tensor, kv_cache: torch.Tensor, slot_mapping: torch.Tensor,
                layer: Layer) -> None:
    """Scatter key/value rows [T, Hkv*D] into ``kv_cache`` at ``slot_mapping`` (int64 [T]); in place."""
    width = layer.num_kv_heads * layer.head_size
    ks = _rows(key, "key", width, layer.dtype)
    vs = _rows(value, "value", width, layer.dtype)
    if ks != vs and key.shape[0] > 1:
        raise PaError(PA_ERR_INVALID_ARGUMENT, "key and value must share a row stride")
    T = key.shape[0]
    if value.shape[0] != T:
        raise PaError(PA_ERR_INVALID_ARGUMENT, "key and value row counts differ")
    sm = _index(slot_mapping, "slot_mapping", torch.int64, (T,))
    c = layer._c()
    _check(_lib.pa_cache_write(ctypes.byref(c), key.data_ptr(), value.data_ptr(), ks, T, sm,
                               _cache(kv_cache, layer), _stream(key.device)))


def copy_blocks(kv_caches, block_pairs: torch.Tensor, layer: Layer) -> None:
    """Copy block src -> dst (both planes) in every cache of ``kv_caches`` for each row
    (src, dst) of ``block_pairs`` (int64 [n, 2] on the GPU); in place, one launch."""
    caches = list(kv_caches)
    if not caches:
        return
    ptrs = [_cache(c, layer) for c in caches]
    pairs = _index(block_pairs, "block_pairs", torch.int64)
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise PaError(PA_ERR_INVALID_ARGUMENT, f"block_pairs must be [n, 2], got {tuple(block_pairs.shape)}")
    dev = caches[0].device
    table = torch.tensor(ptrs, dtype=torch.int64, device=dev)     # device array of cache pointers
    c = layer._c()
    _check(_lib.pa_copy_blocks(ctypes.byref(c), table.data_ptr(), len(caches), pairs, block_pairs.shape[0],
                               _stream(dev)))


def swap_blocks(src_cache: torch.Tensor, dst_cache: torch.Tensor, block_pairs, layer: Layer) -> None:
    """Copy block src of ``src_cache`` -> block dst of ``dst_cache`` (both planes) for each pair
    (src, dst) of ``block_pairs`` (host int64 [n, 2]: a CPU tensor, array or list).  Either cache
    may live in (pinned) host memory; the copies go on the current stream of the GPU side."""
    elems = layer.block_size * layer.num_kv_heads * layer.head_size
    for name, t in (("src_cache", src_cache), ("dst_cache", dst_cache)):
        if t.dim() != 3 or t.shape[0] != 2 or t.shape[2] != elems or not t.is_contiguous() or \
                t.dtype != layer.cache_dtype:
            raise PaError(PA_ERR_INVALID_ARGUMENT,
                          f"{name} must be a contiguous {layer.cache_dtype} tensor [2, blocks, {elems}]")
    pairs = torch.as_tensor(block_pairs, dtype=torch.int64).reshape(-1, 2).contiguous()
    if pairs.is_cuda:
        raise PaError(PA_ERR_INVALID_ARGUMENT, "block_pairs must be on the host")
    dev = src_cache.device if src_cache.is_cuda else dst_cache.device
    if not dev.type == "cuda":
        raise PaError(PA_ERR_INVALID_ARGUMENT, "one of the caches must be a GPU tensor")
    c = layer._c()
    _check(_lib.pa_swap_blocks(ctypes.byref(c), src_cache.data_ptr(), src_cache.shape[1], dst_cache.data_ptr(),
                               dst_cache.shape[1], pairs.data_ptr(), pairs.shape[0], _stream(dev)))


def decode_workspace_size(layer: Layer, num_seqs: int, max_seq_len: int, query_len: int = 1,
                          _clayer: Optional[_CLayer] = None) -> int:
    c = _clayer if _clayer is not None else layer._c()
    if query_len == 1:
        return int(_lib.pa_decode_workspace_size(ctypes.byref(c), num_seqs, max_seq_len))
    return int(_lib.pa_decode_multi_workspace_size(ctypes.byref(c), num_seqs, query_len, max_seq_len))


def decode(query: torch.Tensor, kv_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
           layer: Layer, max_seq_len: int, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, query_len: int = 1) -> torch.Tensor:
    """Decode: query [B * query_len, H*D] -> out [B * query_len, H*D] for B = len(seq_lens) sequences
    (query_len > 1: multi-token decode through pa_decode_multi)."""
    width = layer.num_heads * layer.head_size
    qs = _rows(query, "query", width, layer.dtype)
    B = seq_lens.numel()
    if query.shape[0] != B * query_len:
        raise PaError(PA_ERR_INVALID_ARGUMENT, f"query has {query.shape[0]} rows, expected {B} * {query_len}")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise PaError(PA_ERR_INVALID_ARGUMENT, "block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    bt = _index(block_tables, "block_tables", torch.int32)
    sl = _index(seq_lens, "seq_lens", torch.int32, (B,))
    rows = B * query_len
    if out is None:
        out = torch.empty((rows, width), dtype=layer.dtype, device=query.device)
    elif tuple(out.shape) != (rows, width) or not out.is_contiguous() or out.dtype != layer.dtype:
        raise PaError(PA_ERR_INVALID_ARGUMENT, "out must be a contiguous [rows, H*D] tensor of the layer dtype")
    c = layer._c()
    ws_ptr, ws_bytes = None, 0
    if workspace is None:
        # (a workspace passed in is checked against the need by the library itself)
        need = decode_workspace_size(layer, B, max_seq_len, query_len, c) if B > 0 else 0
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if query_len == 1:
        _check(_lib.pa_decode(ctypes.byref(c), out.data_ptr(), query.data_ptr(), qs, _cache(kv_cache, layer), bt,
                              block_tables.shape[1], sl, B, int(max_seq_len), ws_ptr, ws_bytes,
                              _stream(query.device)))
    else:
        _check(_lib.pa_decode_multi(ctypes.byref(c), out.data_ptr(), query.data_ptr(), qs, _cache(kv_cache, layer),
                                    bt, block_tables.shape[1], sl, B, int(query_len), int(max_seq_len), ws_ptr,
                                    ws_bytes, _stream(query.device)))
    return out


def decode_noalloc(query: torch.Tensor, kv_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                   layer: Layer, max_seq_len: int, out: torch.Tensor) -> torch.Tensor:
    """Decode through pa_decode_noalloc: the library's fixed device scratch array replaces the
    workspace, and ``out`` must be passed (nothing is allocated)."""
    width = layer.num_heads * layer.head_size
    qs = _rows(query, "query", width, layer.dtype)
    B = seq_lens.numel()
    if query.shape[0] != B:
        raise PaError(PA_ERR_INVALID_ARGUMENT, f"query has {query.shape[0]} rows, expected {B}")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise PaError(PA_ERR_INVALID_ARGUMENT, "block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    bt = _index(block_tables, "block_tables", torch.int32)
    sl = _index(seq_lens, "seq_lens", torch.int32, (B,))
    if tuple(out.shape) != (B, width) or not out.is_contiguous() or out.dtype != layer.dtype:
        raise PaError(PA_ERR_INVALID_ARGUMENT, "out must be a contiguous [num_seqs, H*D] tensor of the layer dtype")
    c = layer._c()
    _check(_lib.pa_decode_noalloc(ctypes.byref(c), out.data_ptr(), query.data_ptr(), qs, _cache(kv_cache, layer), bt,
                                  block_tables.shape[1], sl, B, int(max_seq_len), _stream(query.device)))
    return out


def prefill_varlen(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor, kv_cache: Optional[torch.Tensor],
                   block_tables: Optional[torch.Tensor], context_lens: Optional[torch.Tensor],
                   cu_subquery: torch.Tensor, layer: Layer, max_subquery_len: int, max_context_len: int = 0,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Varlen causal prefill over a cached context: query [T, H*D] -> out [T, H*D]."""
    width_q = layer.num_heads * layer.head_size
    width_kv = layer.num_kv_heads * layer.head_size
    qs = _rows(query, "query", width_q, layer.dtype)
    ks = _rows(key, "key", width_kv, layer.dtype)
    vs = _rows(value, "value", width_kv, layer.dtype)
    T = query.shape[0]
    if key.shape[0] != T or value.shape[0] != T:
        raise PaError(PA_ERR_INVALID_ARGUMENT, "query, key and value row counts differ")
    if ks != vs and T > 1:
        raise PaError(PA_ERR_INVALID_ARGUMENT, "key and value must share a row stride")
    N = cu_subquery.numel() - 1
    cu = _index(cu_subquery, "cu_subquery", torch.int32, (N + 1,))
    ctx = _index(context_lens, "context_lens", torch.int32, (N,))
    bt = None
    maxb = 0
    if block_tables is not None:
        if block_tables.dim() != 2 or block_tables.shape[0] != N:
            raise PaError(PA_ERR_INVALID_ARGUMENT, "block_tables must be int32 [num_seqs, max_blocks_per_seq]")
        bt = _index(block_tables, "block_tables", torch.int32)
        maxb = block_tables.shape[1]
    cache = _cache(kv_cache, layer) if kv_cache is not None else None
    if out is None:
        out = torch.empty((T, width_q), dtype=layer.dtype, device=query.device)
    elif tuple(out.shape) != (T, width_q) or not out.is_contiguous() or out.dtype != layer.dtype:
        raise PaError(PA_ERR_INVALID_ARGUMENT, "out must be a contiguous [num_tokens, H*D] tensor of the layer dtype")
    c = layer._c()
    _check(_lib.pa_prefill_varlen(ctypes.byref(c), out.data_ptr(), query.data_ptr(), qs, key.data_ptr(),
                                  value.data_ptr(), ks, cache, bt, maxb, ctx, cu, N, T, int(max_subquery_len),
                                  int(max_context_len), _stream(query.device)))
    return out

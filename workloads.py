"""Seeded synthetic inputs for paged-KV attention.

This module is the only code the GPU path's tests and the fp64 oracle share, and it holds
none of the method's arithmetic: it draws lengths, block tables, slot numbers and N(0, 1)
values, and nothing else.  It never writes into a KV cache and never computes attention.

Shapes follow the problem statement of the reference pages: query [num_tokens,
num_heads * head_size], key/value [num_tokens, num_kv_heads * head_size], the cache
[2, num_blocks, block_size * num_kv_heads * head_size], int32 block tables
[num_seqs, max_blocks_per_seq], int64 slot mapping [num_tokens].  A flattened batch puts
prefill rows first and decode rows after them (aphrodite-engine "xformers.py",
XFormersImpl docstring).

The recipe (also stated in the design notes):
  * integer structure (lengths, permutation of physical blocks) from
    ``numpy.random.default_rng(seed)``;
  * values N(0, 1) from ``torch.Generator`` seeded with ``seed`` on the target device,
    drawn in the layer dtype (fp32, or bf16 / fp16 rounded to nearest even);
  * physical blocks: one random permutation of the pool; each sequence takes the next
    ceil(len / block_size) ids; block-table padding points at a spare block no sequence
    owns (the "poison" block), so a kernel that reads past a sequence's length reads
    never-written cache bytes;
  * slots: token at position p of sequence i goes to slot
    table[i][p // block_size] * block_size + p % block_size;
  * the tokens already cached (positions below the new ones) are returned as context rows
    with their own slots; each side writes them into its own NaN-filled pool.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"
F16 = "f16"


@dataclass
class LayerSpec:
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    dtype: str                                   # F32, BF16 or F16
    scale: float                                 # already rounded to fp32
    alibi_slopes: Optional[np.ndarray] = None    # float32 [num_heads]
    sliding_window: int = 0                      # <= 0: off
    logits_soft_cap: float = 0.0                 # <= 0: off (already rounded to fp32)
    sinks: Optional[np.ndarray] = None           # float32 [num_heads] sink logits
    kv_cache_dtype: str = "auto"                 # "auto" (layer dtype) or "fp8_e4m3"
    k_scale: float = 1.0                         # fp8 cache scales (fp32)
    v_scale: float = 1.0

    @property
    def fp8_cache(self) -> bool:
        return self.kv_cache_dtype == "fp8_e4m3"

    @property
    def torch_dtype(self):
        return {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[self.dtype]

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def row_elems(self) -> int:
        return self.num_kv_heads * self.head_size


@dataclass
class PagedBatch:
    """One flattened batch: prefill sequences first, then decode sequences."""
    layer: LayerSpec
    seed: int
    # prefill part (may be empty)
    prefill_context_lens: np.ndarray          # int32 [Np]
    prefill_query_lens: np.ndarray            # int32 [Np]
    prefill_cu: np.ndarray                    # int32 [Np + 1]
    prefill_block_tables: np.ndarray          # int32 [Np, maxb_p]
    # decode part (may be empty)
    decode_seq_lens: np.ndarray               # int32 [Bd], counts the new token
    decode_block_tables: np.ndarray           # int32 [Bd, maxb_d]
    # new tokens: rows [0, Tp) are prefill rows, rows [Tp, Tp + Bd) decode rows
    query: torch.Tensor                       # [T, H*D]
    key: torch.Tensor                         # [T, Hkv*D]
    value: torch.Tensor                       # [T, Hkv*D]
    slot_mapping: np.ndarray                  # int64 [T]
    # tokens already in the cache before this step
    ctx_key: torch.Tensor                     # [Nc, Hkv*D]
    ctx_value: torch.Tensor                   # [Nc, Hkv*D]
    ctx_slots: np.ndarray                     # int64 [Nc]
    poison_block: int
    used_blocks: int

    @property
    def num_prefill_tokens(self) -> int:
        return int(self.prefill_cu[-1]) if len(self.prefill_cu) else 0

    @property
    def num_decode_tokens(self) -> int:
        return int(len(self.decode_seq_lens))

    @property
    def num_tokens(self) -> int:
        return self.num_prefill_tokens + self.num_decode_tokens


def cumulative_starts(lengths: Sequence[int]) -> np.ndarray:
    """[l0, l1, ...] -> [0, l0, l0 + l1, ...] as int32 (start locations of a flat batch)."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out.astype(np.int32)


def fp32(x: float) -> float:
    return float(np.float32(x))


def alibi_slopes_geometric(num_heads: int) -> np.ndarray:
    """Slopes 2^(-8 (h + 1) / num_heads), rounded to fp32 (the chunked-prefill workload)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / num_heads) for h in range(num_heads)], dtype=np.float32)


def sink_logits(num_heads: int, seed: int) -> np.ndarray:
    """Per-head sink logits, N(0, 2^2) drawn from ``numpy.random.default_rng(seed)``, fp32."""
    return np.random.default_rng(seed).normal(0.0, 2.0, size=num_heads).astype(np.float32)


def _normal(shape: Tuple[int, ...], dtype, device, gen) -> torch.Tensor:
    t = torch.empty(shape, dtype=dtype, device=device)
    if t.numel():
        t.normal_(0.0, 1.0, generator=gen)
    return t


def make_batch(layer: LayerSpec, *, seed: int, prefill: Sequence[Tuple[int, int]] = (),
               decode: Sequence[int] = (), device="cpu", pool_blocks: Optional[int] = None,
               table_width: Optional[int] = None) -> PagedBatch:
    """Draw one batch.

    prefill: (context_len, subquery_len) per prefill sequence.
    decode:  seq_len (including the new token) per decode sequence; each must be >= 1,
             or 0 for a padded row that owns no blocks.
    pool_blocks: physical blocks in the pool (default: exactly enough plus one spare).
    table_width: block-table row width (default: enough for the longest sequence).
    """
    rng = np.random.default_rng([seed, 1])
    bs = layer.block_size
    totals = [c + n for c, n in prefill] + list(decode)
    need = [math.ceil(t / bs) for t in totals]
    used = int(sum(need))
    nb = used + 1 if pool_blocks is None else int(pool_blocks)
    if nb < used + 1:
        raise ValueError(f"pool of {nb} blocks cannot hold {used} used blocks plus a spare")
    perm = rng.permutation(nb).astype(np.int64)
    poison = int(perm[-1])
    layer = dataclasses.replace(layer, num_blocks=nb)

    def tables(part_needs, width):
        width = max(width, 1)
        t = np.full((len(part_needs), width), poison, dtype=np.int32)
        return t

    p_need = need[:len(prefill)]
    d_need = need[len(prefill):]
    wp = table_width if table_width is not None else max(p_need, default=0)
    wd = table_width if table_width is not None else max(d_need, default=0)
    if table_width is not None and max(need, default=0) > table_width:
        raise ValueError("table_width smaller than the longest sequence")
    ptab = tables(p_need, wp)
    dtab = tables(d_need, wd)
    cursor = 0
    for i, k in enumerate(p_need):
        ptab[i, :k] = perm[cursor:cursor + k]
        cursor += k
    for i, k in enumerate(d_need):
        dtab[i, :k] = perm[cursor:cursor + k]
        cursor += k

    def slots(table_row, lo, hi):
        p = np.arange(lo, hi, dtype=np.int64)
        return table_row.astype(np.int64)[p // bs] * bs + p % bs

    ctx_parts: List[np.ndarray] = []
    new_parts: List[np.ndarray] = []
    for i, (c, n) in enumerate(prefill):
        ctx_parts.append(slots(ptab[i], 0, c))
        new_parts.append(slots(ptab[i], c, c + n))
    for i, L in enumerate(decode):
        if L <= 0:
            new_parts.append(np.array([-1], dtype=np.int64))   # padded decode row: not written
            continue
        ctx_parts.append(slots(dtab[i], 0, L - 1))
        new_parts.append(slots(dtab[i], L - 1, L))
    ctx_slots = np.concatenate(ctx_parts) if ctx_parts else np.zeros(0, dtype=np.int64)
    new_slots = np.concatenate(new_parts) if new_parts else np.zeros(0, dtype=np.int64)

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    T = len(new_slots)
    Nc = len(ctx_slots)
    dt = layer.torch_dtype
    H, Hkv, D = layer.num_heads, layer.num_kv_heads, layer.head_size
    query = _normal((T, H * D), dt, device, gen)
    key = _normal((T, Hkv * D), dt, device, gen)
    value = _normal((T, Hkv * D), dt, device, gen)
    ctx_key = _normal((Nc, Hkv * D), dt, device, gen)
    ctx_value = _normal((Nc, Hkv * D), dt, device, gen)

    return PagedBatch(
        layer=layer, seed=seed,
        prefill_context_lens=np.array([c for c, _ in prefill], dtype=np.int32),
        prefill_query_lens=np.array([n for _, n in prefill], dtype=np.int32),
        prefill_cu=cumulative_starts([n for _, n in prefill]),
        prefill_block_tables=ptab,
        decode_seq_lens=np.array(list(decode), dtype=np.int32),
        decode_block_tables=dtab,
        query=query, key=key, value=value,
        slot_mapping=new_slots,
        ctx_key=ctx_key, ctx_value=ctx_value,
        ctx_slots=ctx_slots,
        poison_block=poison, used_blocks=used,
    )


# ---------------------------------------------------------------------------------------
# The five workloads.  Config k uses seed k.
# ---------------------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    index: int
    layer: LayerSpec
    prefill: List[Tuple[int, int]] = field(default_factory=list)
    decode: List[int] = field(default_factory=list)
    pool_blocks: Optional[int] = None
    seed: int = 0
    description: str = ""

    def batch(self, device="cpu") -> PagedBatch:
        return make_batch(self.layer, seed=self.seed, prefill=self.prefill, decode=self.decode,
                          device=device, pool_blocks=self.pool_blocks)


def workload(k: int) -> Workload:
    """Workload k in 1..5 (lengths drawn with numpy default_rng(k), inclusive bounds;
    the batch itself is drawn with seed k)."""
    rng = np.random.default_rng(k)
    if k == 1:
        layer = LayerSpec(8, 8, 64, 16, 32, F32, fp32(1.0 / 8.0))
        return Workload("tiny-fp32-decode", 1, layer, decode=[17, 33, 64, 100], pool_blocks=32, seed=1,
                        description="fp32 decode, B=4, L=[17,33,64,100], H=Hkv=8, D=64, bs=16, pool 32 blocks")
    if k == 2:
        layer = LayerSpec(32, 8, 128, 16, 0, BF16, fp32(1.0 / math.sqrt(128)))
        lens = rng.integers(128, 2048, size=8, endpoint=True).tolist()
        return Workload("varlen-prefill-bf16", 2, layer, prefill=[(0, int(n)) for n in lens], seed=2,
                        description="bf16 causal prefill, 8 prompts U[128,2048], H=32, Hkv=8, D=128, bs=16")
    if k == 3:
        layer = LayerSpec(32, 8, 128, 16, 0, BF16, fp32(1.0 / math.sqrt(128)))
        lens = rng.integers(512, 8192, size=256, endpoint=True).tolist()
        return Workload("batched-decode-bf16", 3, layer, decode=[int(x) for x in lens], seed=3,
                        description="bf16 decode, B=256, L~U[512,8192], H=32, Hkv=8, D=128, bs=16")
    if k == 4:
        layer = LayerSpec(32, 32, 128, 16, 0, BF16, fp32(1.0 / math.sqrt(128)),
                          alibi_slopes=alibi_slopes_geometric(32), sliding_window=4096)
        ctx = rng.integers(1024, 4096, size=4, endpoint=True).tolist()
        dec = rng.integers(256, 4096, size=128, endpoint=True).tolist()
        return Workload("mixed-chunked-prefill-bf16", 4, layer, prefill=[(int(c), 512) for c in ctx],
                        decode=[int(x) for x in dec], seed=4,
                        description="bf16 mixed batch: 4 chunks of 512 on context U[1024,4096] + 128 decodes "
                                    "L~U[256,4096]; H=Hkv=32, D=128, bs=16, ALiBi, window 4096")
    if k == 5:
        layer = LayerSpec(64, 8, 128, 32, 0, BF16, fp32(1.0 / math.sqrt(128)))
        lens = rng.integers(32768, 131072, size=32, endpoint=True).tolist()
        return Workload("long-context-decode-bf16", 5, layer, decode=[int(x) for x in lens],
                        pool_blocks=32 * 131072 // 32, seed=5,
                        description="bf16 decode, B=32, L~U[32768,131072], H=64, Hkv=8, D=128, bs=32, "
                                    "pool 131072 blocks (17.2 GB)")
    raise ValueError(f"no workload {k}")


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Exact bytes of a tensor as numpy (bf16, fp16 -> uint16 bit patterns, fp32 -> float32, uint8 codes)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float32, torch.uint8):
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")

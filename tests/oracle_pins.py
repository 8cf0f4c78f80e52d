"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with:
  * a worked example printed on the reference pages (fixtures under tests/golden/),
  * an independent library routine (torch's scaled_dot_product_attention in fp64, fed with
    contiguous K/V rebuilt from the generator's rows -- never from the oracle's cache),
  * a closed form (window of one key, a single key, a zero query), or
  * an invariance the method must have (relabelled physical blocks, GQA as repeated KV
    heads, decode as the last row of prefill, chunked prefill as rows of full prefill).

``tests/test_oracle.py`` runs them against the real oracle; ``tests/test_oracle_mutants.py``
runs them against copies of the oracle with planted mistakes and expects failures.
"""
from __future__ import annotations

import dataclasses
import json
import os

import numpy as np
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NAN_BF16 = np.uint16(0x7FC0)


# ------------------------------------------------------------------------------ helpers

ORACLE_DTYPE = {wl.F32: oracle.DTYPE_F32, wl.BF16: oracle.DTYPE_BF16, wl.F16: oracle.DTYPE_F16}
NAN_F16 = np.uint16(0x7E00)


def oracle_layer(layer: wl.LayerSpec) -> oracle.OracleLayer:
    return oracle.OracleLayer(layer.num_heads, layer.num_kv_heads, layer.head_size, layer.block_size,
                              layer.num_blocks, ORACLE_DTYPE[layer.dtype], layer.scale, layer.alibi_slopes,
                              layer.sliding_window, layer.logits_soft_cap, layer.sinks,
                              oracle.KV_CACHE_FP8_E4M3 if layer.fp8_cache else oracle.KV_CACHE_AUTO,
                              layer.k_scale, layer.v_scale)


NAN_E4M3 = np.uint8(0x7F)


def nan_pool(layer: wl.LayerSpec) -> np.ndarray:
    shape = (2, layer.num_blocks, layer.block_size * layer.num_kv_heads * layer.head_size)
    if layer.fp8_cache:
        return np.full(shape, NAN_E4M3, dtype=np.uint8)
    if layer.dtype == wl.F32:
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, NAN_F16 if layer.dtype == wl.F16 else NAN_BF16, dtype=np.uint16)


def oracle_cache(batch: wl.PagedBatch) -> np.ndarray:
    """The oracle's own pool: NaN everywhere, then context rows and new rows written by the
    oracle's cache write (as the backends write new K/V before attending)."""
    ol = oracle_layer(batch.layer)
    pool = nan_pool(batch.layer)
    oracle.cache_write(ol, wl.host_bits(batch.ctx_key), wl.host_bits(batch.ctx_value), batch.ctx_slots, pool)
    oracle.cache_write(ol, wl.host_bits(batch.key), wl.host_bits(batch.value), batch.slot_mapping, pool)
    return pool


def f64(t: torch.Tensor) -> torch.Tensor:
    return t.detach().to("cpu").to(torch.float64)


def seq_rows(batch: wl.PagedBatch):
    """Contiguous K/V [n, Hkv, D] (fp64 torch) and the new-token query rows of every
    sequence, rebuilt from the generator's row tensors in the order the generator emits
    them (prefill contexts, then decode contexts), without any cache."""
    L = batch.layer
    Hkv, D, H = L.num_kv_heads, L.head_size, L.num_heads
    ck, cv = f64(batch.ctx_key), f64(batch.ctx_value)
    k, v, q = f64(batch.key), f64(batch.value), f64(batch.query)
    out = []
    cpos = 0
    for i in range(len(batch.prefill_context_lens)):
        c = int(batch.prefill_context_lens[i])
        s, e = int(batch.prefill_cu[i]), int(batch.prefill_cu[i + 1])
        K = torch.cat([ck[cpos:cpos + c], k[s:e]]).view(-1, Hkv, D)
        V = torch.cat([cv[cpos:cpos + c], v[s:e]]).view(-1, Hkv, D)
        out.append(("prefill", i, c, K, V, q[s:e].view(-1, H, D), slice(s, e)))
        cpos += c
    tp = batch.num_prefill_tokens
    for i in range(len(batch.decode_seq_lens)):
        n = int(batch.decode_seq_lens[i])
        if n == 0:
            out.append(("decode", i, 0, None, None, q[tp + i:tp + i + 1].view(-1, H, D), slice(tp + i, tp + i + 1)))
            continue
        K = torch.cat([ck[cpos:cpos + n - 1], k[tp + i:tp + i + 1]]).view(-1, Hkv, D)
        V = torch.cat([cv[cpos:cpos + n - 1], v[tp + i:tp + i + 1]]).view(-1, Hkv, D)
        out.append(("decode", i, n - 1, K, V, q[tp + i:tp + i + 1].view(-1, H, D), slice(tp + i, tp + i + 1)))
        cpos += n - 1
    return out


def sdpa_reference(layer: wl.LayerSpec, K, V, Q, first_pos: int, bias_form: str = "hf"):
    """torch scaled_dot_product_attention in fp64 for query rows at positions
    first_pos .. first_pos + len(Q) - 1 over keys 0 .. len(K) - 1.  GQA by repeat_interleave
    of KV heads; ALiBi as an additive float mask in the row-constant-shifted form
    slope * j ("hf") or slope * (j - i) ("paper"); window and causality as -inf."""
    H = layer.num_heads
    G = H // layer.num_kv_heads
    n_q, n_k = Q.shape[0], K.shape[0]
    Kr = K.permute(1, 0, 2).repeat_interleave(G, dim=0)        # [H, n_k, D]
    Vr = V.permute(1, 0, 2).repeat_interleave(G, dim=0)
    Qr = Q.permute(1, 0, 2)                                     # [H, n_q, D]
    pos = torch.arange(first_pos, first_pos + n_q, dtype=torch.float64)[:, None]
    j = torch.arange(n_k, dtype=torch.float64)[None, :]
    allowed = j <= pos
    if layer.sliding_window and layer.sliding_window > 0:
        allowed = allowed & (pos - j < layer.sliding_window)
    mask = torch.zeros(H, n_q, n_k, dtype=torch.float64)
    if layer.alibi_slopes is not None:
        slopes = torch.tensor(layer.alibi_slopes.astype(np.float64))[:, None, None]
        mask = mask + slopes * ((j - pos) if bias_form == "paper" else j)[None]
    mask = mask.masked_fill(~allowed[None], float("-inf"))
    out = torch.nn.functional.scaled_dot_product_attention(
        Qr[None], Kr[None], Vr[None], attn_mask=mask[None], dropout_p=0.0, scale=float(layer.scale))
    return out[0].permute(1, 0, 2).numpy()                      # [n_q, H, D]


def run_oracle(batch: wl.PagedBatch, pool=None):
    """Oracle outputs for the whole batch: (prefill [Tp, H, D], decode [Bd, H, D])."""
    ol = oracle_layer(batch.layer)
    pool = oracle_cache(batch) if pool is None else pool
    q = wl.host_bits(batch.query)
    k = wl.host_bits(batch.key)
    v = wl.host_bits(batch.value)
    tp = batch.num_prefill_tokens
    pre = dec = None
    if len(batch.prefill_context_lens):
        pre = oracle.prefill(ol, q[:tp], k[:tp], v[:tp], pool, batch.prefill_block_tables,
                             batch.prefill_context_lens, batch.prefill_cu)
    if len(batch.decode_seq_lens):
        dec = oracle.decode(ol, q[tp:], pool, batch.decode_block_tables, batch.decode_seq_lens)
    return pre, dec


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def _layer(H, Hkv, D, bs, dtype=wl.F32, alibi=False, window=0, scale=None):
    return wl.LayerSpec(H, Hkv, D, bs, 0, dtype, wl.fp32(scale if scale is not None else 1.0 / np.sqrt(D)),
                        alibi_slopes=wl.alibi_slopes_geometric(H) if alibi else None, sliding_window=window)


# ------------------------------------------------------------------------------ pins

def pin_slot_worked_example():
    """Slots [35, 2, 17] at block size 16 land in (block, offset) (2,3), (0,2), (1,1)."""
    ex = json.load(open(os.path.join(GOLDEN, "slot_mapping_example.json")))
    bs = ex["block_size"]
    ol = oracle.OracleLayer(1, 1, 2, bs, 3, oracle.DTYPE_F32, 1.0)
    key = np.array([[10.0, 11.0], [20.0, 21.0], [30.0, 31.0]], dtype=np.float32)
    value = -key
    pool = np.zeros((2, 3, bs * 2), dtype=np.float32)
    oracle.cache_write(ol, key, value, np.array(ex["slot_mapping"]), pool)
    written = np.argwhere(pool[0] != 0)
    for t, (b, o) in enumerate(ex["expected_block_offset"]):
        assert np.array_equal(pool[0, b, o * 2:o * 2 + 2], key[t]), f"token {t} key not at block {b} offset {o}"
        assert np.array_equal(pool[1, b, o * 2:o * 2 + 2], value[t]), f"token {t} value not at block {b} offset {o}"
    assert len(written) == 6, "cache write touched other slots"


def pin_negative_slot_skipped():
    ol = oracle.OracleLayer(1, 1, 2, 4, 2, oracle.DTYPE_F32, 1.0)
    pool = np.zeros((2, 2, 8), dtype=np.float32)
    key = np.ones((2, 2), dtype=np.float32)
    oracle.cache_write(ol, key, key, np.array([-1, 5]), pool)
    assert np.count_nonzero(pool) == 4 and np.all(pool[:, 1, 2:4] == 1.0)


def pin_start_loc_worked_example():
    """Start locations of lengths [4, 6] are [0, 4, 10], and a two-prompt flat batch with
    those starts gives each prompt's own attention."""
    ex = json.load(open(os.path.join(GOLDEN, "start_loc_example.json")))
    cu = wl.cumulative_starts(ex["lengths"])
    assert cu.tolist() == ex["expected_start_loc"]
    layer = _layer(2, 1, 8, 4)
    both = wl.make_batch(layer, seed=11, prefill=[(0, 4), (0, 6)])
    assert both.prefill_cu.tolist() == ex["expected_start_loc"]
    pre, _ = run_oracle(both)
    for i, (s, e) in enumerate([(0, 4), (4, 10)]):
        one = wl.make_batch(layer, seed=11, prefill=[(0, e - s)])
        ol = oracle_layer(one.layer)
        alone = oracle.prefill(ol, wl.host_bits(both.query[s:e]), wl.host_bits(both.key[s:e]),
                               wl.host_bits(both.value[s:e]), None, None, None, np.array([0, e - s]))
        _close(pre[s:e], alone, 0.0, f"prompt {i} alone vs in flat batch")


def pin_identity_block_table():
    """With the identity table [0, 1, 2] the paged sequence equals its contiguous rows:
    decode over it matches SDPA over the contiguous rows."""
    ex = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    bs = ex["block_size"]
    n = len(ex["block_table"]) * bs
    layer = _layer(4, 2, 8, bs)
    layer = dataclasses.replace(layer, num_blocks=len(ex["block_table"]))
    g = torch.Generator().manual_seed(5)
    K = torch.randn(n, 2 * 8, generator=g)
    V = torch.randn(n, 2 * 8, generator=g)
    Q = torch.randn(1, 4 * 8, generator=g)
    ol = oracle_layer(layer)
    pool = np.zeros((2, layer.num_blocks, bs * 16), dtype=np.float32)
    # contiguous storage: token p at slot p of the identity table
    oracle.cache_write(ol, K.numpy(), V.numpy(), np.arange(n), pool)
    out = oracle.decode(ol, Q.numpy(), pool, np.array([ex["block_table"]]), np.array([n]))
    ref = sdpa_reference(layer, f64(K).view(n, 2, 8), f64(V).view(n, 2, 8), f64(Q).view(1, 4, 8), n - 1)
    _close(out, ref, 1e-12, "identity block table vs contiguous SDPA")


def _sdpa_batch_check(layer, prefill, decode, seed, tol=1e-12, bias_form="hf"):
    batch = wl.make_batch(layer, seed=seed, prefill=prefill, decode=decode)
    pre, dec = run_oracle(batch)
    for kind, i, c, K, V, Q, rows in seq_rows(batch):
        if K is None:
            continue
        ref = sdpa_reference(batch.layer, K, V, Q, c, bias_form)
        got = pre[rows] if kind == "prefill" else dec[i:i + 1]
        _close(got, ref, tol, f"{kind} seq {i} vs SDPA (H={layer.num_heads}, Hkv={layer.num_kv_heads}, "
                              f"bs={layer.block_size}, alibi={layer.alibi_slopes is not None}, "
                              f"W={layer.sliding_window})")


def pin_sdpa_causal_gqa():
    """Causal prefill and decode, GQA 4:1 and 2:1 and MHA, against fp64 SDPA."""
    for (H, Hkv) in [(4, 4), (4, 2), (8, 2), (4, 1)]:
        for bs in (1, 4, 16):
            _sdpa_batch_check(_layer(H, Hkv, 8, bs), prefill=[(0, 7), (0, bs + 1)], decode=[1, bs, bs + 1, 3 * bs - 1],
                              seed=100 + H * 10 + Hkv + bs)


def pin_sdpa_chunked_context():
    """Subquery rows over a cached context (chunked prefill), against SDPA over the whole
    contiguous sequence."""
    for bs in (2, 16):
        _sdpa_batch_check(_layer(4, 2, 16, bs), prefill=[(5, 3), (bs, bs), (2 * bs + 1, 4), (0, 1)],
                          decode=[], seed=200 + bs)


def pin_sdpa_alibi():
    """ALiBi: the oracle's slope * (j - pos) bias against SDPA with the shifted slope * j
    mask (the two forms give the same attention) and with slope * (j - i)."""
    for form in ("hf", "paper"):
        _sdpa_batch_check(_layer(4, 2, 8, 4, alibi=True), prefill=[(0, 9), (6, 5)], decode=[1, 7, 13],
                          seed=300, bias_form=form)
    # large-magnitude slopes make a sign error visible even over few keys
    layer = _layer(2, 1, 8, 4, alibi=True)
    layer = dataclasses.replace(layer, alibi_slopes=np.array([1.5, 0.25], dtype=np.float32))
    _sdpa_batch_check(layer, prefill=[(3, 6)], decode=[5, 11], seed=301)


def pin_sdpa_window():
    """Sliding window (W keys including the query's own), alone and with ALiBi."""
    for W in (1, 2, 3, 5):
        _sdpa_batch_check(_layer(4, 2, 8, 4, window=W), prefill=[(0, 9), (6, 5)], decode=[1, 4, 10], seed=400 + W)
        _sdpa_batch_check(_layer(4, 4, 8, 2, window=W, alibi=True), prefill=[(3, 4)], decode=[7], seed=410 + W)


def pin_window_one_closed_form():
    """W = 1: each query sees only its own key, so out = v_pos exactly."""
    layer = _layer(4, 2, 8, 4, window=1, alibi=True)
    batch = wl.make_batch(layer, seed=500, prefill=[(3, 5)], decode=[6, 1])
    pre, dec = run_oracle(batch)
    H, G, D = 4, 2, 8
    v = f64(batch.value).view(-1, 2, D).numpy()
    for t in range(batch.num_prefill_tokens):
        for h in range(H):
            _close(pre[t, h], v[t, h // G], 0.0, "W=1 prefill")
    tp = batch.num_prefill_tokens
    for i in range(2):
        for h in range(H):
            _close(dec[i, h], v[tp + i, h // G], 0.0, "W=1 decode")


def pin_single_key_closed_form():
    """A sequence of one token: out = v_0 exactly (decode and prefill)."""
    layer = _layer(4, 1, 8, 16, alibi=True)
    batch = wl.make_batch(layer, seed=600, prefill=[(0, 1)], decode=[1])
    pre, dec = run_oracle(batch)
    v = f64(batch.value).view(-1, 1, 8).numpy()
    for h in range(4):
        _close(pre[0, h], v[0, 0], 0.0, "single-key prefill")
        _close(dec[0, h], v[1, 0], 0.0, "single-key decode")


def pin_zero_query_mean():
    """q = 0 without ALiBi: every visible key has the same score, so out is the mean of the
    visible values (window respected)."""
    for W in (0, 3):
        layer = _layer(2, 1, 8, 4, window=W)
        batch = wl.make_batch(layer, seed=700 + W, prefill=[(5, 4)], decode=[9])
        batch.query.zero_()
        pre, dec = run_oracle(batch)
        for kind, i, c, K, V, Q, rows in seq_rows(batch):
            Vn = V.numpy()
            n_q = Q.shape[0]
            for t in range(n_q):
                pos = c + t
                lo = max(0, pos - W + 1) if W > 0 else 0
                mean = Vn[lo:pos + 1, 0].mean(axis=0)
                got = pre[rows][t] if kind == "prefill" else dec[i]
                for h in range(2):
                    _close(got[h], mean, 1e-14, f"zero-query mean ({kind}, W={W})")


def pin_block_relabel_invariance():
    """Relabelling physical blocks (permuting the pool and the tables alike) changes nothing."""
    layer = _layer(4, 2, 8, 4, alibi=True, window=6)
    batch = wl.make_batch(layer, seed=800, prefill=[(5, 3), (0, 4)], decode=[9, 2, 12], pool_blocks=20)
    pool = oracle_cache(batch)
    pre, dec = run_oracle(batch, pool)
    perm = np.random.default_rng(3).permutation(batch.layer.num_blocks)   # old id -> new id
    pool2 = np.empty_like(pool)
    pool2[:, perm] = pool
    b2 = dataclasses.replace(batch, prefill_block_tables=perm[batch.prefill_block_tables].astype(np.int32),
                             decode_block_tables=perm[batch.decode_block_tables].astype(np.int32))
    pre2, dec2 = run_oracle(b2, pool2)
    _close(pre2, pre, 0.0, "relabelled blocks (prefill)")
    _close(dec2, dec, 0.0, "relabelled blocks (decode)")


def pin_gqa_equals_repeated_kv():
    """GQA with G query heads per KV head equals MHA on KV heads repeated G times."""
    H, Hkv, D, bs = 8, 2, 8, 4
    G = H // Hkv
    gqa = wl.make_batch(_layer(H, Hkv, D, bs, alibi=True), seed=900, prefill=[(3, 4)], decode=[6, 9])
    rep = lambda t: t.view(-1, Hkv, D).repeat_interleave(G, dim=1).reshape(t.shape[0], H * D).contiguous()
    mha_layer = _layer(H, H, D, bs, alibi=True)
    mha = wl.make_batch(mha_layer, seed=900, prefill=[(3, 4)], decode=[6, 9])
    mha = dataclasses.replace(mha, query=gqa.query, key=rep(gqa.key), value=rep(gqa.value),
                              ctx_key=rep(gqa.ctx_key), ctx_value=rep(gqa.ctx_value),
                              slot_mapping=gqa.slot_mapping, ctx_slots=gqa.ctx_slots,
                              prefill_block_tables=gqa.prefill_block_tables,
                              decode_block_tables=gqa.decode_block_tables,
                              layer=dataclasses.replace(mha.layer, num_blocks=gqa.layer.num_blocks))
    p1, d1 = run_oracle(gqa)
    p2, d2 = run_oracle(mha)
    _close(p1, p2, 0.0, "GQA vs repeated-KV MHA (prefill)")
    _close(d1, d2, 0.0, "GQA vs repeated-KV MHA (decode)")


def pin_decode_is_last_prefill_row():
    """Decode of a length-L sequence equals the last row of causal prefill over the same L
    tokens (here: prefill with the first L-1 tokens cached and one new token)."""
    layer = _layer(4, 2, 8, 4, alibi=True, window=5)
    for L in (1, 4, 5, 11):
        dec_b = wl.make_batch(layer, seed=1000 + L, decode=[L])
        pool = oracle_cache(dec_b)
        ol = oracle_layer(dec_b.layer)
        dec = oracle.decode(ol, wl.host_bits(dec_b.query), pool, dec_b.decode_block_tables, dec_b.decode_seq_lens)
        pre = oracle.prefill(ol, wl.host_bits(dec_b.query), wl.host_bits(dec_b.key), wl.host_bits(dec_b.value),
                             pool, dec_b.decode_block_tables, np.array([L - 1]), np.array([0, 1]))
        _close(dec, pre, 0.0, f"decode vs last prefill row (L={L})")


def pin_chunked_equals_full_rows():
    """Chunked prefill (c cached + n new) gives the last n rows of a full prefill of c+n."""
    layer = _layer(4, 2, 8, 4, alibi=True, window=7)
    c, n = 9, 5
    full = wl.make_batch(layer, seed=1100, prefill=[(0, c + n)])
    ol = oracle_layer(full.layer)
    pool = oracle_cache(full)
    q, k, v = wl.host_bits(full.query), wl.host_bits(full.key), wl.host_bits(full.value)
    whole = oracle.prefill(ol, q, k, v, pool, full.prefill_block_tables, np.array([0]), np.array([0, c + n]))
    part = oracle.prefill(ol, q[c:], k[c:], v[c:], pool, full.prefill_block_tables, np.array([c]), np.array([0, n]))
    _close(part, whole[c:], 0.0, "chunked vs full prefill rows")


def pin_padded_decode_row():
    layer = _layer(2, 1, 8, 4)
    batch = wl.make_batch(layer, seed=1200, decode=[5, 0, 3])
    _, dec = run_oracle(batch)
    assert np.all(dec[1] == 0.0), "padded decode row must be zeros"
    assert np.all(np.isfinite(dec))


def pin_bf16_inputs():
    """bf16 inputs are promoted exactly: the oracle on bf16 bit patterns equals SDPA on the
    same values in fp64."""
    _sdpa_batch_check(_layer(4, 2, 16, 4, dtype=wl.BF16, alibi=True, window=6), prefill=[(4, 6)], decode=[3, 9],
                      seed=1300)


def _direct_decode(layer: wl.LayerSpec, K: np.ndarray, V: np.ndarray, Q: np.ndarray, **extra) -> np.ndarray:
    """Oracle decode of one query row over the n rows of K/V ([n, Hkv*D] float32) stored
    through the identity block table; ``extra`` overrides OracleLayer fields."""
    n = K.shape[0]
    bs = layer.block_size
    nb = -(-n // bs)
    ol = dataclasses.replace(oracle_layer(dataclasses.replace(layer, num_blocks=nb)), **extra)
    pool = np.zeros((2, nb, bs * K.shape[1]), dtype=np.float32)
    oracle.cache_write(ol, np.ascontiguousarray(K, dtype=np.float32), np.ascontiguousarray(V, dtype=np.float32),
                       np.arange(n), pool)
    return oracle.decode(ol, np.ascontiguousarray(Q, dtype=np.float32), pool, np.arange(nb)[None], np.array([n]))[0]


def pin_soft_cap_saturation_and_order():
    """Soft-cap c: scores far above c all saturate at c (tanh = 1 exactly in fp64), so two
    keys with scores 1000 and 2000 get equal weight and out is the mean of their values;
    an ALiBi bias added after the cap then splits them by exp(slope * (j - pos)) alone."""
    layer = _layer(1, 1, 4, 4, scale=1.0)
    K = np.array([[1, 0, 0, 0], [2, 0, 0, 0]], dtype=np.float32)
    V = np.array([[1, 2, 3, 4], [-3, 0, 5, 1]], dtype=np.float32)
    Q = np.array([[1000, 0, 0, 0]], dtype=np.float32)
    no_cap = _direct_decode(layer, K, V, Q)
    _close(no_cap[0], V[1], 1e-12, "uncapped: the larger score wins")
    capped = _direct_decode(layer, K, V, Q, logits_soft_cap=2.0)
    _close(capped[0], V.mean(axis=0), 1e-15, "saturated soft-cap: equal weights")
    slope = 0.75
    both = _direct_decode(layer, K, V, Q, logits_soft_cap=2.0, alibi_slopes=np.array([slope], dtype=np.float32))
    w = np.array([np.exp(-slope), 1.0])
    _close(both[0], (w[:, None] * V).sum(axis=0) / w.sum(), 1e-14, "ALiBi after a saturated soft-cap")


def pin_soft_cap_known_value():
    """A score x = c * atanh(1/2) caps to c / 2 (up to the fp32 rounding of x) and a zero
    score stays 0, so out = (e^(c/2) v_0 + v_1) / (e^(c/2) + 1); a very large cap leaves
    the scores unchanged."""
    c = 4.0
    x = float(np.float32(c * np.arctanh(0.5)))
    layer = _layer(1, 1, 4, 4, scale=1.0)
    K = np.array([[1, 0, 0, 0], [0, 1, 0, 0]], dtype=np.float32)
    V = np.array([[2, -1, 0, 4], [1, 1, -2, 0]], dtype=np.float32)
    Q = np.array([[x, 0, 0, 0]], dtype=np.float32)
    got = _direct_decode(layer, K, V, Q, logits_soft_cap=c)
    e = np.exp(c / 2)
    _close(got[0], (e * V[0] + V[1]) / (e + 1), 1e-6, "soft-cap of c atanh(1/2)")
    big = _direct_decode(layer, K, V, Q, logits_soft_cap=1e30)
    _close(big, _direct_decode(layer, K, V, Q), 1e-15, "huge cap = no cap")


def pin_sinks_closed_forms():
    """Sinks: with q = 0 every visible key scores 0, so out = sum of visible v / (n + e^sigma)
    for the head's own sigma; a single key gives v_0 / (1 + e^sigma); sigma = -inf is no
    sink at all; decode stays the last row of prefill."""
    H, Hkv, D = 4, 2, 8
    sig = np.array([0.5, -1.0, 3.0, 2.0], dtype=np.float32)
    for W in (0, 3):
        layer = dataclasses.replace(_layer(H, Hkv, D, 4, window=W), sinks=sig)
        batch = wl.make_batch(layer, seed=1400 + W, prefill=[(5, 4)], decode=[9, 1])
        batch.query.zero_()
        pre, dec = run_oracle(batch)
        for kind, i, cpos, K, V, Q, rows in seq_rows(batch):
            Vn = V.numpy()
            for t in range(Q.shape[0]):
                pos = cpos + t
                lo = max(0, pos - W + 1) if W > 0 else 0
                got = pre[rows][t] if kind == "prefill" else dec[i]
                for h in range(H):
                    ref = Vn[lo:pos + 1, h // (H // Hkv)].sum(axis=0) / (pos + 1 - lo + np.exp(np.float64(sig[h])))
                    _close(got[h], ref, 1e-14, f"sink closed form ({kind}, W={W}, head {h})")
    layer = dataclasses.replace(_layer(H, Hkv, D, 4, alibi=True, window=5),
                                sinks=np.full(H, -np.inf, dtype=np.float32))
    batch = wl.make_batch(layer, seed=1410, prefill=[(3, 5)], decode=[7, 2])
    p1, d1 = run_oracle(batch)
    p2, d2 = run_oracle(dataclasses.replace(batch, layer=dataclasses.replace(batch.layer, sinks=None)))
    _close(p1, p2, 0.0, "sink -inf vs no sink (prefill)")
    _close(d1, d2, 0.0, "sink -inf vs no sink (decode)")
    layer = dataclasses.replace(_layer(H, Hkv, D, 4, alibi=True), sinks=sig, logits_soft_cap=wl.fp32(1.5))
    for L in (1, 6):
        b = wl.make_batch(layer, seed=1420 + L, decode=[L])
        pool = oracle_cache(b)
        ol = oracle_layer(b.layer)
        dec = oracle.decode(ol, wl.host_bits(b.query), pool, b.decode_block_tables, b.decode_seq_lens)
        pre = oracle.prefill(ol, wl.host_bits(b.query), wl.host_bits(b.key), wl.host_bits(b.value),
                             pool, b.decode_block_tables, np.array([L - 1]), np.array([0, 1]))
        _close(dec, pre, 0.0, f"decode vs last prefill row with sinks and soft-cap (L={L})")


def pin_f16_promotion():
    """fp16 elements are read exactly: every one of the 65536 bit patterns, passed through a
    one-key decode (q = 0, K = 0, so out = v_0), equals numpy's float16 value, NaN and
    infinities included; the Python helper agrees with numpy too."""
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib_vals = codes.view(np.float16).astype(np.float64)
    helper = oracle.f16_bits_to_f64(codes)
    assert np.array_equal(np.isnan(helper), np.isnan(lib_vals))
    fin = ~np.isnan(lib_vals)
    assert np.array_equal(helper[fin], lib_vals[fin]), "f16_bits_to_f64 disagrees with numpy"
    D = 65536
    ol = oracle.OracleLayer(1, 1, D, 1, 1, oracle.DTYPE_F16, 1.0)
    pool = np.zeros((2, 1, D), dtype=np.uint16)
    oracle.cache_write(ol, np.zeros((1, D), dtype=np.uint16), codes[None], np.array([0]), pool)
    out = oracle.decode(ol, np.zeros((1, D), dtype=np.uint16), pool, np.array([[0]]), np.array([1]))[0, 0]
    assert np.array_equal(np.isnan(out), np.isnan(lib_vals))
    assert np.array_equal(out[fin], lib_vals[fin]), "oracle fp16 promotion disagrees with numpy"


def pin_f16_inputs():
    """fp16 layers: the oracle on fp16 bit patterns equals SDPA on the same values in fp64."""
    _sdpa_batch_check(_layer(4, 2, 16, 4, dtype=wl.F16, alibi=True, window=6), prefill=[(4, 6)], decode=[3, 9],
                      seed=1500)


def _e4m3_values(codes: np.ndarray) -> np.ndarray:
    """Values of FP8 E4M3 codes by torch's float8_e4m3fn type (the library's own decoding)."""
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def _fp8_layer(**kw) -> oracle.OracleLayer:
    base = dict(num_heads=1, num_kv_heads=1, head_size=256, block_size=1, num_blocks=1, dtype=oracle.DTYPE_F32,
                scale=1.0, kv_cache_dtype=oracle.KV_CACHE_FP8_E4M3)
    base.update(kw)
    return oracle.OracleLayer(**base)


def pin_e4m3_code_table():
    """Every FP8 E4M3 code is read as torch's float8_e4m3fn value (NaN codes as NaN): a one-key
    decode with q = 0 returns the value row, here all 256 codes, times v_scale = 1."""
    ol = _fp8_layer()
    pool = np.zeros((2, 1, 256), dtype=np.uint8)
    pool[1, 0] = np.arange(256)
    out = oracle.decode(ol, np.zeros((1, 256), dtype=np.float32), pool, np.array([[0]]), np.array([1]))[0, 0]
    ref = _e4m3_values(np.arange(256))
    assert np.array_equal(np.isnan(out), np.isnan(ref)), "NaN codes differ"
    fin = ~np.isnan(ref)
    assert np.array_equal(out[fin], ref[fin]), "E4M3 code values differ from torch float8_e4m3fn"


def pin_e4m3_quantize():
    """The fp8 cache write stores, for each element, torch's float8_e4m3fn rounding (nearest,
    ties to even) of the fp32 quotient x / scale; quotients of magnitude 464 and above (which
    torch turns into NaN) saturate to +-448, NaN stays NaN.  Checked on every midpoint between
    neighbouring codes, the codes themselves, points just off the midpoints, and random values,
    with scales 1 and 0.75."""
    pos = _e4m3_values(np.arange(127))                      # finite non-negative code values
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([pos, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                           np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.random.default_rng(9).uniform(-470, 470, 2000)]).astype(np.float32)
    vals = np.concatenate([vals, -vals, np.array([464.0, 1e6, np.inf, -np.inf, np.nan, -0.0], dtype=np.float32)])
    n = vals.size
    for scale in (1.0, 0.75):
        ol = _fp8_layer(head_size=1, num_blocks=n, k_scale=scale, v_scale=scale)
        pool = np.zeros((2, n, 1), dtype=np.uint8)
        oracle.cache_write(ol, vals[:, None], vals[:, None], np.arange(n), pool)
        q = (vals / np.float32(scale)).astype(np.float32)    # the fp32 quotient
        expect = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        big = np.abs(q) >= 464
        expect[big] = np.where(np.signbit(q[big]), 0xFE, 0x7E)
        nan = np.isnan(q)
        expect[nan] = np.where(np.signbit(q[nan]), 0xFF, 0x7F)
        for plane in (0, 1):
            got = pool[plane, :, 0]
            bad = np.flatnonzero(got != expect)
            assert bad.size == 0, (f"scale {scale}: code of {q[bad[0]]!r} is {got[bad[0]]:#x}, "
                                   f"expected {expect[bad[0]]:#x}")


def pin_fp8_cache_is_dequantized_cache():
    """Attention over an fp8 cache equals attention over an fp32 cache holding code value *
    scale (exact for the power-of-two scales used), decode and chunked prefill alike; the
    dequantized pool is built from torch's float8 decoding, not from the oracle."""
    for ks, vs in ((0.5, 2.0), (0.125, 0.25)):
        layer = dataclasses.replace(_layer(8, 2, 16, 4, alibi=True, window=9), kv_cache_dtype="fp8_e4m3",
                                    k_scale=ks, v_scale=vs)
        batch = wl.make_batch(layer, seed=1600, prefill=[(5, 4), (0, 3)], decode=[1, 7, 14])
        pool8 = oracle_cache(batch)
        p8, d8 = run_oracle(batch, pool8)
        f32_layer = dataclasses.replace(batch.layer, kv_cache_dtype="auto")
        deq = _e4m3_values(pool8.reshape(-1)).reshape(pool8.shape)
        deq[0] *= ks
        deq[1] *= vs
        pool32 = deq.astype(np.float32)
        assert np.array_equal(pool32.astype(np.float64), deq, equal_nan=True), "scaled codes must be exact in fp32"
        p32, d32 = run_oracle(dataclasses.replace(batch, layer=f32_layer), pool32)
        _close(p8, p32, 0.0, f"fp8 vs dequantized fp32 cache, prefill (scales {ks}, {vs})")
        _close(d8, d32, 0.0, f"fp8 vs dequantized fp32 cache, decode (scales {ks}, {vs})")


def pin_decode_multi():
    """Multi-token decode: one query row equals decode exactly; k rows equal the rows of a
    chunked prefill over the first L - k tokens with the k tokens new (decode reads the new
    tokens' K/V from the cache, prefill from the rows, the same bits after a cache write)."""
    layer = _layer(8, 2, 16, 4, alibi=True, window=7)
    lens = [9, 3, 0, 14]
    for k in (1, 3):
        b = wl.make_batch(layer, seed=1700 + k, prefill=[(max(L - k, 0), k if L else 0) for L in lens])
        pool = oracle_cache(b)
        ol = oracle_layer(b.layer)
        q, kk, vv = wl.host_bits(b.query), wl.host_bits(b.key), wl.host_bits(b.value)
        # padded sequence (L = 0): the generator gives it no rows, multi-token decode wants k rows
        rows = []
        pos = 0
        for L in lens:
            n = k if L else 0
            rows.append(q[pos:pos + n] if n else np.zeros((k, q.shape[1]), dtype=q.dtype))
            pos += n
        qm = np.concatenate(rows)
        tables = b.prefill_block_tables
        got = oracle.decode_multi(ol, qm, pool, tables, np.array(lens), k)
        ref = oracle.prefill(ol, q, kk, vv, pool, tables, b.prefill_context_lens, b.prefill_cu)
        pos = 0
        for i, L in enumerate(lens):
            if L == 0:
                assert np.all(got[i * k:(i + 1) * k] == 0.0), "padded sequence rows must be zeros"
                continue
            _close(got[i * k:(i + 1) * k], ref[pos:pos + k], 0.0, f"decode_multi vs chunked prefill (k={k}, L={L})")
            pos += k
        if k == 1:
            live = [i for i, L in enumerate(lens) if L]
            dec = oracle.decode(ol, qm, pool, tables, np.array(lens))
            _close(got[live], dec[live], 0.0, "decode_multi with one row vs decode")


def _numbered_cache(nb, elems, planes=2):
    """[planes, nb, elems] fp32 cache whose every element is distinct: 1000 * plane + 10 * block + index."""
    c = np.zeros((planes, nb, elems), dtype=np.float32)
    for pl in range(planes):
        for b in range(nb):
            c[pl, b] = 1000 * pl + 10 * b + np.arange(elems) / 1000.0
    return c


def pin_copy_blocks_map():
    """copy_blocks applies a source -> destinations map (the pages' Dict[int, List[int]],
    flattened to pairs) to every layer's cache, both planes, and nothing else: expected
    arrays built by slicing here, not by the oracle."""
    bs, Hkv, D = 2, 2, 4
    ol = oracle.OracleLayer(2, Hkv, D, bs, 5, oracle.DTYPE_F32, 1.0)
    elems = bs * Hkv * D
    layers = [_numbered_cache(5, elems) + 100 * l for l in range(3)]
    src_to_dsts = {0: [3, 4], 2: [1]}
    pairs = np.array([(s, d) for s, ds in src_to_dsts.items() for d in ds] + [(7, 0), (1, -1)])  # last two skipped
    got = [c.copy() for c in layers]
    oracle.copy_blocks(ol, got, pairs)
    for l, c in enumerate(layers):
        want = c.copy()
        want[:, 3] = c[:, 0]
        want[:, 4] = c[:, 0]
        want[:, 1] = c[:, 2]
        assert np.array_equal(got[l], want), f"layer {l}: copy_blocks moved the wrong bits"


def pin_swap_blocks_map():
    """swap_blocks moves block src of one cache to block dst of another with a different block
    count (both planes); an index out of range moves nothing and fails."""
    bs, Hkv, D = 2, 1, 4
    ol = oracle.OracleLayer(1, Hkv, D, bs, 3, oracle.DTYPE_F32, 1.0)
    elems = bs * Hkv * D
    src = _numbered_cache(3, elems)
    dst = _numbered_cache(6, elems) + 5000
    want = dst.copy()
    for s_, d_ in [(2, 0), (0, 5), (1, 2)]:
        want[:, d_] = src[:, s_]
    got = dst.copy()
    oracle.swap_blocks(ol, src, got, np.array([(2, 0), (0, 5), (1, 2)]))
    assert np.array_equal(got, want), "swap_blocks moved the wrong bits"
    untouched = dst.copy()
    try:
        oracle.swap_blocks(ol, src, untouched, np.array([(0, 1), (3, 0)]))
    except RuntimeError:
        pass
    else:
        raise AssertionError("swap_blocks accepted a source block out of range")
    assert np.array_equal(untouched, dst), "a rejected swap_blocks moved bits"


PINS = [
    pin_slot_worked_example, pin_negative_slot_skipped, pin_start_loc_worked_example, pin_identity_block_table,
    pin_sdpa_causal_gqa, pin_sdpa_chunked_context, pin_sdpa_alibi, pin_sdpa_window, pin_window_one_closed_form,
    pin_single_key_closed_form, pin_zero_query_mean, pin_block_relabel_invariance, pin_gqa_equals_repeated_kv,
    pin_decode_is_last_prefill_row, pin_chunked_equals_full_rows, pin_padded_decode_row, pin_bf16_inputs,
    pin_copy_blocks_map, pin_swap_blocks_map, pin_soft_cap_saturation_and_order, pin_soft_cap_known_value,
    pin_sinks_closed_forms, pin_f16_promotion, pin_f16_inputs, pin_e4m3_code_table, pin_e4m3_quantize,
    pin_fp8_cache_is_dequantized_cache, pin_decode_multi,
]

"""Seeded sweep over layer geometries and options that the fixed parity grids do not combine:
query heads per KV head from 1 to 32 (including counts that do not split evenly into groups),
head sizes 64 / 128 / 256, block sizes 8 to 64, bf16 / fp16 / fp32, an fp8 cache, ALiBi, sliding
windows, soft-caps, sinks and signed scales.  Each case runs a mixed batch (chunked prefill rows
and decode rows, some padded) and a multi-token decode through the library, and compares every
output with the oracle (the cache write bit for bit)."""
import math

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

CASES = 400


def _case(seed: int):
    rng = np.random.default_rng([seed, 77])
    wide = seed >= 64        # later cases: more sequences (past the compact prefill grid's 64) and longer ones
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 9, 11, 12, 16, 20, 24, 32]))
    Hkv = int(rng.choice([1, 2, 4]))
    if G * Hkv > 64:
        Hkv = 1
    D = int(rng.choice([64, 128, 128, 256]))
    bs = int(rng.choice([8, 16, 16, 32, 64]))
    dtype = [wl.BF16, wl.BF16, wl.F16, wl.F32][int(rng.integers(4))]
    fp8 = dtype != wl.F32 and Hkv * D <= 512 and rng.random() < 0.35
    H = G * Hkv
    alibi = rng.random() < 0.3
    window = int(rng.integers(1, 600)) if rng.random() < 0.3 else 0
    softcap = float(rng.choice([2.0, 5.0, 30.0])) if rng.random() < 0.2 else 0.0
    sinks = rng.random() < 0.2
    scale = (1.0 / math.sqrt(D)) * float(rng.choice([1.0, 1.0, 2.5, -1.0]))
    layer = wl.LayerSpec(H, Hkv, D, bs, 0, dtype, wl.fp32(scale),
                         alibi_slopes=wl.alibi_slopes_geometric(H) if alibi else None, sliding_window=window,
                         logits_soft_cap=wl.fp32(softcap), sinks=wl.sink_logits(H, seed=seed) if sinks else None,
                         kv_cache_dtype="fp8_e4m3" if fp8 else "auto", k_scale=wl.fp32(0.02) if fp8 else 1.0,
                         v_scale=wl.fp32(0.015) if fp8 else 1.0)
    budget = 1500 if fp8 else 4000          # tokens per batch (the oracle's fp8 write is slow)
    if wide and not fp8:
        budget = 12000
    n_pre = int(rng.integers(0, 4)) if not wide else int(rng.choice([0, 2, 9, 70]))
    max_sub = 300 if n_pre < 9 else 40
    prefill = [(int(rng.integers(0, budget // max(4, n_pre))), int(rng.integers(1, max_sub))) for _ in range(n_pre)]
    n_dec = int(rng.integers(1, 7)) if not wide else int(rng.choice([1, 5, 40]))
    decode = [int(x) for x in rng.integers(1, max(2, budget // max(2, n_dec // 4)), size=n_dec)]
    decode[int(rng.integers(n_dec))] = 0 if n_dec > 1 else decode[0]
    k = int(rng.integers(2, 7))
    return layer, prefill, decode, k


@pytest.mark.parametrize("seed", range(CASES))
def test_random_layer_sweep(seed):
    layer, prefill, decode, k = _case(seed)
    print(f"sweep case {seed}: {layer.num_heads}/{layer.num_kv_heads} heads D={layer.head_size} "
          f"bs={layer.block_size} {layer.dtype} cache={layer.kv_cache_dtype} alibi={layer.alibi_slopes is not None} "
          f"window={layer.sliding_window} cap={layer.logits_soft_cap} sinks={layer.sinks is not None} "
          f"scale={layer.scale:.4f}; prefill {prefill}, decode {decode}, k={k}", flush=True)
    batch = wl.make_batch(layer, seed=500 + seed, prefill=prefill, decode=decode, device=gh.device())
    cache, pre, dec = gh.gpu_run(batch)
    torch.cuda.synchronize()
    pool = gh.oracle_pool(batch)
    assert np.array_equal(wl.host_bits(cache).view(np.uint8), pool.view(np.uint8)), "cache differs"
    if pre is not None:
        gh.assert_close(gh.to_f64(pre), gh.oracle_prefill(batch, pool), batch.layer, f"case {seed} prefill")
    if dec is not None:
        ref, _ = gh.oracle_decode(batch, pool)
        gh.assert_close(gh.to_f64(dec), ref, batch.layer, f"case {seed} decode")

    # multi-token decode with k rows over the decode sequences long enough for it (others padded)
    lens = np.array([L if L >= k else 0 for L in batch.decode_seq_lens], dtype=np.int32)
    width = layer.num_heads * layer.head_size
    gen = torch.Generator(device=gh.device())
    gen.manual_seed(900 + seed)
    q = torch.empty((len(lens) * k, width), dtype=batch.query.dtype, device=gh.device())
    q.normal_(0.0, 1.0, generator=gen)
    pl = gh.player(batch.layer)
    out = gh.pa().decode(q, cache, gh.i32(batch.decode_block_tables), gh.i32(lens), pl, int(max(lens.max(), 1)),
                         query_len=k)
    torch.cuda.synchronize()
    ref = oracle.decode_multi(gh.olayer(batch.layer), wl.host_bits(q), pool, batch.decode_block_tables, lens, k)
    gh.assert_close(gh.to_f64(out), ref, batch.layer, f"case {seed} multi-token decode k={k}")


# Head size 256 over an fp8 cache with ALiBi: the most register-bound prefill instantiations (one
# wavefront per SIMD, codes held one tile ahead), with and without soft-caps, windows and fp16.
HEAD256_CASES = 48


@pytest.mark.parametrize("seed", range(HEAD256_CASES))
def test_head256_fp8_alibi_prefill(seed):
    rng = np.random.default_rng([seed, 256])
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    Hkv = int(rng.choice([1, 2]))
    bs = int(rng.choice([8, 16, 32]))
    cap = float(rng.choice([0.0, 5.0, 30.0]))
    window = int(rng.integers(1, 500)) if rng.random() < 0.3 else 0
    scale = (1.0 / 16.0) * float(rng.choice([1.0, 2.5, -1.0]))
    dtype = wl.BF16 if rng.random() < 0.7 else wl.F16
    H = G * Hkv
    layer = wl.LayerSpec(H, Hkv, 256, bs, 0, dtype, wl.fp32(scale), alibi_slopes=wl.alibi_slopes_geometric(H),
                         sliding_window=window, logits_soft_cap=wl.fp32(cap), kv_cache_dtype="fp8_e4m3",
                         k_scale=wl.fp32(0.02), v_scale=wl.fp32(0.015))
    prefill = [(int(rng.integers(0, 400)), int(rng.integers(1, 150))) for _ in range(int(rng.integers(1, 6)))]
    print(f"head-256 fp8 ALiBi case {seed}: {H}/{Hkv} heads bs={bs} {dtype} cap={cap} window={window} "
          f"scale={scale:.4f}; prefill {prefill}", flush=True)
    batch = wl.make_batch(layer, seed=seed, prefill=prefill, decode=[], device=gh.device())
    cache, pre, _ = gh.gpu_run(batch)
    torch.cuda.synchronize()
    pool = gh.oracle_pool(batch)
    assert np.array_equal(wl.host_bits(cache).view(np.uint8), pool.view(np.uint8)), "cache differs"
    gh.assert_close(gh.to_f64(pre), gh.oracle_prefill(batch, pool), batch.layer, f"head-256 fp8 case {seed}")


# Head size 256 over an fp8 cache at 2.5 times the default logit scale, with many short contexts:
# the cases where staging V as code * v_scale rounded to bf16 had pushed outputs near 4 past the
# bf16 bound, and which exact V codes keep inside it.  ALiBi with a soft-cap still stages rounded V
# at this head size, so those draws run without the cap here (that pair is covered above).
HEAD256_EXACT_V_SEEDS = list(range(32)) + [147, 248]


@pytest.mark.parametrize("seed", HEAD256_EXACT_V_SEEDS)
def test_head256_fp8_exact_v_prefill(seed):
    rng = np.random.default_rng([seed, 2561])
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    Hkv = int(rng.choice([1, 2]))
    bs = int(rng.choice([8, 16, 32]))
    cap = float(rng.choice([0.0, 0.0, 5.0, 30.0]))
    alibi = rng.random() < 0.5
    if alibi:
        cap = 0.0
    window = int(rng.integers(1, 500)) if rng.random() < 0.3 else 0
    scale = (1.0 / 16.0) * float(rng.choice([1.0, 2.5, 2.5, -1.0]))
    dtype = wl.BF16 if rng.random() < 0.7 else wl.F16
    H = G * Hkv
    layer = wl.LayerSpec(H, Hkv, 256, bs, 0, dtype, wl.fp32(scale),
                         alibi_slopes=wl.alibi_slopes_geometric(H) if alibi else None, sliding_window=window,
                         logits_soft_cap=wl.fp32(cap), kv_cache_dtype="fp8_e4m3", k_scale=wl.fp32(0.02),
                         v_scale=wl.fp32(0.015))
    n = int(rng.integers(1, 40))
    ctx_max = int(rng.choice([25, 400]))
    prefill = [(int(rng.integers(0, ctx_max)), int(rng.integers(1, 60))) for _ in range(n)]
    print(f"head-256 fp8 exact-V case {seed}: {H}/{Hkv} heads bs={bs} {dtype} alibi={alibi} cap={cap} "
          f"window={window} scale={scale:.4f}; prefill {prefill}", flush=True)
    batch = wl.make_batch(layer, seed=seed, prefill=prefill, decode=[], device=gh.device())
    cache, pre, _ = gh.gpu_run(batch)
    torch.cuda.synchronize()
    pool = gh.oracle_pool(batch)
    assert np.array_equal(wl.host_bits(cache).view(np.uint8), pool.view(np.uint8)), "cache differs"
    gh.assert_close(gh.to_f64(pre), gh.oracle_prefill(batch, pool), batch.layer, f"head-256 fp8 exact-V case {seed}")

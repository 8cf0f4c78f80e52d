"""GPU parity: libpa (through the C ABI) against the fp64 oracle on the same seeded inputs.

Cache write, block copy and block swap: bit-exact over the whole pool (unused slots keep their NaN
fill).  Attention (plain, ALiBi, windows, logits soft-cap, sink logits): bf16 max-abs <= 2e-2 and
mean-abs <= 2e-3, fp32 max-abs <= 1e-4, fp16 max-abs <= 5e-3 and mean-abs <= 5e-4.  Small grids are compared
element by element; the five full-size workloads run in the same launch configuration the
benchmark times and are compared on sampled sequences / rows (the oracle computes those one by
one)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _layer(H, Hkv, D, bs, dtype=wl.BF16, alibi=False, window=0, scale=None, softcap=0.0, sinks=False, fp8=False):
    """fp8=True: an FP8 E4M3 cache with k_scale 0.02 and v_scale 0.015 (N(0, 1) rows then use
    codes up to about 250, well inside the format's range)."""
    return wl.LayerSpec(H, Hkv, D, bs, 0, dtype, wl.fp32(scale if scale is not None else 1.0 / math.sqrt(D)),
                        alibi_slopes=wl.alibi_slopes_geometric(H) if alibi else None, sliding_window=window,
                        logits_soft_cap=wl.fp32(softcap), sinks=wl.sink_logits(H, seed=H + D) if sinks else None,
                        kv_cache_dtype="fp8_e4m3" if fp8 else "auto", k_scale=wl.fp32(0.02) if fp8 else 1.0,
                        v_scale=wl.fp32(0.015) if fp8 else 1.0)


def _check_full(batch, what):
    """Run everything on the GPU and compare everything against the oracle."""
    _say(f"[{what}] gpu run")
    cache, pre, dec = gh.gpu_run(batch)
    _say(f"[{what}] oracle")
    pool = gh.oracle_pool(batch)
    assert np.array_equal(gh.wl.host_bits(cache).view(np.uint8), pool.view(np.uint8)), f"{what}: cache differs"
    if pre is not None:
        ref = gh.oracle_prefill(batch, pool)
        gh.assert_close(gh.to_f64(pre), ref, batch.layer, f"{what} prefill")
    if dec is not None:
        ref, _ = gh.oracle_decode(batch, pool)
        gh.assert_close(gh.to_f64(dec), ref, batch.layer, f"{what} decode")


# ------------------------------------------------------------------------------ cache write

@pytest.mark.parametrize("H,Hkv,D,bs,dtype", [
    (8, 8, 64, 16, wl.F32), (32, 8, 128, 16, wl.BF16), (64, 8, 128, 32, wl.BF16), (4, 1, 64, 8, wl.BF16),
    (6, 3, 128, 256, wl.F32), (32, 8, 128, 16, wl.F16),
])
def test_cache_write_bit_exact(H, Hkv, D, bs, dtype):
    layer = _layer(H, Hkv, D, bs, dtype)
    batch = wl.make_batch(layer, seed=31, prefill=[(3, 5), (0, 40)], decode=[1, 17, 0, 2 * bs + 3],
                          device=gh.device(), pool_blocks=None)
    _say(f"cache write H={H} Hkv={Hkv} D={D} bs={bs} {dtype}")
    cache = gh.gpu_pool(batch)
    torch.cuda.synchronize()
    pool = gh.oracle_pool(batch)
    assert np.array_equal(wl.host_bits(cache).view(np.uint8), pool.view(np.uint8))


@pytest.mark.parametrize("dtype,k_scale,v_scale", [(wl.BF16, 1.0, 1.0), (wl.BF16, 0.0371, 0.0029), (wl.F16, 0.5, 3.0),
                                                   (wl.F32, 0.013, 0.21)])
def test_cache_write_fp8_bit_exact(dtype, k_scale, v_scale):
    """Quantizing cache write into an fp8 (E4M3) cache: every code equals the oracle's, including
    saturated codes (small scales push many quotients past 448) and special values."""
    layer = dataclasses.replace(_layer(16, 4, 128, 16, dtype), kv_cache_dtype="fp8_e4m3",
                                k_scale=wl.fp32(k_scale), v_scale=wl.fp32(v_scale))
    batch = wl.make_batch(layer, seed=33, prefill=[(3, 5), (0, 40)], decode=[1, 17, 0, 35], device=gh.device())
    specials = torch.tensor([float("nan"), float("inf"), -float("inf"), 0.0, -0.0, 1e30, -1e-30, 448.0, 464.0],
                            dtype=torch.float32).to(batch.key.dtype).to(gh.device())
    batch.key[0, :specials.numel()] = specials
    batch.value[1, -specials.numel():] = specials
    _say(f"fp8 cache write {dtype} scales {k_scale} {v_scale}")
    cache = gh.gpu_pool(batch)
    torch.cuda.synchronize()
    pool = gh.oracle_pool(batch)
    got = cache.cpu().numpy()
    bad = np.argwhere(got != pool)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0].tolist()}: {got[tuple(bad[0])]:#x} vs {pool[tuple(bad[0])]:#x}"


def test_cache_write_strided_rows_and_padding():
    """key/value as column slices of a wider [T, 3 * Hkv * D] tensor; slot -1 rows are skipped."""
    layer = _layer(8, 2, 128, 16)
    batch = wl.make_batch(layer, seed=32, decode=[5, 0, 9, 0, 33], device=gh.device())
    T, W = batch.key.shape
    wide = torch.zeros(T, 3 * W, dtype=torch.bfloat16, device=gh.device())
    wide[:, W:2 * W] = batch.key
    wide[:, 2 * W:] = batch.value
    strided = dataclasses.replace(batch, key=wide[:, W:2 * W], value=wide[:, 2 * W:])
    assert strided.key.stride(0) == 3 * W
    cache = gh.gpu_pool(strided)
    torch.cuda.synchronize()
    pool = gh.oracle_pool(batch)
    assert np.array_equal(wl.host_bits(cache).view(np.uint8), pool.view(np.uint8))


# ------------------------------------------------------------------------------ block copy / swap

def _random_cache(layer, nb, rng, dev):
    """[2, nb, block elements] cache of random bit patterns (NaNs and infinities included)."""
    elems = layer.block_size * layer.num_kv_heads * layer.head_size
    if layer.dtype in (wl.BF16, wl.F16):
        bits = rng.integers(0, 1 << 16, size=(2, nb, elems), dtype=np.uint16)
        return torch.from_numpy(bits.view(np.int16)).view(layer.torch_dtype).to(dev)
    bits = rng.integers(0, 1 << 32, size=(2, nb, elems), dtype=np.uint32)
    return torch.from_numpy(bits.view(np.float32)).to(dev)


def _bits(t):
    return wl.host_bits(t).view(np.uint16 if t.dtype in (torch.bfloat16, torch.float16) else np.uint32)


@pytest.mark.parametrize("H,Hkv,D,bs,dtype", [(8, 2, 128, 16, wl.BF16), (4, 4, 64, 8, wl.F32), (16, 8, 128, 256, wl.BF16),
                                               (8, 8, 64, 32, wl.F16)])
def test_copy_blocks_bit_exact(H, Hkv, D, bs, dtype):
    layer = _layer(H, Hkv, D, bs, dtype)
    nb = 64
    layer = dataclasses.replace(layer, num_blocks=nb)
    _say(f"copy_blocks {layer}")
    rng = np.random.default_rng(90 + bs)
    dev = gh.device()
    caches = [_random_cache(layer, nb, rng, dev) for _ in range(3)]
    perm = rng.permutation(nb)
    srcs, dsts = perm[:16], perm[16:40]                   # no destination is also a source
    pairs = [(int(srcs[i % 16]), int(d)) for i, d in enumerate(dsts)] + [(nb, 0), (0, -1)]   # last two skipped
    before = [wl.host_bits(c) for c in caches]          # the oracle's element types (uint16 bits or float32)
    gh.pa().copy_blocks(caches, gh.i64(np.array(pairs)), gh.player(layer))
    torch.cuda.synchronize()
    ol = gh.olayer(layer)
    ref = [b.copy() for b in before]
    oracle.copy_blocks(ol, ref, np.array(pairs))
    for l in range(3):
        assert np.array_equal(_bits(caches[l]), ref[l].view(_bits(caches[l]).dtype)), f"layer {l}: copy_blocks bits differ"


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_swap_blocks_device_host_device(dtype):
    layer = dataclasses.replace(_layer(8, 2, 64, 16, dtype), num_blocks=32)
    _say(f"swap_blocks {layer}")
    rng = np.random.default_rng(95)
    dev = gh.device()
    pl = gh.player(layer)
    gpu = _random_cache(layer, 32, rng, dev)
    host = _random_cache(layer, 48, rng, torch.device("cpu")).pin_memory()
    gpu2 = _random_cache(layer, 32, rng, dev)
    out_pairs = [(3, 10), (4, 11), (5, 12), (0, 47), (31, 0), (7, 30)]        # a run of three, then singles
    in_pairs = [(10, 1), (11, 2), (47, 30), (0, 29)]
    g0, h0, g20 = wl.host_bits(gpu), wl.host_bits(host), wl.host_bits(gpu2)
    gh.pa().swap_blocks(gpu, host, out_pairs, pl)                             # device -> pinned host
    gh.pa().swap_blocks(host, gpu2, in_pairs, pl)                             # pinned host -> device
    gh.pa().swap_blocks(gpu, gpu2, [(1, 5), (2, 6)], pl)                       # device -> device
    torch.cuda.synchronize()
    ol = gh.olayer(layer)
    h_ref, g2_ref = h0.copy(), g20.copy()
    oracle.swap_blocks(ol, g0, h_ref, np.array(out_pairs))
    oracle.swap_blocks(ol, h_ref, g2_ref, np.array(in_pairs))
    oracle.swap_blocks(ol, g0, g2_ref, np.array([(1, 5), (2, 6)]))
    u = np.uint16 if dtype == wl.BF16 else np.uint32
    assert np.array_equal(_bits(host), h_ref.view(u)), "device -> host swap bits differ"
    assert np.array_equal(_bits(gpu2), g2_ref.view(u)), "host -> device / device -> device swap bits differ"
    assert np.array_equal(_bits(gpu), g0.view(u)), "the source cache changed"
    with pytest.raises(gh.pa().PaError):
        gh.pa().swap_blocks(gpu, host, [(32, 0)], pl)


# ------------------------------------------------------------------------------ decode grid

DECODE_LAYERS = [
    _layer(8, 8, 64, 16, wl.F32, scale=0.125),
    _layer(32, 8, 128, 16),
    _layer(64, 8, 128, 32),
    _layer(32, 32, 128, 16, alibi=True, window=100),
    _layer(16, 2, 64, 8),
    _layer(12, 2, 128, 64),                 # 6 heads per KV head: padded group
    _layer(32, 2, 128, 16, window=300),     # 16 heads per KV head: two head groups
    _layer(4, 4, 128, 32, wl.F32, alibi=True, window=37),
    _layer(6, 3, 64, 256, alibi=True),
    _layer(8, 2, 128, 16, scale=-0.09),     # negative scale
    _layer(8, 8, 64, 16, alibi=True, scale=0.0),   # zero scale: weights from ALiBi alone
    # logits soft-cap (caps that bite: scaled scores of a few units) and sink logits
    _layer(32, 8, 128, 16, scale=0.3, softcap=5.0, sinks=True),
    _layer(8, 8, 64, 16, wl.F32, alibi=True, window=100, softcap=3.0, sinks=True),
    _layer(64, 8, 128, 32, sinks=True),
    _layer(16, 2, 64, 8, scale=-0.4, softcap=2.0),
    _layer(32, 32, 128, 16, alibi=True, softcap=4.0, scale=0.25),
    # fp16
    _layer(32, 8, 128, 16, wl.F16),
    _layer(64, 8, 128, 32, wl.F16, sinks=True),
    _layer(32, 32, 128, 16, wl.F16, alibi=True, window=100),
    _layer(16, 2, 64, 8, wl.F16, softcap=3.0, scale=0.3),
    # fp8 (E4M3) cache
    _layer(32, 8, 128, 16, fp8=True),
    _layer(64, 8, 128, 32, fp8=True, sinks=True),
    _layer(32, 32, 128, 16, wl.F16, fp8=True, alibi=True, window=100),
    _layer(16, 2, 64, 8, fp8=True, softcap=3.0, scale=0.3),
    _layer(12, 2, 128, 64, wl.F16, fp8=True),
    # fp8 cache with 5 or more query heads per KV head at head size 128: the MFMA decode kernel
    _layer(64, 8, 128, 16, wl.F16, fp8=True, alibi=True, window=300),
    _layer(40, 8, 128, 32, fp8=True, softcap=5.0, scale=0.3, sinks=True),
    # 17 to 32 query heads per KV head (two blocks of MFMA columns in the MFMA decode kernel)
    _layer(32, 1, 128, 16, alibi=True),
    _layer(24, 1, 128, 32, wl.F16, sinks=True, softcap=4.0, scale=0.25),
    _layer(32, 1, 128, 16, fp8=True, window=500),
    # query heads per KV head that do not split evenly into groups of at most 8 (the VALU kernel's
    # last group is short): 9 at head size 64, 11 with block size 8, 9 in fp32
    _layer(18, 2, 64, 16),
    _layer(11, 1, 128, 8, alibi=True),
    _layer(9, 1, 64, 16, wl.F32),
    _layer(14, 2, 64, 16, alibi=True, window=200),      # 7 heads per KV head: a padded group of 8
    # head size 256
    _layer(16, 8, 256, 16),
    _layer(8, 8, 256, 16, wl.F16, alibi=True, window=300),
    _layer(16, 4, 256, 32, fp8=True, softcap=30.0, scale=0.15),
    _layer(4, 2, 256, 16, wl.F32, sinks=True),
    # KV heads per work unit: 4 (groups of 4, KV heads divisible by 4), 2 (groups of 4 over 2 or 6 KV
    # heads; groups of 8 over an even count), 1 (an odd KV head count)
    _layer(16, 4, 128, 16, alibi=True),
    _layer(24, 6, 128, 16, window=700),
    _layer(12, 3, 128, 32),
    _layer(16, 2, 128, 16, wl.F16, sinks=True),
    _layer(24, 3, 128, 16),
]
DECODE_LENS = [1, 2, 31, 32, 33, 127, 129, 511, 512, 513, 1000, 1025, 2049, 0, 4100]


@pytest.mark.parametrize("li", range(len(DECODE_LAYERS)))
def test_decode_grid(li):
    layer = DECODE_LAYERS[li]
    _say(f"decode grid layer {li}: {layer}")
    batch = wl.make_batch(layer, seed=40 + li, decode=DECODE_LENS, device=gh.device())
    _check_full(batch, f"decode layer {li}")


@pytest.mark.parametrize("layer", [_layer(32, 8, 128, 16), _layer(64, 8, 128, 16, fp8=True)])
def test_decode_strided_query_and_determinism(layer):
    """A query view with a row stride of three rows (the VALU kernel, and the MFMA kernel through
    an fp8 cache with 8 query heads per KV head) equals the contiguous query's output bit for bit."""
    batch = wl.make_batch(layer, seed=50, decode=[700, 3000, 1, 64], device=gh.device())
    pl = gh.player(batch.layer)
    cache = gh.gpu_pool(batch, pl)
    width = layer.num_heads * layer.head_size
    wide = torch.zeros(4, 3 * width, dtype=torch.bfloat16, device=gh.device())
    wide[:, 128:128 + width] = batch.query
    q = wide[:, 128:128 + width]
    bt, sl = gh.i32(batch.decode_block_tables), gh.i32(batch.decode_seq_lens)
    a = gh.pa().decode(q, cache, bt, sl, pl, 3000)
    b = gh.pa().decode(batch.query, cache, bt, sl, pl, 3000)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "decode is not deterministic"
    pool = gh.oracle_pool(batch)
    ref, _ = gh.oracle_decode(batch, pool)
    gh.assert_close(gh.to_f64(a), ref, batch.layer, "strided-query decode")


def test_decode_workspace_errors():
    layer = _layer(32, 8, 128, 16)
    batch = wl.make_batch(layer, seed=51, decode=[3000, 2000], device=gh.device())
    pl = gh.player(batch.layer)
    cache = gh.gpu_pool(batch, pl)
    need = gh.pa().decode_workspace_size(pl, 2, 3000)
    assert need > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device=gh.device())
    with pytest.raises(gh.pa().PaError) as e:
        gh.pa().decode(batch.query, cache, gh.i32(batch.decode_block_tables), gh.i32(batch.decode_seq_lens), pl,
                       3000, workspace=small)
    assert e.value.status == gh.pa().PA_ERR_WORKSPACE


def test_unsupported_head_size_raises():
    pl = gh.pa().Layer(4, 4, 96, 16, 4, torch.bfloat16, 0.1)
    q = torch.zeros(1, 4 * 96, dtype=torch.bfloat16, device=gh.device())
    cache = torch.zeros(2, 4, 16 * 4 * 96, dtype=torch.bfloat16, device=gh.device())
    with pytest.raises(gh.pa().PaError) as e:
        gh.pa().decode(q, cache, gh.i32(np.zeros((1, 1))), gh.i32(np.ones(1)), pl, 1)
    assert e.value.status == gh.pa().PA_ERR_UNSUPPORTED


# ------------------------------------------------------------------------------ prefill grid

PREFILL_LAYERS = [
    _layer(32, 8, 128, 16),
    _layer(32, 32, 128, 16, alibi=True, window=100),
    _layer(8, 2, 64, 32),
    _layer(8, 8, 64, 16, wl.F32),
    _layer(12, 4, 128, 16, window=64),
    _layer(4, 1, 128, 8, alibi=True),
    _layer(4, 2, 128, 16, wl.F32, alibi=True, window=50),
    _layer(8, 4, 64, 8, window=40),                     # 8-token blocks at D = 64
    _layer(8, 2, 128, 16, scale=-0.09),                 # negative scale
    _layer(8, 8, 64, 16, alibi=True, scale=0.0),        # zero scale: weights from ALiBi alone
    _layer(4, 4, 128, 32, alibi=True, window=700),
    _layer(16, 2, 128, 64),                             # 8 heads per KV head: two workgroups of 4 heads
    _layer(8, 8, 128, 256, alibi=True, window=300),     # 256-token blocks
    _layer(24, 4, 128, 16, alibi=True, window=150),     # 6 heads per KV head: workgroups of 2 heads
    _layer(20, 4, 64, 16),                              # 5 heads per KV head: workgroups of 1 head
    _layer(48, 4, 128, 32, wl.F16, sinks=True),         # 12 heads per KV head: three workgroups of 4 heads
    # logits soft-cap and sink logits
    _layer(32, 8, 128, 16, scale=0.3, softcap=5.0, sinks=True),
    _layer(32, 32, 128, 16, alibi=True, window=100, softcap=4.0, scale=0.25),
    _layer(8, 2, 64, 32, sinks=True),
    _layer(4, 2, 128, 16, wl.F32, alibi=True, window=50, softcap=3.0, sinks=True),
    _layer(8, 2, 128, 16, scale=-0.3, softcap=2.0, sinks=True),
    _layer(8, 8, 64, 16, alibi=True, softcap=2.5),
    # fp16
    _layer(32, 8, 128, 16, wl.F16),
    _layer(32, 32, 128, 16, wl.F16, alibi=True, window=100),
    _layer(8, 2, 64, 32, wl.F16, sinks=True),
    _layer(8, 4, 128, 16, wl.F16, alibi=True, softcap=4.0, scale=0.25),
    _layer(8, 2, 128, 16, wl.F16, scale=-0.09),
    # fp8 (E4M3) cache: cached rows dequantized into the tiles, new rows at full precision
    _layer(32, 8, 128, 16, fp8=True),
    _layer(32, 32, 128, 16, wl.F16, fp8=True, alibi=True, window=100),
    _layer(8, 2, 64, 8, fp8=True, sinks=True),
    _layer(8, 4, 128, 32, fp8=True, softcap=4.0, scale=0.25),
    # head size 256
    _layer(16, 8, 256, 16),
    _layer(8, 8, 256, 16, wl.F16, alibi=True, window=300),
    _layer(16, 4, 256, 32, fp8=True, softcap=30.0, scale=0.15, sinks=True),
    _layer(4, 2, 256, 16, wl.F32, alibi=True),
    # fp32 workgroup shapes: 1, 2 and 4 query heads per workgroup, several head blocks per KV head
    _layer(12, 4, 64, 16, wl.F32, window=90),           # 3 heads per KV head: workgroups of 1 head, 128 rows
    _layer(16, 4, 128, 32, wl.F32, sinks=True),         # 4 heads per KV head: 32 rows per workgroup
    _layer(16, 2, 64, 8, wl.F32, alibi=True, softcap=3.0),  # 8 heads per KV head: two workgroups of 4 heads
    _layer(12, 2, 256, 16, wl.F32, window=200),         # 6 heads per KV head: three workgroups of 2 heads
]
PREFILL_SEQS = [(0, 1), (0, 5), (0, 128), (0, 129), (1, 64), (15, 127), (16, 130), (17, 300), (200, 33),
                (1000, 257), (63, 1), (64, 64), (0, 0)]


@pytest.mark.parametrize("li", range(len(PREFILL_LAYERS)))
def test_prefill_grid(li):
    layer = PREFILL_LAYERS[li]
    _say(f"prefill grid layer {li}: {layer}")
    batch = wl.make_batch(layer, seed=60 + li, prefill=PREFILL_SEQS, device=gh.device())
    _check_full(batch, f"prefill layer {li}")


def test_prefill_without_context_arguments():
    """No cached context: kv_cache, block_tables and context_lens may all be omitted."""
    layer = _layer(32, 8, 128, 16)
    batch = wl.make_batch(layer, seed=70, prefill=[(0, 200), (0, 7), (0, 129)], device=gh.device())
    pl = gh.player(batch.layer)
    out = gh.pa().prefill_varlen(batch.query, batch.key, batch.value, None, None, None, gh.i32(batch.prefill_cu),
                                 pl, 200, 0)
    torch.cuda.synchronize()
    pool = gh.oracle_pool(batch)
    ref = gh.oracle_prefill(batch, pool)
    gh.assert_close(gh.to_f64(out), ref, batch.layer, "context-free prefill")


@pytest.mark.parametrize("fp8", [False, True])
def test_mixed_batch_small(fp8):
    layer = _layer(16, 4, 128, 16, alibi=True, window=200, fp8=fp8)
    batch = wl.make_batch(layer, seed=71, prefill=[(100, 150), (0, 90), (333, 1)], decode=[1, 250, 700, 0],
                          device=gh.device())
    _check_full(batch, f"mixed small{' fp8' if fp8 else ''}")


@pytest.mark.parametrize("k,layer", [(4, _layer(32, 8, 128, 16)), (2, _layer(8, 8, 64, 32, alibi=True, window=500))])
def test_multi_token_decode_as_chunked_prefill(k, layer):
    """Speculative ("uniform batch") decode: every sequence brings k query tokens at the end of
    its cached context, causal among themselves -- chunked prefill with context L - k and a
    k-token subquery."""
    rng = np.random.default_rng(72 + k)
    lens = rng.integers(k + 1, 3000, size=24)
    batch = wl.make_batch(layer, seed=73 + k, prefill=[(int(L) - k, k) for L in lens], device=gh.device())
    _check_full(batch, f"multi-token decode k={k}")


# ------------------------------------------------------------------------------ full-size workloads

# (query_len, layer, number of extra sequences).  Query rows times query heads per KV head ("virtual
# heads") decide the kernel: up to 8 the VALU decode kernel (from 5 the MFMA decode kernel for an
# fp8 cache), 9 to 32 at head size 128 the MFMA decode kernel, more (16-bit layers) the MFMA
# prefill kernel with every key from the cache; fp32 layers always the VALU decode kernel.
MULTI_CASES = [
    (2, _layer(32, 8, 128, 16), 0),                               # 8 virtual heads: VALU decode
    (4, _layer(32, 8, 128, 16), 0),                               # 16: MFMA decode
    (3, _layer(32, 32, 128, 16, alibi=True, window=300), 0),      # 3 rows of one head: VALU decode, padded group of 4
    (2, _layer(64, 8, 128, 32, fp8=True), 0),                     # 16, fp8 cache: MFMA decode
    (4, _layer(32, 8, 128, 16, wl.F16, alibi=True, sinks=True, softcap=4.0, scale=0.25), 0),   # 16: MFMA decode
    (3, _layer(24, 8, 128, 16, alibi=True, window=50), 0),        # 9 (padded to 16 columns): MFMA decode
    (2, _layer(32, 8, 128, 16, fp8=True, alibi=True, window=500), 0),   # 8, fp8 cache: MFMA decode
    (4, _layer(16, 2, 64, 8, wl.F16, sinks=True, softcap=3.0, scale=0.3), 0),   # 32: prefill kernel
    (2, _layer(8, 8, 64, 16, wl.F32, alibi=True, window=40), 0),  # fp32: decode kernels
    (3, _layer(6, 2, 64, 16, wl.F32), 0),                         # 9 in fp32: VALU decode, groups of 5 and 4
    (8, _layer(8, 1, 128, 16, alibi=True), 0),                    # 64: prefill kernel
    (8, _layer(32, 8, 128, 16, alibi=True, window=700), 0),       # 32: MFMA decode, two column blocks
    (5, _layer(32, 8, 128, 32, fp8=True, sinks=True), 0),         # 20, fp8 cache: MFMA decode, two column blocks
    (4, _layer(16, 4, 256, 16, alibi=True, window=300), 0),       # head size 256: prefill kernel
    (3, _layer(32, 8, 128, 16, window=1000), 64),                 # 12, 80 sequences: MFMA decode
    (12, _layer(32, 8, 128, 16, window=1000), 64),                # 48, 80 sequences (no compact grid): prefill kernel
]


@pytest.mark.parametrize("ci", range(len(MULTI_CASES)))
def test_decode_multi(ci):
    """Multi-token decode (pa_decode_multi): k query rows per sequence, every K/V already in the
    cache, against the oracle's multi-token decode; a padded sequence (length 0) gives zero rows."""
    k, layer, extra = MULTI_CASES[ci]
    rng = np.random.default_rng(80 + ci)
    lens = [k, k + 1, 31, 129, 1000, 0, 2049, 4100] + rng.integers(k, 3000, size=8 + extra).tolist()
    live = [L for L in lens if L]
    batch = wl.make_batch(layer, seed=81 + ci, prefill=[(L - k, k) for L in live], device=gh.device())
    _say(f"decode_multi k={k} layer {ci}: {batch.layer}")
    pl = gh.player(batch.layer)
    cache = gh.gpu_pool(batch, pl)
    width = layer.num_heads * layer.head_size
    q = torch.zeros(len(lens) * k, width, dtype=batch.query.dtype, device=gh.device())
    tables = np.zeros((len(lens), batch.prefill_block_tables.shape[1]), dtype=np.int32)
    j = 0
    for i, L in enumerate(lens):
        if L:
            q[i * k:(i + 1) * k] = batch.query[j * k:(j + 1) * k]
            tables[i] = batch.prefill_block_tables[j]
            j += 1
    out = gh.pa().decode(q, cache, gh.i32(tables), gh.i32(np.array(lens)), pl, max(lens), query_len=k)
    torch.cuda.synchronize()
    pool = gh.oracle_pool(batch)
    ref = oracle.decode_multi(gh.olayer(batch.layer), wl.host_bits(q), pool, tables, np.array(lens), k)
    gh.assert_close(gh.to_f64(out), ref, batch.layer, f"decode_multi k={k} layer {ci}")


def test_graph_capture_replays():
    """The library neither allocates, nor synchronizes, nor clears memory with memset, so a whole
    step -- cache write, prefill, decode, multi-token decode (2 rows: VALU decode kernel; 4 rows,
    16 virtual heads: MFMA decode kernel) -- can be captured in a HIP graph: three replays, with
    eager work in between, each reproduce the eager outputs bit for bit."""
    layer = _layer(16, 4, 128, 16, alibi=True, window=200, sinks=True)
    batch = wl.make_batch(layer, seed=95, prefill=[(100, 150), (0, 90)], decode=[1, 250, 700, 0],
                          device=gh.device())
    pa = gh.pa()
    pl = gh.player(batch.layer)
    cache = gh.gpu_pool(batch, pl)
    tp = batch.num_prefill_tokens
    slots = gh.i64(batch.slot_mapping)
    p_args = (batch.query[:tp], batch.key[:tp], batch.value[:tp], cache, gh.i32(batch.prefill_block_tables),
              gh.i32(batch.prefill_context_lens), gh.i32(batch.prefill_cu), pl, int(batch.prefill_query_lens.max()),
              int(batch.prefill_context_lens.max()))
    d_bt, d_sl = gh.i32(batch.decode_block_tables), gh.i32(batch.decode_seq_lens)
    q_dec = batch.query[tp:]
    # multi-token decode over the two prefill sequences, their last 2 rows as the query rows
    m_bt = gh.i32(batch.prefill_block_tables)
    m_sl = gh.i32(batch.prefill_context_lens + batch.prefill_query_lens)
    q_multi = torch.stack([batch.query[int(batch.prefill_cu[i + 1]) - 2:int(batch.prefill_cu[i + 1])]
                           for i in range(2)]).reshape(4, -1).contiguous()
    q_multi4 = torch.stack([batch.query[int(batch.prefill_cu[i + 1]) - 4:int(batch.prefill_cu[i + 1])]
                            for i in range(2)]).reshape(8, -1).contiguous()
    out_pre, out_dec, out_multi = torch.empty_like(p_args[0]), torch.empty_like(q_dec), torch.empty_like(q_multi)
    out_multi4 = torch.empty_like(q_multi4)
    ws_d = torch.empty(pa.decode_workspace_size(pl, 4, 700), dtype=torch.uint8, device=gh.device())
    ws_m = torch.empty(pa.decode_workspace_size(pl, 2, 400, 2), dtype=torch.uint8, device=gh.device())
    ws_m4 = torch.empty(pa.decode_workspace_size(pl, 2, 400, 4), dtype=torch.uint8, device=gh.device())

    def step():
        pa.cache_write(batch.key, batch.value, cache, slots, pl)
        pa.prefill_varlen(*p_args, out=out_pre)
        pa.decode(q_dec, cache, d_bt, d_sl, pl, 700, out=out_dec, workspace=ws_d)
        pa.decode(q_multi, cache, m_bt, m_sl, pl, 400, out=out_multi, workspace=ws_m, query_len=2)
        pa.decode(q_multi4, cache, m_bt, m_sl, pl, 400, out=out_multi4, workspace=ws_m4, query_len=4)

    outs = (out_pre, out_dec, out_multi, out_multi4)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("prefill", "decode", "multi-token decode", "4-row decode"), outs, ref):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"replay {rep}: {name} differs"


def _sample(n, k, rng, must=()):
    pick = set(int(x) for x in must)
    pick.update(int(x) for x in rng.choice(n, size=min(k, n), replace=False))
    return sorted(pick)


def test_workload1_full():
    W = wl.workload(1)
    _say(W.description)
    batch = W.batch(gh.device())
    _check_full(batch, W.name)


def test_workload2_full():
    """Configuration 2 at full size: the whole cache bit-exact, every prefill row against the oracle
    (max-abs and mean-abs over the whole output)."""
    W = wl.workload(2)
    _say(W.description)
    batch = W.batch(gh.device())
    cache, pre, _ = gh.gpu_run(batch)
    pool = gh.oracle_pool(batch)
    assert np.array_equal(wl.host_bits(cache).view(np.uint8), pool.view(np.uint8)), "cache write differs"
    ref = gh.oracle_prefill(batch, pool)
    mx, mean = gh.assert_close(gh.to_f64(pre), ref, batch.layer, W.name)
    _say(f"{W.name}: {batch.num_prefill_tokens} rows, max abs {mx:.3e}, mean abs {mean:.3e}")


def test_long_prompt_prefill_sampled_rows():
    """The long-prompt prefill shape bench.py times (4 x 8192 new tokens, 32 / 8 heads, head size 128,
    block size 16, seed 12): the cache write bit-exact, sampled rows against the oracle."""
    lay = wl.LayerSpec(32, 8, 128, 16, 0, wl.BF16, wl.fp32(1.0 / np.sqrt(128)))
    batch = wl.make_batch(lay, seed=12, prefill=[(0, 8192)] * 4, device=gh.device())
    _say("long prompts: 4 x 8192 tokens, H=32, Hkv=8, D=128, bs=16")
    cache, pre, _ = gh.gpu_run(batch)
    pool = gh.oracle_pool(batch)
    assert np.array_equal(wl.host_bits(cache).view(np.uint8), pool.view(np.uint8)), "cache write differs"
    T = batch.num_prefill_tokens
    sel = np.zeros(T, dtype=bool)
    sel[::97] = True
    sel[batch.prefill_cu[:-1]] = True
    sel[batch.prefill_cu[1:] - 1] = True
    ref = gh.oracle_prefill(batch, pool, row_select=sel)
    gh.assert_close(gh.to_f64(pre)[sel], ref[sel].reshape(int(sel.sum()), -1), batch.layer, "long prompts")
    del batch, cache, pre
    torch.cuda.empty_cache()


def test_workload3_full():
    """Configuration 3 at full size: all 256 decode rows against the oracle."""
    W = wl.workload(3)
    _say(W.description)
    batch = W.batch(gh.device())
    cache, _, dec = gh.gpu_run(batch)
    pool = gh.oracle_pool(batch)
    assert np.array_equal(wl.host_bits(cache).view(np.uint8), pool.view(np.uint8)), "cache write differs"
    del cache
    ref, _ = gh.oracle_decode(batch, pool)
    mx, mean = gh.assert_close(gh.to_f64(dec), ref, batch.layer, W.name)
    _say(f"{W.name}: max abs {mx:.3e}, mean abs {mean:.3e}")


def test_workload4_full():
    """Configuration 4 at full size: all 2048 prefill rows and all 128 decode rows against the
    oracle, the whole cache bit-exact."""
    W = wl.workload(4)
    _say(W.description)
    batch = W.batch(gh.device())
    cache, pre, dec = gh.gpu_run(batch)
    pool = gh.oracle_pool(batch)
    assert np.array_equal(wl.host_bits(cache).view(np.uint8), pool.view(np.uint8)), "cache write differs"
    del cache
    ref, _ = gh.oracle_decode(batch, pool)
    mx, mean = gh.assert_close(gh.to_f64(dec), ref, batch.layer, W.name + " decode")
    _say(f"{W.name} decode: max abs {mx:.3e}, mean abs {mean:.3e}")
    ref = gh.oracle_prefill(batch, pool)
    mx, mean = gh.assert_close(gh.to_f64(pre), ref, batch.layer, W.name + " prefill")
    _say(f"{W.name} prefill: max abs {mx:.3e}, mean abs {mean:.3e}")


def test_workload5_full():
    """Configuration 5 at full size (17.2 GB pool): all 32 decode rows against the oracle."""
    W = wl.workload(5)
    _say(W.description)
    batch = W.batch(gh.device())
    cache, _, dec = gh.gpu_run(batch)
    del cache
    torch.cuda.empty_cache()
    lens = batch.decode_seq_lens
    pool = gh.oracle_pool(batch, decode_seqs=range(len(lens)))
    ref, _ = gh.oracle_decode(batch, pool)
    mx, mean = gh.assert_close(gh.to_f64(dec), ref, batch.layer, W.name)
    _say(f"{W.name}: max abs {mx:.3e}, mean abs {mean:.3e}")
    del batch, dec, pool
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------------ split-KV cut points

@pytest.mark.parametrize("layer", [_layer(32, 8, 128, 16), _layer(64, 8, 128, 32, alibi=True, window=3000),
                                   _layer(64, 8, 128, 32, fp8=True)])
def test_decode_split_cut_invariance(layer):
    """The even split cuts the concatenated key tiles of all sequences at fixed fractions, so the
    sequences placed before a sequence decide where its cuts fall.  One batch of 23 + 12 sequences;
    its last 12 are decoded behind 0, 1, 5 and 23 of the others (suffixes of the same batch, so
    their query, K and V are the same bytes in every placement and only the cut points move).  Every
    placement matches the oracle, and the placements agree with each other within the tolerance."""
    rng = np.random.default_rng(97)
    core = rng.integers(300, 9000, size=12).tolist()
    ahead = rng.integers(40, 7000, size=23).tolist()
    batch = wl.make_batch(layer, seed=98, decode=ahead + core, device=gh.device())
    pl = gh.player(batch.layer)
    cache = gh.gpu_pool(batch, pl)
    n0 = len(ahead)
    idx = list(range(n0, n0 + len(core)))
    pool = gh.oracle_pool(batch, decode_seqs=idx)
    ref, _ = gh.oracle_decode(batch, pool, idx)
    ref = ref.reshape(len(core), -1)
    bt, sl = gh.i32(batch.decode_block_tables), gh.i32(batch.decode_seq_lens)
    outs = []
    for extra in (0, 1, 5, 23):
        i0 = n0 - extra
        _say(f"split cut invariance: {extra} sequences ahead of {len(core)}")
        out = gh.pa().decode(batch.query[i0:], cache, bt[i0:].contiguous(), sl[i0:].contiguous(), pl,
                             int(max(ahead + core)))
        torch.cuda.synchronize()
        got = gh.to_f64(out).reshape(extra + len(core), -1)[extra:]
        gh.assert_close(got, ref, batch.layer, f"cut invariance, {extra} ahead")
        outs.append(got)
    for k in range(1, len(outs)):
        gh.assert_close(outs[k], outs[0], batch.layer, f"placement {k} against placement 0")


@pytest.mark.parametrize("n,fp8", [(1500, False), (2600, False), (2600, True)])
def test_decode_many_sequences(n, fp8):
    """Many short sequences (lengths 0 to 300, some padded) against the oracle.  Up to 2048
    sequences each split wavefront scans all of them (64 per step) to find its first sequence; 2600
    take the planning kernel, whose threads scan chunks of sequences and search inside a chunk.  The
    fp8 case (8 query heads per KV head) runs the MFMA decode kernel; its lengths stay below 40,
    since the oracle's quantizing cache write searches the code table element by element."""
    layer = _layer(64, 8, 128, 16, fp8=True) if fp8 else _layer(32, 8, 128, 16)
    rng = np.random.default_rng(99)
    lens = rng.integers(0, 40 if fp8 else 300, size=n)
    lens[::97] = 0
    batch = wl.make_batch(layer, seed=99, decode=lens.tolist(), device=gh.device())
    _check_full(batch, f"{n} sequences")


# ------------------------------------------------------------------------------ NaN propagation

@pytest.mark.parametrize("plane", [0, 1])
def test_prefill_nan_in_visible_cached_row_propagates(plane):
    """The pools are NaN-filled so that a read of an unwritten slot shows in the output.  This
    checks that a NaN in a visible cached K (plane 0) or V (plane 1) row does reach every output
    row that sees it, under the prefill kernel's build flags, while the other sequences' rows stay
    finite."""
    layer = _layer(32, 8, 128, 16)
    batch = wl.make_batch(layer, seed=96, prefill=[(200, 70), (150, 90), (0, 40)], device=gh.device())
    pl = gh.player(batch.layer)
    cache = gh.gpu_pool(batch, pl)
    L = batch.layer
    # cached key 37 of sequence 1: block table row 1, block 37 // 16, offset 37 % 16 (all KV heads)
    blk = int(batch.prefill_block_tables[1][37 // L.block_size])
    off = (37 % L.block_size) * L.row_elems
    cache[plane, blk, off:off + L.row_elems] = float("nan")
    _, pre, _ = gh.gpu_run(batch, cache=cache, pl=pl)
    got = gh.to_f64(pre)
    cu = batch.prefill_cu
    assert np.isnan(got[cu[1]:cu[2]]).all(), "rows that see the NaN row are not all NaN"
    assert np.isfinite(got[:cu[1]]).all() and np.isfinite(got[cu[2]:]).all(), "NaN leaked into other sequences"

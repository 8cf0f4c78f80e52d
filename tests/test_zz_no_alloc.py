"""pa_decode_noalloc (decode with the library's fixed device scratch array instead of a caller
workspace) against pa_decode on the same inputs: two calls in a row, the second on a smaller
batch, each bit-identical to pa_decode (the same kernels and split: the VALU decode kernel, and
the MFMA decode kernel for an fp8 cache with 8 query heads per KV head) and within the bf16
tolerance of the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import gpu_harness as gh
import workloads as wl

pytestmark = pytest.mark.gpu


def _layer(H, Hkv, D, bs, **kw):
    return wl.LayerSpec(H, Hkv, D, bs, 0, wl.BF16, wl.fp32(1.0 / math.sqrt(D)), **kw)


@pytest.mark.parametrize("first,second", [
    ((_layer(32, 8, 128, 16), 301, [4100, 1, 2049, 0, 513, 3000, 77] * 6),
     (_layer(32, 8, 128, 16), 302, [17, 900, 33])),
    ((_layer(64, 8, 128, 32, alibi_slopes=wl.alibi_slopes_geometric(64), sliding_window=700), 303,
      [5000, 12000, 1, 640] * 4),
     (_layer(8, 8, 64, 16), 304, [3, 129])),
    # an fp8 cache with 8 query heads per KV head: the MFMA decode kernel
    ((_layer(64, 8, 128, 16, kv_cache_dtype="fp8_e4m3", k_scale=wl.fp32(0.02), v_scale=wl.fp32(0.015)), 305,
      [3000, 1, 700, 0, 2049]),
     (_layer(32, 8, 128, 16), 306, [40, 600])),
])
def test_decode_noalloc_matches_decode(first, second):
    pa = gh.pa()
    for layer, seed, lens in (first, second):
        print(f"noalloc decode: {layer.num_heads}/{layer.num_kv_heads} heads D={layer.head_size} "
              f"bs={layer.block_size} seed {seed}, {len(lens)} sequences", flush=True)
        batch = wl.make_batch(layer, seed=seed, decode=lens, device=gh.device())
        pl = gh.player(batch.layer)
        cache = gh.gpu_pool(batch, pl)
        bt, sl = gh.i32(batch.decode_block_tables), gh.i32(batch.decode_seq_lens)
        mx = int(max(lens))
        ref = pa.decode(batch.query, cache, bt, sl, pl, mx)
        out = torch.full_like(batch.query, float("nan"))
        got = pa.decode_noalloc(batch.query, cache, bt, sl, pl, mx, out=out)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "noalloc decode differs from pa_decode"
        pool = gh.oracle_pool(batch)
        want, _ = gh.oracle_decode(batch, pool)
        gh.assert_close(gh.to_f64(got), want, batch.layer, "noalloc decode")

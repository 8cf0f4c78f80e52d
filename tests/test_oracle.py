"""The fp64 oracle against its pins (CPU only).  See oracle_pins.py for what each pin ties
the oracle to."""
import numpy as np
import pytest

import oracle_pins as pins
import workloads as wl


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin()


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_against_sdpa(oracle_lib, seed):
    """Random small shapes: head counts, block sizes, lengths around block boundaries,
    ALiBi and window on/off, fp32 and bf16, prefill with and without context and decode."""
    rng = np.random.default_rng(seed)
    H, Hkv = [(4, 4), (4, 2), (4, 1), (8, 2)][seed % 4]
    bs = [1, 2, 4, 16][rng.integers(4)]
    D = [4, 8, 64][rng.integers(3)]
    W = [0, 1, 3, 1000][rng.integers(4)]
    alibi = bool(rng.integers(2))
    dtype = [wl.F32, wl.BF16][seed % 2]
    k = int(rng.integers(1, 3))
    lens = [k * bs, k * bs + 1, max(1, k * bs - 1)]
    prefill = [(0, lens[0]), (lens[1], 3), (int(rng.integers(0, 20)), int(rng.integers(1, 20)))]
    decode = lens + [int(rng.integers(1, 40))]
    layer = pins._layer(H, Hkv, D, bs, dtype=dtype, alibi=alibi, window=W)
    pins._sdpa_batch_check(layer, prefill, decode, seed=2000 + seed)


def test_threads_reported(oracle_lib):
    layer = pins._layer(2, 1, 8, 4)
    batch = wl.make_batch(layer, seed=1, decode=[5, 6])
    pool = pins.oracle_cache(batch)
    _, used = oracle_lib.decode(pins.oracle_layer(batch.layer), wl.host_bits(batch.query), pool,
                                batch.decode_block_tables, batch.decode_seq_lens, num_threads=2,
                                return_threads=True)
    assert used == 2


def test_oracle_rejects_out_of_range_block(oracle_lib):
    layer = pins._layer(2, 1, 8, 4)
    batch = wl.make_batch(layer, seed=1, decode=[5])
    pool = pins.oracle_cache(batch)
    bad = batch.decode_block_tables.copy()
    bad[0, 0] = batch.layer.num_blocks + 3
    with pytest.raises(RuntimeError):
        oracle_lib.decode(pins.oracle_layer(batch.layer), wl.host_bits(batch.query), pool, bad,
                          batch.decode_seq_lens)

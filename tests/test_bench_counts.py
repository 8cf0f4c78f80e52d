"""The algorithmic counts behind every rate bench.py reports, checked on the CPU.

Prefill flops are 4 * head_size per visible (query row, key, query head); decode bytes are the
visible K and V rows of every sequence; cache-write bytes are the written rows, read and written.
Each count is compared with a brute-force enumeration of visible pairs (a key is visible from
position pos iff key <= pos and, with a window W > 0, pos - key < W) and, where one exists, with a
closed form.
"""
import numpy as np
import pytest

import bench
import workloads as wl


def _layer(H, Hkv, D, window=0, dtype=wl.BF16):
    return wl.LayerSpec(H, Hkv, D, 16, 0, dtype, wl.fp32(1.0 / np.sqrt(D)), sliding_window=window)


def _visible_pairs(context, n, window):
    count = 0
    for t in range(n):
        pos = context + t
        for key in range(pos + 1):
            if window <= 0 or pos - key < window:
                count += 1
    return count


@pytest.mark.parametrize("window", [0, 1, 7, 100])
def test_prefill_flops_brute_force(window):
    lay = _layer(4, 2, 64, window)
    prefill = [(0, 5), (3, 17), (40, 33), (0, 1)]
    batch = wl.make_batch(lay, seed=3, prefill=prefill)
    pairs = sum(_visible_pairs(c, n, window) for c, n in prefill)
    assert bench.prefill_flops(batch) == pairs * 4 * 64 * 4


def test_prefill_flops_closed_form_causal():
    # no context, no window: sum over prompts of n (n + 1) / 2 visible pairs per head
    lay = _layer(32, 8, 128)
    lens = [128, 300, 2048]
    batch = wl.make_batch(lay, seed=5, prefill=[(0, n) for n in lens])
    assert bench.prefill_flops(batch) == 4 * 128 * 32 * sum(n * (n + 1) // 2 for n in lens)


@pytest.mark.parametrize("window,dtype", [(0, wl.BF16), (50, wl.BF16), (0, wl.F32)])
def test_decode_bytes(window, dtype):
    lay = _layer(8, 2, 64, window, dtype)
    lens = [1, 17, 49, 50, 51, 200, 0]
    batch = wl.make_batch(lay, seed=7, decode=lens)
    elt = 4 if dtype == wl.F32 else 2
    visible = sum(_visible_pairs(L - 1, 1, window) for L in lens if L > 0)
    assert visible == sum(min(L, window) if window > 0 else L for L in lens)
    assert bench.decode_bytes(batch) == visible * 2 * 64 * 2 * elt


def test_cache_write_bytes_counts_written_rows_only():
    lay = _layer(8, 2, 64)
    batch = wl.make_batch(lay, seed=9, prefill=[(10, 6)], decode=[5, 9])
    written = int((batch.slot_mapping >= 0).sum())
    assert written == 6 + 2
    assert bench.cache_write_bytes(batch) == written * 2 * 64 * 2 * 2 * 2
    batch.slot_mapping = batch.slot_mapping.copy()
    batch.slot_mapping[0] = -1                      # a padded token is not written
    assert bench.cache_write_bytes(batch) == (written - 1) * 2 * 64 * 2 * 2 * 2

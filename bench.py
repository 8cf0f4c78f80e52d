"""Benchmark of the paged-KV attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--no-cpu-baseline] [--no-block-moves]
                    [--no-fp8] [--no-long-prefill]

One step is one pass of the whole hot path over one synthetic batch, all inputs resident in HBM:
pa_cache_write of the step's new K/V rows, pa_prefill_varlen over the prefill rows and pa_decode
over the decode rows (a workload without prefill or decode rows skips that call).  The default
workload is the chunked-prefill mixed batch (4 chunks of 512 new tokens on contexts U[1024, 4096],
plus 128 decode sequences with L ~ U[256, 4096], 32 query = 32 KV heads, head size 128, block
size 16, ALiBi, window 4096, bf16), the one workload that exercises every step of the path.

Each call is bracketed by HIP events on the stream it runs on (torch's current stream), so the
per-call times are kernel times; the K timed steps are bracketed by torch.cuda.synchronize().

Prints ONE JSON line:
  value         decode KV-read throughput of the headline workload, GB/s = visible K+V bytes /
                decode time (median over the timed steps)
  secondary     prefill attention TFLOP/s (4 * head_size flops per visible (row, key, head)),
                cache-write GB/s (bytes read + written), each with its fraction of peak and the
                median / min / mean call times; `configs`: the other four workloads, each built,
                timed (W warm-up + K timed calls of its own step) and freed in turn, with the same
                rates and fractions (--no-configs skips them); and,
                outside the timed steps, pa_copy_blocks GB/s (1024 scattered blocks of the
                workload's geometry in a scratch cache, bytes read + written) and pa_swap_blocks
                GB/s to and from pinned host memory (--no-block-moves skips them); and, also outside
                the timed steps, decode and prefill over an FP8 (E4M3) copy of the cache (--no-fp8);
                and prefill on long prompts (4 x 8192 new tokens, workload 2's head geometry), where
                per-workgroup fixed costs are amortized, with an fp32 prefill batch against the fp32
                matrix-unit peak (--no-long-prefill skips both); and the cache write with
                a cold Infinity Cache (512 MB written just before each timed call)
  roofline      the dominant call (decode, HBM-bound): achieved GB/s per launch vs 8 TB/s;
                traffic = HBM bytes per call measured with rocprofv3 FETCH_SIZE + WRITE_SIZE
                (profiles/decode_traffic.json), null when the decode source changed since
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded sample of the same
                workload: decode sequences (GB/s of visible K+V, `value`) and prefill rows
                (GFLOP/s, `prefill`), with the thread count and the CPU model
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "decode KV-read GB/s (% HBM peak); prefill attn TFLOP/s (% MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
DECODE_SOURCES = ("paged_kv_cache_242_amd/csrc/decode.hip", "paged_kv_cache_242_amd/csrc/pa_device.h")
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, 2.5 PFLOP/s
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(batch: wl.PagedBatch) -> int:
    L = batch.layer
    W = L.sliding_window
    lens = batch.decode_seq_lens.astype(np.int64)
    vis = np.minimum(lens, W) if W and W > 0 else lens
    return int(vis.sum()) * L.num_kv_heads * L.head_size * 2 * L.elt_bytes


def prefill_flops(batch: wl.PagedBatch) -> int:
    L = batch.layer
    W = L.sliding_window
    total = 0
    for c, n in zip(batch.prefill_context_lens.astype(np.int64), batch.prefill_query_lens.astype(np.int64)):
        pos = c + np.arange(n, dtype=np.int64)
        vis = np.minimum(pos + 1, W) if W and W > 0 else pos + 1
        total += int(vis.sum())
    return total * L.num_heads * 4 * L.head_size


def cache_write_bytes(batch: wl.PagedBatch) -> int:
    L = batch.layer
    rows = int((batch.slot_mapping >= 0).sum())
    return rows * L.row_elems * L.elt_bytes * 2 * 2      # K and V, read + written


def decode_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: int):
    """HBM bytes per decode call (plan + split + merge kernels) from the committed rocprofv3 counter
    summary, or None when there is none for this workload or the decode kernel source changed
    since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("decode_source_sha256") != decode_source_hash():
        return None
    entry = data.get("workloads", {}).get(str(workload))
    return None if entry is None else entry.get("hbm_bytes_per_call")


def copy_probe(gib: float):
    """A plain device copy of a known size (for calibrating the FETCH_SIZE / WRITE_SIZE counters)."""
    dev = torch.device("cuda:0")
    n = int(gib * (1 << 30))
    x = torch.ones(n, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "calls": 3}), flush=True)
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def oracle_layer(L):
    import oracle
    return oracle.OracleLayer(L.num_heads, L.num_kv_heads, L.head_size, L.block_size, L.num_blocks,
                              oracle.DTYPE_F32 if L.dtype == wl.F32 else oracle.DTYPE_BF16, L.scale,
                              L.alibi_slopes, L.sliding_window)


def cpu_prefill_baseline(batch: wl.PagedBatch, pool: np.ndarray, budget_s: float = 12.0):
    """Time the oracle's prefill on this machine's host cores over a bounded sample of the prefill
    rows of the same batch (every k-th row, k sized for ~budget_s of CPU work), in GFLOP/s of the
    same algorithmic count as the GPU figure (4 * head_size per visible (row, key, head))."""
    import oracle
    L = batch.layer
    ol = oracle_layer(L)
    tp = batch.num_prefill_tokens
    q, k, v = (wl.host_bits(x[:tp]) for x in (batch.query, batch.key, batch.value))
    W = L.sliding_window
    # visible keys of every prefill row
    vis = np.zeros(tp, dtype=np.int64)
    for i, (c, n) in enumerate(zip(batch.prefill_context_lens, batch.prefill_query_lens)):
        a = int(batch.prefill_cu[i])
        pos = int(c) + np.arange(int(n), dtype=np.int64)
        vis[a:a + int(n)] = np.minimum(pos + 1, W) if W and W > 0 else pos + 1
    per_vis = L.num_heads * 4 * L.head_size
    stride = max(1, tp // 16)
    used = 0
    while True:
        sel = np.zeros(tp, dtype=bool)
        sel[::stride] = True
        t0 = time.perf_counter()
        _, used = oracle.prefill(ol, q, k, v, pool, batch.prefill_block_tables, batch.prefill_context_lens,
                                 batch.prefill_cu, row_select=sel, return_threads=True)
        dt = time.perf_counter() - t0
        flops = int(vis[sel].sum()) * per_vis
        if dt >= 0.5 * budget_s or stride == 1:
            break
        stride = max(1, int(stride * dt / budget_s))
    return {"value": flops / dt / 1e9, "unit": "GFLOP/s", "cores": int(used),
            "sample": f"fp64 oracle prefill of {int(sel.sum())} of the {tp} prefill rows of the same batch "
                      f"(every {stride}th row; {flops / 1e9:.1f} GFLOP, {dt:.1f} s)"}


def cpu_baseline(batch: wl.PagedBatch, pool: np.ndarray, budget_s: float = 20.0):
    """Time the oracle's decode on this machine's host cores over a bounded sample of the
    decode sequences of the same batch (longest-first is not used: a seeded random subset)."""
    import oracle
    L = batch.layer
    ol = oracle_layer(L)
    tp = batch.num_prefill_tokens
    q = wl.host_bits(batch.query[tp:])
    lens = batch.decode_seq_lens
    order = np.random.default_rng(batch.seed).permutation(len(lens))
    # Calibrate on a small slice, then size the sample for ~budget_s of CPU work, cycling over the
    # sequences (in the same seeded order) as often as the budget allows, at most `max_passes` times.
    max_passes = 1000
    done_bytes = 0
    done_time = 0.0
    used = 0
    calls = 0
    start = 0
    chunk = 4
    while start < max_passes * len(order):
        pos = start % len(order)
        idx = order[pos:pos + min(chunk, len(order) - pos)]
        t0 = time.perf_counter()
        _, used = oracle.decode(ol, q[idx], pool, batch.decode_block_tables[idx], lens[idx], return_threads=True)
        dt = time.perf_counter() - t0
        vis = np.minimum(lens[idx], L.sliding_window) if L.sliding_window > 0 else lens[idx]
        nbytes = int(vis.astype(np.int64).sum()) * L.num_kv_heads * L.head_size * 2 * L.elt_bytes
        done_bytes += nbytes
        done_time += dt
        calls += len(idx)
        start += len(idx)
        per_seq = done_time / calls
        remaining = budget_s - done_time
        if remaining <= 0:
            break
        chunk = max(1, int(remaining / max(per_seq, 1e-9)))
    return {
        "value": done_bytes / done_time / 1e9,
        "unit": "GB/s",
        "cores": int(used),
        "kind": "oracle",
        "sample": f"fp64 oracle decode of {calls} sequences ({calls / len(lens):.1f} passes over the {len(lens)} "
                  f"decode sequences of the same batch, seeded order; {done_bytes / 1e9:.2f} GB of visible K+V, "
                  f"{done_time:.1f} s) on {cpu_model()}",
        "cpu_model": cpu_model(),
    }


def block_moves(pa, L, dev, num_pairs: int = 1024, reps: int = 10):
    """Timing of pa.copy_blocks (one layer, num_pairs scattered pairs inside a scratch cache of
    the workload's layer geometry) and pa.swap_blocks (num_pairs blocks device -> pinned host
    and back, in runs).  Outside the timed step; the step's own cache is not touched."""
    elems = L.block_size * L.row_elems
    bb = elems * L.elt_bytes                                    # bytes per block and plane
    nb = 4 * num_pairs
    layer = pa.Layer(L.num_heads, L.num_kv_heads, L.head_size, L.block_size, nb, L.torch_dtype, L.scale, None, 0)
    scratch = torch.zeros((2, nb, elems), dtype=L.torch_dtype, device=dev)
    perm = np.random.default_rng(0).permutation(nb)
    pairs = torch.as_tensor(np.stack([perm[:num_pairs], perm[num_pairs:2 * num_pairs]], 1), device=dev)
    host = torch.zeros((2, num_pairs, elems), dtype=L.torch_dtype).pin_memory()
    runs_out = np.stack([np.arange(num_pairs), np.arange(num_pairs)], 1)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, fn, nbytes in (
            ("copy_blocks", lambda: pa.copy_blocks([scratch], pairs, layer), 2 * 2 * num_pairs * bb),
            ("swap_blocks_d2h", lambda: pa.swap_blocks(scratch, host, runs_out, layer), 2 * num_pairs * bb),
            ("swap_blocks_h2d", lambda: pa.swap_blocks(host, scratch, runs_out, layer), 2 * num_pairs * bb)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": ms, "blocks": num_pairs, "bytes_per_call": nbytes, "GB_per_s": nbytes / (ms * 1e-3) / 1e9}
    out["copy_blocks"]["frac_hbm_peak"] = out["copy_blocks"]["GB_per_s"] / HBM_PEAK_GBPS
    del scratch, host
    torch.cuda.empty_cache()
    return out


def cold_cache_write_leg(pa, batch, cache, slots, layer, dev, reps: int = 10):
    """Outside the timed steps: pa_cache_write timed after writing a 512 MB scratch buffer, so that
    its ~70 MB of key/value rows and cache lines come from HBM rather than the 256 MB Infinity
    Cache."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ts = []
    for r in range(reps):
        scratch.fill_(r & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pa.cache_write(batch.key, batch.value, cache, slots, layer)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del scratch
    torch.cuda.empty_cache()
    ms = float(np.median(ts))
    gbps = cache_write_bytes(batch) / (ms * 1e-3) / 1e9
    return {"ms": ms, "GB_per_s": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS, "flush_bytes": 512 << 20}


def _prefill_leg(pa, dev, lay, prefill, seed, reps: int = 5):
    """Median time and rate of one prefill call on a seeded batch (outside the timed steps)."""
    batch = wl.make_batch(lay, seed=seed, prefill=prefill, device=dev)
    L = batch.layer
    layer = pa.Layer(L.num_heads, L.num_kv_heads, L.head_size, L.block_size, L.num_blocks, L.torch_dtype, L.scale,
                     None, 0)
    cache = torch.zeros((2, L.num_blocks, L.block_size * L.row_elems), dtype=L.torch_dtype, device=dev)
    if batch.ctx_key.shape[0]:
        pa.cache_write(batch.ctx_key, batch.ctx_value, cache, torch.as_tensor(batch.ctx_slots, device=dev), layer)
    i32 = lambda a: torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32, device=dev)
    args = (batch.query, batch.key, batch.value, cache, i32(batch.prefill_block_tables),
            i32(batch.prefill_context_lens), i32(batch.prefill_cu), layer, int(batch.prefill_query_lens.max()),
            int(batch.prefill_context_lens.max()))
    out = torch.empty_like(batch.query)
    for _ in range(2):
        pa.prefill_varlen(*args, out=out)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pa.prefill_varlen(*args, out=out)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    flops = prefill_flops(batch)
    ms = float(np.median(ts))
    del batch, cache, out
    torch.cuda.empty_cache()
    return ms, flops


def long_prefill_leg(pa, dev, reps: int = 5):
    """Outside the timed steps: causal prefill of 4 prompts of 8192 tokens with no cached context
    (32 query / 8 KV heads, head size 128, block size 16, bf16, seed 12).  Each wavefront then
    walks ~128 key tiles instead of the ~5-15 of the configured prompts."""
    lay = wl.LayerSpec(32, 8, 128, 16, 0, wl.BF16, wl.fp32(1.0 / np.sqrt(128)))
    ms, flops = _prefill_leg(pa, dev, lay, [(0, 8192)] * 4, 12, reps)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"shape": "4 x 8192 new tokens, H=32, Hkv=8, D=128, bs=16, causal, no context", "ms": ms,
            "gflop_per_call": flops / 1e9, "TFLOP_per_s": tflops, "frac_mfma_peak": tflops / MFMA_BF16_PEAK_TFLOPS}


def f32_prefill_leg(pa, dev, reps: int = 5):
    """Outside the timed steps: the fp32 prefill kernel on 2 prompts of 1024 tokens and 2 chunks of
    256 rows on 2000-token contexts (32 query / 8 KV heads, head size 128, block size 16, seed 7),
    against the fp32 matrix-unit peak."""
    lay = wl.LayerSpec(32, 8, 128, 16, 0, wl.F32, wl.fp32(1.0 / np.sqrt(128)))
    ms, flops = _prefill_leg(pa, dev, lay, [(0, 1024)] * 2 + [(2000, 256)] * 2, 7, reps)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"shape": "fp32: 2 x 1024 new tokens + 2 x 256 rows on 2000-token contexts, H=32, Hkv=8, D=128, bs=16",
            "ms": ms, "gflop_per_call": flops / 1e9, "TFLOP_per_s": tflops,
            "frac_f32_mfma_peak": tflops / MFMA_F32_PEAK_TFLOPS}


def fp8_cache_leg(pa, L, layer, cache, dev, dec_args, pre_args, reps: int = 10):
    """Outside the timed steps: the same batch over an FP8 (E4M3) copy of the cache, quantized
    from it by pa_cache_write (k_scale 0.02, v_scale 0.015 for N(0, 1) rows).  Decode GB/s counts
    the fp8 bytes read; prefill TFLOP/s the same flops as the bf16 run."""
    import dataclasses
    l8 = dataclasses.replace(layer, kv_cache_dtype="fp8_e4m3", k_scale=0.02, v_scale=0.015)
    rows = cache.view(2, -1, L.row_elems)
    c8 = torch.empty(cache.shape, dtype=torch.uint8, device=dev)
    pa.cache_write(rows[0], rows[1], c8, torch.arange(rows.shape[1], device=dev), l8)
    res = {"k_scale": 0.02, "v_scale": 0.015}

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    if dec_args is not None:
        q, bt, sl, mx, nbytes = dec_args
        out = torch.empty_like(q)
        ws = torch.empty(max(pa.decode_workspace_size(l8, sl.numel(), mx), 1), dtype=torch.uint8, device=dev)
        ms = timed(lambda: pa.decode(q, c8, bt, sl, l8, mx, out=out, workspace=ws))
        res["decode"] = {"ms": ms, "GB_per_s": nbytes / 2 / (ms * 1e-3) / 1e9,
                         "frac_hbm_peak": nbytes / 2 / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    if pre_args is not None:
        q, k, v, bt, ctx, cu, mq, mc, flops = pre_args
        out = torch.empty_like(q)
        ms = timed(lambda: pa.prefill_varlen(q, k, v, c8, bt, ctx, cu, l8, mq, mc, out=out))
        res["prefill"] = {"ms": ms, "TFLOP_per_s": flops / (ms * 1e-3) / 1e12}
    del c8
    torch.cuda.empty_cache()
    return res


def ms_stats(ts):
    ts = [float(t) for t in ts]
    return {"ms": float(np.median(ts)), "ms_min": float(np.min(ts)), "ms_mean": float(np.mean(ts))}


def decode_side_bytes(batch: wl.PagedBatch) -> dict:
    """Bytes a decode call moves beside the visible K+V (not part of the algorithmic count):
    query rows read, output rows written, block-table entries of the visible blocks read."""
    L = batch.layer
    B = len(batch.decode_seq_lens)
    lens = batch.decode_seq_lens.astype(np.int64)
    return {"query_bytes": B * L.num_heads * L.head_size * L.elt_bytes,
            "out_bytes": B * L.num_heads * L.head_size * L.elt_bytes,
            "block_table_bytes": int(((lens + L.block_size - 1) // L.block_size).sum()) * 4}


class StepRunner:
    """One workload's step (cache write, prefill, decode; each present part) on the GPU with HIP
    events around every call on the stream the calls run on."""

    def __init__(self, pa, W, dev, layer_kw=None):
        self.pa, self.W, self.dev = pa, W, dev
        t0 = time.perf_counter()
        batch = W.batch(dev)
        L = batch.layer
        self.L = L
        slopes = torch.tensor(L.alibi_slopes, device=dev) if L.alibi_slopes is not None else None
        self.layer = pa.Layer(L.num_heads, L.num_kv_heads, L.head_size, L.block_size, L.num_blocks, L.torch_dtype,
                              L.scale, slopes, L.sliding_window)
        self.cache = torch.full((2, L.num_blocks, L.block_size * L.row_elems), float("nan"), dtype=L.torch_dtype,
                                device=dev)
        if batch.ctx_key.shape[0]:
            pa.cache_write(batch.ctx_key, batch.ctx_value, self.cache, torch.as_tensor(batch.ctx_slots, device=dev),
                           self.layer)
        batch.ctx_key = batch.ctx_value = None                       # context is in the cache now
        self.batch = batch
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        self.setup_s = time.perf_counter() - t0
        i32 = lambda a: torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32, device=dev)
        self.slots = torch.as_tensor(batch.slot_mapping, device=dev)
        tp = batch.num_prefill_tokens
        self.tp = tp
        self.has_pre = len(batch.prefill_context_lens) > 0
        self.has_dec = len(batch.decode_seq_lens) > 0
        if self.has_pre:
            self.p_bt, self.p_ctx, self.p_cu = (i32(batch.prefill_block_tables), i32(batch.prefill_context_lens),
                                                i32(batch.prefill_cu))
            self.p_maxq, self.p_maxc = int(batch.prefill_query_lens.max()), int(batch.prefill_context_lens.max())
            self.q_pre, self.k_pre, self.v_pre = batch.query[:tp], batch.key[:tp], batch.value[:tp]
            self.out_pre = torch.empty_like(self.q_pre)
        if self.has_dec:
            self.d_bt, self.d_sl = i32(batch.decode_block_tables), i32(batch.decode_seq_lens)
            self.d_max = int(batch.decode_seq_lens.max())
            self.q_dec = batch.query[tp:]
            self.out_dec = torch.empty_like(self.q_dec)
            ws_bytes = pa.decode_workspace_size(self.layer, len(batch.decode_seq_lens), self.d_max)
            self.ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)

    def prefill(self):
        self.pa.prefill_varlen(self.q_pre, self.k_pre, self.v_pre, self.cache, self.p_bt, self.p_ctx, self.p_cu,
                               self.layer, self.p_maxq, self.p_maxc, out=self.out_pre)

    def decode(self):
        self.pa.decode(self.q_dec, self.cache, self.d_bt, self.d_sl, self.layer, self.d_max, out=self.out_dec,
                       workspace=self.ws)

    def run(self, steps: int, warmup: int):
        """warmup + steps steps; returns per-call times (ms) of the timed steps and the wall time of
        the timed steps (bracketed by torch.cuda.synchronize())."""
        parts = [("cw", lambda: self.pa.cache_write(self.batch.key, self.batch.value, self.cache, self.slots,
                                                      self.layer))]
        if self.has_pre:
            parts.append(("pre", self.prefill))
        if self.has_dec:
            parts.append(("dec", self.decode))
        n = steps + warmup
        ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
              for k, _ in parts}

        def step(s):
            for k, fn in parts:
                ev[k][s][0].record(self.stream)
                fn()
                ev[k][s][1].record(self.stream)

        for s in range(warmup):
            step(s)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(warmup, n):
            step(s)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        times = {k: [ev[k][s][0].elapsed_time(ev[k][s][1]) for s in range(warmup, n)] for k, _ in parts}
        return times, wall

    def results(self, times):
        b = self.batch
        out = {}
        cw = ms_stats(times["cw"])
        gbps = cache_write_bytes(b) / (cw["ms"] * 1e-3) / 1e9
        out["cache_write"] = dict(cw, bytes_per_call=cache_write_bytes(b), GB_per_s=gbps,
                                  frac_hbm_peak=gbps / HBM_PEAK_GBPS)
        if self.has_pre:
            st = ms_stats(times["pre"])
            flops = prefill_flops(b)
            tf = flops / (st["ms"] * 1e-3) / 1e12
            out["prefill"] = dict(st, gflop_per_call=flops / 1e9, TFLOP_per_s=tf,
                                  frac_mfma_peak=tf / MFMA_BF16_PEAK_TFLOPS, rows=self.tp,
                                  seqs=int(len(b.prefill_context_lens)))
        if self.has_dec:
            st = ms_stats(times["dec"])
            nbytes = decode_bytes(b)
            gbps = nbytes / (st["ms"] * 1e-3) / 1e9
            out["decode"] = dict(st, gb_per_call=nbytes / 1e9, GB_per_s=gbps, frac_hbm_peak=gbps / HBM_PEAK_GBPS,
                                 seqs=int(len(b.decode_seq_lens)), **decode_side_bytes(b))
        return out

    def free(self):
        for name in list(vars(self)):
            if name not in ("pa", "W", "dev", "L", "setup_s"):
                delattr(self, name)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def multi_token_leg(pa, r, ks=(2, 4, 8), reps: int = 10):
    """Multi-token decode (pa_decode_multi) over a decode workload's cache: query_len = k rows per
    sequence at the end of its cached tokens (N(0, 1) queries, seed 7).  GB/s counts each sequence's
    visible K+V once, as for single-token decode."""
    b, L, layer = r.batch, r.L, r.layer
    B = len(b.decode_seq_lens)
    G = L.num_heads // L.num_kv_heads
    nbytes = decode_bytes(b)
    gen = torch.Generator(device=r.dev)
    gen.manual_seed(7)
    res = {}
    for k in ks:
        q = torch.empty((B * k, L.num_heads * L.head_size), dtype=L.torch_dtype, device=r.dev)
        q.normal_(0.0, 1.0, generator=gen)
        out = torch.empty_like(q)
        ws = torch.empty(max(pa.decode_workspace_size(layer, B, r.d_max, k), 1), dtype=torch.uint8, device=r.dev)
        run = lambda: pa.decode(q, r.cache, r.d_bt, r.d_sl, layer, r.d_max, out=out, workspace=ws, query_len=k)
        for _ in range(2):
            run()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(r.stream)
            run()
            e1.record(r.stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        st = ms_stats(ts)
        gbps = nbytes / (st["ms"] * 1e-3) / 1e9
        if L.dtype == wl.F32 or k * G <= 8:
            kern = "VALU decode"
        elif k * G <= 32 and L.head_size == 128 and L.block_size >= 16:
            kern = "MFMA decode"
        else:
            kern = "MFMA prefill"
        res[str(k)] = dict(st, GB_per_s=gbps, frac_hbm_peak=gbps / HBM_PEAK_GBPS, kernels=kern)
        del q, out, ws
    return res


def config_leg(pa, k: int, dev, steps: int, warmup: int):
    """Workload k built, timed and freed: its own step (cache write, prefill and / or decode)."""
    W = wl.workload(k)
    log(f"config {k}: {W.description}")
    r = StepRunner(pa, W, dev)
    times, _ = r.run(steps, warmup)
    res = r.results(times)
    if k == 3:
        res["multi_token_decode"] = multi_token_leg(pa, r)
    res["workload"] = f"{W.name}: {W.description}"
    res["setup_s"] = round(r.setup_s, 1)
    r.free()
    del r
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-configs", action="store_true", help="skip the legs of the other four workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-block-moves", action="store_true", help="skip the copy_blocks / swap_blocks timing")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-cache timing")
    ap.add_argument("--no-long-prefill", action="store_true", help="skip the long-prompt prefill timing")
    ap.add_argument("--no-multi-token", action="store_true", help="skip the multi-token decode timing")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--copy-probe", type=float, default=0.0, metavar="GIB",
                    help="only run a plain device copy of GIB GiB (counter calibration) and exit")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe > 0:
        return copy_probe(args.copy_probe)
    import paged_kv_cache_242_amd as pa

    dev = torch.device("cuda:0")
    W = wl.workload(args.workload)
    log(f"workload {args.workload}: {W.description}")
    R = StepRunner(pa, W, dev)
    L, batch, layer, cache = R.L, R.batch, R.layer, R.cache
    log(f"setup {R.setup_s:.1f} s; pool {cache.numel() * cache.element_size() / 1e9:.2f} GB")
    times, wall = R.run(args.steps, args.warmup)
    log(f"timed {args.steps} steps in {wall * 1e3:.2f} ms")
    secondary = R.results(times)

    if args.workload == 3 and not args.no_multi_token:
        secondary["multi_token_decode"] = multi_token_leg(pa, R)
    secondary["cache_write_cold"] = cold_cache_write_leg(pa, batch, cache, R.slots, layer, dev)
    if not args.no_block_moves:
        secondary.update(block_moves(pa, L, dev))
    if not args.no_fp8 and L.dtype != wl.F32:
        secondary["fp8_cache"] = fp8_cache_leg(
            pa, L, layer, cache, dev,
            (R.q_dec, R.d_bt, R.d_sl, R.d_max, decode_bytes(batch)) if R.has_dec else None,
            (R.q_pre, R.k_pre, R.v_pre, R.p_bt, R.p_ctx, R.p_cu, R.p_maxq, R.p_maxc, prefill_flops(batch))
            if R.has_pre else None)
    if not args.no_long_prefill and L.dtype != wl.F32:
        secondary["prefill_long_prompts"] = long_prefill_leg(pa, dev)
        secondary["prefill_fp32"] = f32_prefill_leg(pa, dev)

    value, unit = None, "GB/s"
    if R.has_dec:
        d = secondary["decode"]
        value = d["GB_per_s"]
        roofline = {"bound": "hbm", "achieved": value, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": value / HBM_PEAK_GBPS, "traffic": measured_traffic(args.workload),
                    "kernel": "pa_decode (decode_split_kernel + decode_merge_kernel; decode_plan_kernel only above 2048 sequences)",
                    "algorithmic_bytes_per_launch": decode_bytes(batch), "ms_median": d["ms"]}
    else:
        value, unit = secondary["prefill"]["TFLOP_per_s"], "TFLOP/s"
        roofline = {"bound": "mfma", "achieved": value, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": value / MFMA_BF16_PEAK_TFLOPS, "traffic": None, "kernel": "prefill_mfma_kernel",
                    "algorithmic_flops_per_launch": prefill_flops(batch), "ms_median": secondary["prefill"]["ms"]}
    if R.has_pre and R.has_dec:
        p = secondary["prefill"]
        secondary["prefill_roofline"] = {"bound": "mfma", "achieved": p["TFLOP_per_s"], "peak": MFMA_BF16_PEAK_TFLOPS,
                                         "unit": "TFLOP/s", "frac": p["frac_mfma_peak"],
                                         "kernel": "prefill_mfma_kernel",
                                         "algorithmic_flops_per_launch": prefill_flops(batch)}

    cpu = None
    if not args.no_cpu_baseline and (R.has_dec or R.has_pre):
        log("cpu baseline (oracle) ...")
        pool = wl.host_bits(cache)                                  # exact bytes the GPU used
        if R.has_dec:
            cpu = cpu_baseline(batch, pool, args.cpu_budget * (0.5 if R.has_pre else 1.0))
        if R.has_pre:
            pre = cpu_prefill_baseline(batch, pool, args.cpu_budget * (0.5 if R.has_dec else 1.0))
            if cpu is None:
                cpu = dict(pre, kind="oracle", cpu_model=cpu_model())
            else:
                cpu["prefill"] = pre
        del pool

    cfg_info = {"workload": f"{W.name} (config {W.index}): {W.description}", "seed": W.seed,
                "num_tokens": batch.num_tokens, "prefill_rows": R.tp if R.has_pre else 0,
                "decode_seqs": int(len(batch.decode_seq_lens)), "parallelism": "single GPU"}
    R.free()
    del R, batch, cache
    if not args.no_configs:
        configs = {}
        for k in (1, 2, 3, 4, 5):
            if k != args.workload:
                configs[str(k)] = config_leg(pa, k, dev, args.steps, args.warmup)
        secondary["configs"] = configs

    line = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": L.dtype,
        "data": "synthetic",
        "config": cfg_info,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

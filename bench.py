#!/usr/bin/env python3
"""Paged KV-cache attention benchmark on one MI355X.

Workload: 8B-shaped grouped-query decode — 64 sequences, 32 q heads over 8 kv
heads, head_dim 128, bf16, block_size 16, lengths uniform in [512, 4096]
(seed 1001), blocks handed out from a shuffled pool of 1.1x the need.

One step is one decode step of that batch, through the C ABI:
  1. host block manager: every sequence grows by one token
     (pa_seq_append_batch) and gets its slot;
  2. pa_append_decode_args, with the step's slots and lengths passed from
     host arrays in the launch arguments (the block tables were uploaded once
     before the first step): the step's new K/V rows are scattered into the
     paged pool, each new token's block is entered in the device table, and
     the step's queries attend over their sequences, in the library's default
     KV partitions (pa_decode_partition_tokens: here 1536 tokens, 1-3 per
     sequence, merged by log-sum-exp).
``--unfused-step`` runs the same step as pa_write_kv + pa_decode with the
whole table exported (pa_block_tables) and uploaded every step.
The step's new K/V rows and queries are generated before timing and are
resident in HBM. W untimed warm-up steps, then K timed steps between two
device synchronisations.

Printed: one JSON line. ``value`` is the whole-step KV throughput (logical
K+V bytes the decode must read per step, over the step time). ``roofline``
is the decode op (pa_append_decode_args: partition + merge kernels), timed in every fourth timed
step with a pair of HIP events around the call on the stream it runs on (the
only events in the loop: a pair costs about 6 us of stream time, so the other
steps run without),
against 8 TB/s HBM. ``cpu_baseline`` is the CPU oracle
(fp64 gather + softmax attention) timed on this host on the same workload.
``prefill`` is the chunked causal prefill workload (16 x 512-token chunks
over U[0, 7680] cached tokens, bs 32) timed the same way against the bf16
MFMA peak. ``decode_fp8`` times pa_decode over an FP8 (E4M3) pool of the same
batch shape (seed 1006), with the bytes it must read (1-byte K/V codes).
``mixed_step`` runs serving steps that mix decode and chunked prefill
(pa_step eager, and the same step captured once as a HIP graph and replayed).
``prefix_cache`` times token-aware appends with block lookups against blind
appends and decodes the shared-prompt batch; ``tiered_block_sizes`` decodes
batches split into per-length-tier pools against one bs-16 pool;
``decode_skewed`` decodes a batch of short sequences with one very long one,
in the library's default partitions and in fixed 512-token ones.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode KV GB/s and % of HBM peak; decode tok/s at batch 64, 8B shape"
HBM_PEAK_GBPS = 8000.0
SAMPLE_STEPS = 60   # decode steps after the timed region, each between its own event pair
BF16_MFMA_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "decode": ["decode.hip", "device_common.h", "launch.h"],
    "decode_fp8": ["decode.hip", "device_common.h", "launch.h"],
    "decode_prefix": ["decode.hip", "device_common.h", "launch.h"],
    "prefill": ["prefill.hip", "device_common.h", "launch.h"],
}


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it does not write back and invalidate the caches at system
    scope, which costs stream time and delays the work after it (about 6 us
    per event pair around a decode launch with torch's default events). Same
    use as TimingEvent(): record(stream), then
    elapsed_time(later_event) in ms once the device is synchronised."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        import torch  # noqa: F401  (its HIP runtime is the one the library uses)
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self._ev = ctypes.c_void_p()
        if TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream) -> None:
        if TimingEvent._hip.hipEventRecord(self._ev, stream.cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end: "TimingEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        if TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        try:
            TimingEvent._hip.hipEventDestroy(self._ev)
        except Exception:
            pass


def settle(fn, seconds: float) -> None:
    """Run ``fn`` (GPU work, no side effects) back to back for about
    ``seconds`` before a timed leg: the GPU leaves its idle clocks over the
    first tens of milliseconds of load (measured: the prefill launch takes
    620 us in its first 30 launches, 540 us after about 90)."""
    import torch
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_calls(fn, n: int, stream) -> dict:
    """Time ``fn`` (one call of the op on ``stream``) two ways: n calls each
    between its own pair of fence-free HIP events (per-call samples: mean,
    median, min), then n calls back to back between one pair (the average
    time per call when the GPU runs them in a row, launch gaps included)."""
    import numpy as np
    import torch
    e0 = [TimingEvent() for _ in range(n)]
    e1 = [TimingEvent() for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        e0[i].record(stream)
        fn()
        e1[i].record(stream)
    r0, r1 = TimingEvent(), TimingEvent()
    r0.record(stream)
    for _ in range(n):
        fn()
    r1.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) for a, b in zip(e0, e1)]) * 1e3
    return {"calls": n, "us_mean": float(us.mean()), "us_median": float(np.median(us)), "us_min": float(us.min()),
            "us_back_to_back": r0.elapsed_time(r1) * 1e3 / n}


def blas_info() -> dict:
    """Thread count and vendor of the BLAS NumPy uses (the oracle's matmuls)."""
    import numpy as np
    info = {"threads": 1, "blas": "unknown"}
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        info["threads"] = max([1] + [int(i.get("num_threads", 1)) for i in pools])
        blas = [i for i in pools if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
    except Exception:
        pass
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        info["numpy_blas"] = f"{b.get('name')} {b.get('version')}"
    except Exception:
        pass
    return info


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(which: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[which]:
        with open(os.path.join(ROOT, "paged_kv_cache_indirect_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(which: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(PROFILES, f"{which}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(which):
        return None
    return float(m_bytes.group(1))


def decode_bytes(wl, lens) -> int:
    """Algorithmic bytes of one decode call: K+V rows of every valid token,
    q and out, the ceil(L / bs) table entries in use, and seq_lens."""
    import numpy as np
    L = np.asarray(lens, dtype=np.int64)
    kv = int(L.sum()) * wl.Hkv * wl.D * 2 * wl.kv_elem_bytes
    qo = 2 * wl.B * wl.Hq * wl.D * wl.elem_bytes
    tables = int(((L + wl.block_size - 1) // wl.block_size).sum()) * 4
    return kv + qo + tables + 4 * wl.B


# --------------------------------------------------------------------- decode
def run_decode(args):
    import numpy as np
    import torch

    import workloads as W
    from tests import harness
    from paged_kv_cache_indirect_amd import (pa_append_decode_args, pa_block_tables, pa_decode,
                                             pa_decode_partition_tokens, pa_decode_partition_tokens_for_lengths,
                                             pa_decode_workspace_bytes, pa_seq_append_batch, pa_write_kv)

    dev = torch.device("cuda:0")
    # warm-up steps, the timed steps, then SAMPLE_STEPS more steps each
    # between its own event pair (per-launch median and min)
    S = args.warmup + args.steps + SAMPLE_STEPS
    # The 8B-shaped batch (same lengths, values and queries), its shuffled
    # pool sized at 1.1x the blocks the sequences need after all S steps.
    base = W.config("gqa8b")
    need = sum(-(-(int(L) + S) // base.block_size) for L in base.seq_lens)
    wl = W.make_decode("gqa8b", base.seq_lens, Hq=base.Hq, Hkv=base.Hkv, D=base.D, block_size=base.block_size,
                       dtype=base.dtype, seed=base.seed, num_blocks=-(-11 * need // 10))
    log(f"[bench] building gqa8b cache: B={wl.B} nb={wl.num_blocks} max_len={wl.max_seq_len}")
    cache = harness.GpuCache(wl, device=dev, poison=False)
    pool = cache.pool
    B, Hq, Hkv, D, bs = wl.B, wl.Hq, wl.Hkv, wl.D, wl.block_size

    # Step inputs, resident in HBM before timing.
    ks, vs, qs = [], [], []
    for s in range(S):
        k, v, q = wl.decode_step_inputs(s)
        ks.append(k); vs.append(v); qs.append(q)
    k_steps = harness.to_device(np.stack(ks), wl.dtype, dev)    # [S, B, Hkv, D]
    v_steps = harness.to_device(np.stack(vs), wl.dtype, dev)
    q_steps = harness.to_device(np.stack(qs), wl.dtype, dev)    # [S, B, Hq, D]
    out = torch.empty((B, Hq, D), dtype=q_steps.dtype, device=dev)

    # Grid and table width sized once for the longest sequence after S steps.
    max_len = wl.max_seq_len + S
    max_blocks = -(-max_len // bs)
    pt = args.partition_tokens    # 0: the library's choice
    pt_used = pt or pa_decode_partition_tokens(pool, B, max_len)
    ws_bytes = pa_decode_workspace_bytes(B, Hq, D, max_len, pt)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    seq_ids = np.arange(B, dtype=np.int64)
    stream = torch.cuda.current_stream()
    # The timed steps run without events in between (one fence-free pair
    # brackets the whole region); the sample steps after them each have a
    # pair around the decode call.
    t_end = args.warmup + args.steps
    timed_events = set(range(t_end, S))
    ev_dec0 = {s: TimingEvent() for s in timed_events}
    ev_dec1 = {s: TimingEvent() for s in timed_events}
    region0, region1 = TimingEvent(), TimingEvent()
    lens_per_step = []
    ring = 2

    if not args.unfused_step:
        # Fused step: the device tables are uploaded once; each step's slots
        # and lengths travel in the launch arguments of pa_append_decode_args
        # (no host-to-device copy per step), which scatters the new rows,
        # enters each new token's block in the device table and decodes.
        tables0, lens0 = pa_block_tables(pool, seq_ids, max_blocks)
        tab_d = torch.from_numpy(tables0).to(dev)
        lens_host = lens0.astype(np.int32)
        slots_h = np.empty((B, 1), dtype=np.int64)
        torch.cuda.synchronize()

        def step(s: int) -> None:
            pa_seq_append_batch(pool, seq_ids, 1, slots_h)
            lens_host[:] += 1
            lens_per_step.append(lens_host.copy())
            if s in ev_dec0:
                ev_dec0[s].record(stream)
            pa_append_decode_args(pool, out, q_steps[s], k_steps[s], v_steps[s], slots_h, tab_d, lens_host,
                                  wl.scale, max_len, pt, workspace)
            if s in ev_dec1:
                ev_dec1[s].record(stream)
    else:
        # Separate scatter and decode, with the whole table exported and
        # uploaded every step.
        # Packed per-step metadata: slots int64 [B] | seq_lens int32 [B] | tables int32 [B, max_blocks].
        off_lens = 8 * B
        off_tab = off_lens + 4 * B
        nbytes = off_tab + 4 * B * max_blocks
        pinned = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(ring)]
        dmeta = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(ring)]
        copied = [torch.cuda.Event() for _ in range(ring)]
        host_views = []
        for p in pinned:
            a = p.numpy()
            host_views.append((a[:off_lens].view(np.int64), a[off_lens:off_tab].view(np.int32),
                               a[off_tab:].view(np.int32)))
        dev_views = [(d[:off_lens].view(torch.int64), d[off_lens:off_tab].view(torch.int32),
                      d[off_tab:].view(torch.int32).view(B, max_blocks)) for d in dmeta]

        def step(s: int) -> None:
            r = s % ring
            copied[r].synchronize()                    # pinned[r]'s previous copy has landed
            slots_h, lens_h, tab_h = host_views[r]
            pa_seq_append_batch(pool, seq_ids, 1, slots_h)
            pa_block_tables(pool, seq_ids, max_blocks, tab_h, lens_h)
            lens_per_step.append(lens_h.copy())
            dmeta[r].copy_(pinned[r], non_blocking=True)
            copied[r].record(stream)
            slots_d, lens_d, tab_d = dev_views[r]
            pa_write_kv(pool, k_steps[s], v_steps[s], slots_d)
            if s in ev_dec0:
                ev_dec0[s].record(stream)
            pa_decode(pool, out, q_steps[s], tab_d, lens_d, wl.scale, max_len, pt, workspace)
            if s in ev_dec1:
                ev_dec1[s].record(stream)

    settle_ws = cache.workspace_for(pt)
    settle(lambda: cache.decode(pt, settle_ws), 0.05)   # read-only decodes of the built cache
    del settle_ws
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    log(f"[bench] warm-up done ({args.warmup} steps); timing {args.steps} steps")
    t0 = time.perf_counter()
    region0.record(stream)
    for s in range(args.warmup, t_end):
        step(s)
    region1.record(stream)
    host_s = time.perf_counter() - t0          # host side of the steps (launches are asynchronous)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"[bench] timed decode steps done: {elapsed * 1e3:.2f} ms (host {host_s * 1e3:.2f} ms)")
    for s in range(t_end, S):
        step(s)
    torch.cuda.synchronize()

    timed = range(args.warmup, t_end)
    sampled = sorted(timed_events)
    dec_ms = [ev_dec0[s].elapsed_time(ev_dec1[s]) for s in sampled]
    step_bytes = [decode_bytes(wl, lens_per_step[s]) for s in timed]
    step_kv = [int(np.asarray(lens_per_step[s], np.int64).sum()) * Hkv * D * 2 * wl.elem_bytes
               for s in timed]
    region_us = region0.elapsed_time(region1) * 1e3 / args.steps   # GPU time per step, steps back to back
    achieved = float(np.mean(step_bytes)) / (region_us * 1e-6) / 1e9
    res = {
        "elapsed_s": elapsed,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "host_us_per_step": host_s * 1e6 / args.steps,
        "value": sum(step_kv) / elapsed / 1e9,
        "tok_per_s": B * args.steps / elapsed,
        "region_us_per_launch": region_us,
        "event_samples": len(dec_ms),
        "decode_us_mean": float(np.mean(dec_ms)) * 1e3,
        "decode_us_median": float(np.median(dec_ms)) * 1e3,
        "decode_us_min": float(np.min(dec_ms)) * 1e3,
        "bytes_per_launch": float(np.mean(step_bytes)),
        "kv_bytes_per_step": float(np.mean(step_kv)),
        "achieved_gbps": achieved,
        "partition_tokens": pt_used if (pt or args.unfused_step) else
        sorted({pa_decode_partition_tokens_for_lengths(pool, lens_per_step[s], max_len) for s in timed}),
        "mean_len": float(np.mean([np.mean(lens_per_step[s]) for s in timed])),
        "max_len_bound": max_len,
        "num_blocks": wl.num_blocks,
    }
    cache.close()
    del cache, k_steps, v_steps, q_steps, workspace
    torch.cuda.empty_cache()
    return wl, res


# ------------------------------------------------------------ every config
def oracle_decode_seconds(wl, min_seconds: float = 1.0):
    """The oracle's fp64 paged decode of the whole batch on this host (cache
    built first, not timed), repeated until ``min_seconds`` have passed;
    returns (seconds per batch, repetitions)."""
    import oracle.attention as OA
    from oracle.cache import OracleCache
    ora = OracleCache(wl, poison=False)
    q = wl.queries()
    reps, total = 0, 0.0
    while reps == 0 or total < min_seconds:
        t0 = time.perf_counter()
        OA.paged_decode(q, ora.k_cache, ora.v_cache, ora.block_tables, ora.seq_lens, wl.scale, wl.dtype)
        total += time.perf_counter() - t0
        reps += 1
    return total / reps, reps


def run_configs(args):
    """The decode configurations, each as configured: the tiny fp32 batch
    (latency), the 8B-shaped batch as a plain read-only pa_decode in the
    library's partition, the long-context batch in 512-token partitions and
    in the library's partition, and the shared-prefix batch (logical and
    unique K/V bytes). Each GPU figure is over at least 50 calls; each config
    also times the CPU oracle on the same batch once (``--no-cpu-baseline``
    skips those)."""
    import numpy as np
    import torch

    import workloads as W
    from tests import harness
    from paged_kv_cache_indirect_amd import pa_decode_partition_tokens

    n = max(50, args.config_calls)
    stream = torch.cuda.current_stream()
    out = {}
    plan = [("C1_tiny", "tiny", [0]), ("C2_gqa8b", "gqa8b", [0]), ("C3_long", "long", [512, 0]),
            ("C4_prefix", "prefix", [0])]
    for key, name, pts in plan:
        wl = W.config(name)
        log(f"[bench] config {key}: B={wl.B} max_len={wl.max_seq_len} {wl.dtype}")
        cache = harness.GpuCache(wl, poison=False)
        nbytes = decode_bytes(wl, wl.seq_lens)
        res = {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "D": wl.D, "block_size": wl.block_size,
               "dtype": wl.dtype, "seed": wl.seed, "mean_len": float(np.mean(wl.seq_lens)),
               "bytes_per_call": nbytes, "kv_bytes": wl.kv_bytes()}
        if wl.prefix_len:
            res["unique_kv_bytes"] = wl.unique_kv_bytes()
            res["hbm_bytes_per_call_measured"] = measured_traffic("decode_prefix")
        for pt in pts:
            ws = cache.workspace_for(pt)
            settle(lambda: cache.decode(pt, ws), 0.05)
            t = time_calls(lambda: cache.decode(pt, ws), n, stream)
            used = pt or pa_decode_partition_tokens(cache.pool, wl.B, wl.max_seq_len)
            sec = t["us_back_to_back"] * 1e-6
            leg = dict(t, partition_tokens=used, gbps=nbytes / sec / 1e9,
                       frac=nbytes / sec / 1e9 / HBM_PEAK_GBPS, tok_per_s=wl.B / sec)
            if wl.prefix_len:
                leg["unique_gbps"] = wl.unique_kv_bytes() / sec / 1e9
            res["partition_" + ("default" if pt == 0 else str(pt))] = leg
            log(f"[bench]   pt {used}: {t['us_back_to_back']:.1f} us/call back to back, "
                f"{t['us_median']:.1f} us median per call, {leg['gbps']:.0f} GB/s")
        cache.close()
        del cache
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            sec, reps = oracle_decode_seconds(wl, 0.5)
            res["cpu_oracle"] = {"seconds_per_batch": sec, "repetitions": reps, "gbps": nbytes / sec / 1e9,
                                 "tok_per_s": wl.B / sec, **blas_info()}
            log(f"[bench]   cpu oracle: {sec:.2f} s per batch")
        wl.drop_cached()
        out[key] = res
    return out


# ----------------------------------------------------------------- FP8 decode
def run_decode_fp8(args):
    """pa_decode over an FP8 (E4M3) pool of the 8B-shaped batch: back-to-back
    launches bracketed by HIP events on the launch stream."""
    import numpy as np
    import torch

    import workloads as W
    from tests import harness

    dev = torch.device("cuda:0")
    from paged_kv_cache_indirect_amd import pa_decode_partition_tokens

    wl = W.config("gqa8b_fp8")
    log(f"[bench] building gqa8b_fp8 cache: B={wl.B} nb={wl.num_blocks}")
    cache = harness.GpuCache(wl, device=dev, poison=False)
    pt = args.partition_tokens    # 0: the library's choice
    pt_used = pt or pa_decode_partition_tokens(cache.pool, wl.B, wl.max_seq_len)
    ws = cache.workspace_for(pt)
    settle(lambda: cache.decode(pt, ws), 0.05)
    stream = torch.cuda.current_stream()
    tm = time_calls(lambda: cache.decode(pt, ws), max(50, args.config_calls), stream)
    t = tm["us_back_to_back"] * 1e-6
    nbytes = decode_bytes(wl, wl.seq_lens)
    gbps = nbytes / t / 1e9
    cache.close()
    log(f"[bench] fp8 decode: {t * 1e6:.1f} us back to back, {gbps:.0f} GB/s")
    return {
        "workload": "8B-shaped GQA decode over an FP8 (OCP E4M3) pool: batch 64, 32 q / 8 kv heads, "
                    "head_dim 128, bf16 q/out, block_size 16, lengths U[512,4096] (seed 1006), "
                    "per-tensor scales k 0.0137 / v 0.0129",
        "partition_tokens": pt_used, **tm,
        "tok_per_s": wl.B / t,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": measured_traffic("decode_fp8"),
                     "bytes_per_launch": nbytes},
    }


def run_decode_skewed(args):
    """A batch whose one long sequence dominates (63 x 512 tokens + 1 x 32768,
    8B-shaped heads): pa_decode in the library's default partition (chosen by
    the kernel from the device lengths) and in a fixed 512, and
    pa_append_decode_args (lengths on the host, no new tokens) in its
    length-based default."""
    import numpy as np
    import torch

    import workloads as W
    from tests import harness
    from paged_kv_cache_indirect_amd import (pa_append_decode_args, pa_decode_partition_tokens,
                                             pa_decode_partition_tokens_for_lengths)

    wl = W.make_decode("skewed", [512] * 63 + [32768], Hq=32, Hkv=8, D=128, block_size=16, dtype="bf16", seed=77)
    cache = harness.GpuCache(wl, poison=False)
    res = {"workload": "63 x 512-token sequences + 1 x 32768, Hq 32 / Hkv 8, D 128, bf16, bs 16 (seed 77)"}
    stream = torch.cuda.current_stream()
    for label, pt in (("default", 0), ("fixed_512", 512)):
        ws = cache.workspace_for(pt)
        for _ in range(3):
            cache.decode(pt, ws)
        n = 20
        e0, e1 = TimingEvent(), TimingEvent()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            cache.decode(pt, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / n * 1e-3
        nbytes = decode_bytes(wl, wl.seq_lens)
        # partition_tokens 0: chosen by the kernel from the device lengths (max_seq_len >= 8192),
        # the same partition the host rule gives for these lengths
        used = pt or pa_decode_partition_tokens_for_lengths(cache.pool, wl.seq_lens, wl.max_seq_len)
        res[label] = {"partition_tokens": used, "us_mean": t * 1e6, "gbps": nbytes / t / 1e9,
                      "frac": nbytes / t / 1e9 / HBM_PEAK_GBPS}
    # Lengths on the host: the partition comes from the lengths themselves.
    lens = np.asarray(wl.seq_lens, dtype=np.int32)
    no_slots = np.full(wl.B, -1, dtype=np.int64)
    rows = torch.zeros((wl.B, wl.Hkv, wl.D), dtype=torch.bfloat16, device="cuda")
    ws = cache.workspace_for(0)

    def host_call():
        pa_append_decode_args(cache.pool, cache.out, cache.q, rows, rows, no_slots, cache.block_tables, lens,
                              wl.scale, wl.max_seq_len, 0, ws)
    for _ in range(3):
        host_call()
    n = 20
    e0, e1 = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        host_call()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / n * 1e-3
    nbytes = decode_bytes(wl, wl.seq_lens)
    res["host_lengths"] = {"partition_tokens": pa_decode_partition_tokens_for_lengths(cache.pool, lens, wl.max_seq_len),
                           "us_mean": t * 1e6, "gbps": nbytes / t / 1e9, "frac": nbytes / t / 1e9 / HBM_PEAK_GBPS}
    cache.close()
    log(f"[bench] skewed batch: default pt {res['default']['partition_tokens']} {res['default']['us_mean']:.1f} us, "
        f"pt 512 {res['fixed_512']['us_mean']:.1f} us, host lengths pt {res['host_lengths']['partition_tokens']} "
        f"{res['host_lengths']['us_mean']:.1f} us")
    return res


# ----------------------------------------------------------------- mixed step
def run_mixed(args):
    """Mixed serving steps (decode + chunked prefill + the scatter of all new
    rows) through pa_step (eager) and through a captured step graph, each on
    its own pool; GPU time per step from HIP events around the launch, host
    time per step (block manager appends, table export, metadata uploads,
    launch) by clock; the steps' K/V rows and queries are staged in HBM first."""
    import numpy as np
    import torch

    import workloads as W
    from tests import harness

    wl = W.config("mixed")
    p = wl.plan
    res = {}
    runs = 2                                         # fresh pools per run; the steps of both are averaged
    for mode in ("eager", "graph"):
        log(f"[bench] mixed step ({mode}): Bd={p['Bd']} Bp={p['Bp']} chunk={p['chunk']} steps={p['steps']} "
            f"runs={runs}")
        gpu_ms, host_ms, prep_ms, launch_ms, steps_bytes, steps_flops = [], [], [], [], [], []
        for _ in range(runs):
            run = harness.MixedRunner(wl, use_graph=(mode == "graph"))
            run.stage_inputs()                       # step inputs resident in HBM before timing
            stream = torch.cuda.current_stream()
            for s in range(p["steps"]):
                t0 = time.perf_counter()
                run.prepare(s)
                t1 = time.perf_counter()
                e0, e1 = TimingEvent(), TimingEvent()
                e0.record(stream)
                run.launch()
                e1.record(stream)
                t2 = time.perf_counter()
                host = (t2 - t0) * 1e3
                torch.cuda.synchronize()
                if s < 2:                            # the first two steps warm up (and capture)
                    continue
                host_ms.append(host)
                prep_ms.append((t1 - t0) * 1e3)
                launch_ms.append((t2 - t1) * 1e3)
                gpu_ms.append(e0.elapsed_time(e1))
                lens = run.host_lens
                dl = lens[:p["Bd"]].astype(np.int64)
                steps_bytes.append(int(dl.sum()) * wl.Hkv * wl.D * 2 * wl.elem_bytes +
                                   run.T * wl.Hkv * wl.D * 2 * 2 * wl.elem_bytes)
                ctx = lens[p["Bd"]:].astype(np.int64) - p["chunk"]
                n = p["chunk"]
                steps_flops.append(4.0 * wl.D * wl.Hq * float(np.sum(n * ctx + n * (n + 1) // 2)))
            run.close()
        t = float(np.mean(gpu_ms)) * 1e-3
        floor = float(np.mean(steps_bytes)) / (HBM_PEAK_GBPS * 1e9) + \
            float(np.mean(steps_flops)) / (BF16_MFMA_PEAK_TFLOPS * 1e12)
        # host time = the harness's preparation (block-manager appends, table
        # export, input uploads) + the launch call (pa_step or the graph launch)
        res[mode] = {"gpu_us_per_step": t * 1e6, "host_us_per_step": float(np.mean(host_ms)) * 1e3,
                     "host_prepare_us_per_step": float(np.mean(prep_ms)) * 1e3,
                     "host_launch_us_per_step": float(np.mean(launch_ms)) * 1e3,
                     "roofline_floor_us": floor * 1e6, "frac_of_floor": floor / t, "timed_steps": len(gpu_ms)}
    res["workload"] = ("mixed serving step: 56 decode sequences U[512,4096] + 8 chunked-prefill sequences "
                       "(256-token chunks over cached context U[0,4096]), Hq 32 / Hkv 8, D 128, bf16, bs 16 "
                       "(seed 1007); step = scatter of all new rows + decode + prefill")
    res["floor"] = ("decode K/V + scatter bytes at 8 TB/s plus causal prefill flops at 2.5 PFLOP/s, "
                    "per step")
    log(f"[bench] mixed step: eager {res['eager']['gpu_us_per_step']:.1f} us, "
        f"graph {res['graph']['gpu_us_per_step']:.1f} us")
    return res


# --------------------------------------------------- prefix cache and tiers
def run_prefix_cache(args):
    """Host cost and effect of prefix caching: the 48-request shared-prompt
    batch appended with token ids (pa_seq_append_tokens: hashing, lookups,
    shared blocks) versus the same token counts appended blind
    (pa_seq_append), on two empty pools; then decode over the cached pool."""
    import numpy as np
    import torch

    import workloads as W
    from tests import harness
    from paged_kv_cache_indirect_amd import (pa_alloc_pool, pa_decode_partition_tokens, pa_free_pool,
                                             pa_pool_prefix_stats,
                                             pa_pool_stats, pa_seq_append, pa_seq_append_tokens)

    wl = W.config("prompt_cache")
    blind_need = int(sum(-(-int(L) // wl.block_size) for L in wl.seq_lens))   # no sharing at all
    shape = (blind_need, wl.block_size, wl.Hkv, wl.D)
    kc = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    res = {"workload": "48 requests sharing a 1000-token prompt plus own tokens U[1,600] (seed 1008), bs 16"}
    ntok = int(sum(len(op[2]) for op in wl.ops))
    for mode in ("tokens", "blind"):
        best = None
        for _ in range(5):
            pool = pa_alloc_pool(kc, vc)
            t0 = time.perf_counter()
            for op in wl.ops:
                if mode == "tokens":
                    pa_seq_append_tokens(pool, op[1], op[2])
                else:
                    pa_seq_append(pool, op[1], len(op[2]))
            dt = time.perf_counter() - t0
            st = pa_pool_stats(pool)
            ps = pa_pool_prefix_stats(pool)
            pa_free_pool(pool)
            best = dt if best is None else min(best, dt)
        res[mode] = {"host_ns_per_token": best / ntok * 1e9, "used_blocks": st["used_blocks"],
                     "shared_blocks": st["shared_blocks"]}
        if mode == "tokens":
            res[mode].update({"lookups": ps["lookups"], "hits": ps["hits"], "cached_blocks": ps["cached_blocks"]})
    del kc, vc
    torch.cuda.empty_cache()
    cache = harness.GpuCache(wl, poison=False)
    ppt = 0      # the library's choice
    ppt_used = pa_decode_partition_tokens(cache.pool, wl.B, wl.max_seq_len)
    ws = cache.workspace_for(ppt)
    for _ in range(3):
        cache.decode(ppt, ws)
    n = 20
    stream = torch.cuda.current_stream()
    e0 = [TimingEvent() for _ in range(n)]
    e1 = [TimingEvent() for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        e0[i].record(stream)
        cache.decode(ppt, ws)
        e1[i].record(stream)
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b) for a, b in zip(e0, e1)])) * 1e-3
    nbytes = decode_bytes(wl, wl.seq_lens)
    cache.close()
    res["decode"] = {"partition_tokens": ppt_used, "us_mean": t * 1e6, "logical_gbps": nbytes / t / 1e9,
                     "unique_kv_bytes": wl.unique_kv_bytes(), "logical_kv_bytes": wl.kv_bytes()}
    log(f"[bench] prefix cache: {res['tokens']['host_ns_per_token']:.0f} ns/token with lookups, "
        f"{res['blind']['host_ns_per_token']:.0f} blind; decode {t * 1e6:.1f} us")
    return res


def run_tiered(args):
    """Block-size tiers by length class: each batch split into per-tier pools
    (pa_tier_block_size) and decoded with one pa_decode per pool on one
    stream, against the same batch in one bs-16 pool. Tail waste from the
    block manager's slot counts."""
    import numpy as np
    import torch

    import workloads as W
    from tests import harness
    from paged_kv_cache_indirect_amd import pa_pool_stats, pa_tier_block_size

    out = {}
    for name in ("gqa8b", "long"):
        base = W.config(name)
        groups = {}
        for L in base.seq_lens.tolist():
            groups.setdefault(pa_tier_block_size(L), []).append(L)
        layouts = {"single_bs16": [(16, base.seq_lens.tolist())], "tiered": sorted(groups.items())}
        res = {}
        for label, parts in layouts.items():
            caches = []
            for i, (bs, lens) in enumerate(parts):
                wl = W.make_decode(f"{name}_{label}_{bs}", lens, Hq=32, Hkv=8, D=128, block_size=bs, dtype="bf16",
                                   seed=base.seed + 100 * (i + 1))
                caches.append((wl, harness.GpuCache(wl, poison=False)))
            wss = [c.workspace_for(0) for _, c in caches]
            for _ in range(3):
                for (_, c), w in zip(caches, wss):
                    c.decode(0, w)
            n = 20
            stream = torch.cuda.current_stream()
            e0, e1 = TimingEvent(), TimingEvent()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n):
                for (_, c), w in zip(caches, wss):
                    c.decode(0, w)
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / n * 1e-3
            nbytes = sum(decode_bytes(wl, wl.seq_lens) for wl, _ in caches)
            alloc = sum(pa_pool_stats(c.pool)["allocated_slots"] for _, c in caches)
            filled = sum(pa_pool_stats(c.pool)["filled_slots"] for _, c in caches)
            res[label] = {"block_sizes": [bs for bs, _ in parts], "seqs_per_pool": [len(l) for _, l in parts],
                          "us_per_batch": t * 1e6, "gbps": nbytes / t / 1e9, "frac": nbytes / t / 1e9 / HBM_PEAK_GBPS,
                          "tail_waste_slots": alloc - filled, "tail_waste_frac": (alloc - filled) / alloc}
            for _, c in caches:
                c.close()
            del caches
            torch.cuda.empty_cache()
        out[name] = res
        log(f"[bench] tiers {name}: single {res['single_bs16']['us_per_batch']:.1f} us, "
            f"tiered {res['tiered']['us_per_batch']:.1f} us")
    return out


# -------------------------------------------------------------------- prefill
def causal_flops(wl) -> float:
    """4 * D * Hq * sum_b sum_i (ctx_b + i + 1): QK^T and PV over the
    causally valid (query, key) pairs only."""
    total = 0
    for L, n in zip(wl.seq_lens.tolist(), wl.q_lens.tolist()):
        ctx = L - n
        total += n * ctx + n * (n + 1) // 2
    return 4.0 * wl.D * wl.Hq * total


def run_prefill(args):
    import numpy as np
    import torch

    import workloads as W
    from tests import harness
    from paged_kv_cache_indirect_amd import PaError

    dev = torch.device("cuda:0")
    wl = W.config("prefill")
    log(f"[bench] building prefill cache: B={wl.B} T={int(wl.q_lens.sum())} nb={wl.num_blocks}")
    cache = harness.GpuCache(wl, device=dev, poison=False)
    try:
        cache.prefill()
    except PaError as e:
        cache.close()
        return wl, {"status": f"unavailable: {e}"}
    torch.cuda.synchronize()
    n = max(50, args.prefill_iters)
    settle(cache.prefill, 0.1)
    stream = torch.cuda.current_stream()
    tm = time_calls(cache.prefill, n, stream)
    flops = causal_flops(wl)
    t = tm["us_back_to_back"] * 1e-6
    tflops = flops / t / 1e12
    cache.close()
    log(f"[bench] prefill: {t * 1e6:.1f} us back to back, {tm['us_median']:.1f} us median per call, "
        f"{tflops:.1f} TFLOP/s")
    traffic = measured_traffic("prefill")
    res = {
        "workload": "16 x 512-token causal chunks over paged context U[0,7680] (seed 1004), "
                    "Hq 32 / Hkv 8, D 128, bf16, block_size 32",
        "calls": n, "us_back_to_back": tm["us_back_to_back"], "us_mean": tm["us_mean"],
        "us_median": tm["us_median"], "us_min": tm["us_min"],
        "tokens_per_s": int(wl.q_lens.sum()) / t,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "traffic": traffic,
                     "flops_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        import oracle.attention as OA
        from oracle.cache import OracleCache
        ora = OracleCache(wl, poison=False)
        t0 = time.perf_counter()
        OA.paged_prefill_masked(wl.queries(), wl.cu_q_lens(), ora.k_cache, ora.v_cache, ora.block_tables,
                                ora.seq_lens, wl.scale, wl.dtype)
        sec = time.perf_counter() - t0
        res["cpu_oracle"] = {"seconds": sec, "gflops": flops / sec / 1e9, **blas_info(),
                             "what": "oracle's matrix-form fp64 causal prefill of the whole workload, once"}
        log(f"[bench] prefill cpu oracle: {sec:.1f} s ({flops / sec / 1e9:.1f} GFLOP/s)")
        del ora
    wl.drop_cached()
    return wl, res


# --------------------------------------------------------------- CPU oracle
def run_cpu_baseline(args, wl):
    """The oracle's fp64 paged decode of the same 64-sequence batch (cache as
    built before the timed steps), repeated for about ``cpu_seconds``."""
    import numpy as np

    import oracle.attention as OA
    from oracle.cache import OracleCache

    log("[bench] cpu baseline: building oracle cache")
    ora = OracleCache(wl, poison=False)
    q = wl.queries()
    nbytes = decode_bytes(wl, ora.seq_lens)
    kv = int(ora.seq_lens.astype(np.int64).sum()) * wl.Hkv * wl.D * 2 * wl.elem_bytes
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
    except Exception:
        pass
    reps, t_total = 0, 0.0
    while reps == 0 or (t_total < args.cpu_seconds and reps < 100):
        t0 = time.perf_counter()
        OA.paged_decode(q, ora.k_cache, ora.v_cache, ora.block_tables, ora.seq_lens, wl.scale, wl.dtype)
        t_total += time.perf_counter() - t0
        reps += 1
        log(f"[bench] cpu baseline rep {reps}: {t_total:.1f} s")
    t = t_total / reps
    info = blas_info()
    return {
        "value": kv / t / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle", "blas": info.get("blas"),
        "numpy_blas": info.get("numpy_blas"),
        "sample": f"full 64-sequence decode batch (one step, mean length {float(ora.seq_lens.mean()):.0f}), "
                  f"fp64 NumPy gather + exact softmax attention, {reps} repetition(s), {t:.2f} s each; "
                  f"host has {len(os.sched_getaffinity(0))} cores available",
        "tok_per_s": wl.B / t,
        "bytes_per_call": nbytes,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--unfused-step", action="store_true",
                    help="decode step as pa_write_kv + whole-table upload + pa_decode (default: pa_append_decode_args)")
    ap.add_argument("--partition-tokens", type=int, default=0,
                    help="KV partition of the decode legs (0: the library's choice, pa_decode_partition_tokens)")
    ap.add_argument("--prefill-iters", type=int, default=50, help="prefill calls timed (at least 50)")
    ap.add_argument("--config-calls", type=int, default=50, help="calls timed per config leg (at least 50)")
    ap.add_argument("--legs", default="all",
                    help="comma list of legs to run besides the headline decode step: configs, prefill, fp8, "
                         "mixed, extras, cpu (default all)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-cache decode leg")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed-step (eager vs graph) leg")
    ap.add_argument("--no-extras", action="store_true", help="skip the prefix-cache and block-size-tier legs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before the decode steps, run one plain 1 GiB device-to-device copy: "
                         "the reference that scales hardware byte counters (FETCH_SIZE, WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(every workload here runs on a single MI355X); run with --gpus 1.", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        return 2
    import paged_kv_cache_indirect_amd  # noqa: F401  (fails loudly if libpa.so is missing)

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")   # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 1073741824 bytes read, 1073741824 bytes written")
        del src, dst
        torch.cuda.empty_cache()

    legs = {"configs", "prefill", "fp8", "mixed", "extras", "cpu"} if args.legs == "all" else \
        set(x.strip() for x in args.legs.split(",") if x.strip())
    if args.no_prefill:
        legs.discard("prefill")
    if args.no_fp8:
        legs.discard("fp8")
    if args.no_mixed:
        legs.discard("mixed")
    if args.no_extras:
        legs.discard("extras")
    if args.no_cpu_baseline:
        legs.discard("cpu")
    args.no_cpu_baseline = "cpu" not in legs

    wl, dec = run_decode(args)
    frac = dec["achieved_gbps"] / HBM_PEAK_GBPS
    log(f"[bench] decode: {dec['region_us_per_launch']:.1f} us/launch back to back "
        f"({dec['decode_us_median']:.1f} us median per launch), {dec['achieved_gbps']:.0f} GB/s "
        f"({100 * frac:.1f}% of HBM peak); step {dec['ms_per_step'] * 1e3:.1f} us")
    configs = run_configs(args) if "configs" in legs else None
    pre = run_prefill(args)[1] if "prefill" in legs else None
    if configs is not None and pre is not None:
        configs["C5_prefill"] = {k: v for k, v in pre.items() if k != "roofline"}
        configs["C5_prefill"]["frac"] = pre["roofline"]["frac"]
        configs["C5_prefill"]["tflops"] = pre["roofline"]["achieved"]
    fp8 = run_decode_fp8(args) if "fp8" in legs else None
    mixed = run_mixed(args) if "mixed" in legs else None
    pcache = run_prefix_cache(args) if "extras" in legs else None
    tiers = run_tiered(args) if "extras" in legs else None
    skewed = run_decode_skewed(args) if "extras" in legs else None
    cpu = run_cpu_baseline(args, wl) if "cpu" in legs else None

    line = {
        "metric": METRIC,
        "value": dec["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "8B-shaped GQA paged decode step: batch 64, 32 q / 8 kv heads, head_dim 128, "
                        "bf16, block_size 16, lengths U[512,4096] (seed 1001), shuffled pool of 1.1x need; "
                        + ("step = block-manager append + table export/H2D + KV scatter + decode"
                           if args.unfused_step else
                           "step = block-manager append + fused KV scatter, table fill-in and decode with "
                           "slots/lengths in the launch arguments (pa_append_decode_args)") + " (library's KV partitions)",
            "global_batch": wl.B,
            "partition_tokens": dec["partition_tokens"],
            "mean_seq_len": dec["mean_len"],
        },
        "decode": {
            "tok_per_s": dec["tok_per_s"],
            "tok_per_s_8b_32_layers": dec["tok_per_s"] / 32.0,
            "launch_us_back_to_back": dec["region_us_per_launch"],
            "launch_us_mean": dec["decode_us_mean"],
            "launch_us_median": dec["decode_us_median"],
            "launch_us_min": dec["decode_us_min"],
            "event_timed_launches": dec["event_samples"],
            "kv_gbps_kernel": dec["kv_bytes_per_step"] / (dec["region_us_per_launch"] * 1e-6) / 1e9,
            "host_us_per_step": dec["host_us_per_step"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": dec["achieved_gbps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": frac,
            "traffic": None if args.unfused_step else measured_traffic("decode"),
            "kernel": ("paged decode (DecodeKernel; log-sum-exp MergeKernel only for sequences split into partitions)"
                       if args.unfused_step else
                       "fused append + paged decode (DecodeKernel with the step's new rows; log-sum-exp "
                       "MergeKernel only for sequences split into partitions)"),
            "bytes_per_launch": dec["bytes_per_launch"],
            "timing": "timed steps back to back between one pair of fence-free HIP events on the launch "
                      "stream; achieved = algorithmic bytes per launch / (region time / steps)",
        },
        "cpu_baseline": cpu,
        "configs": configs,
        "prefill": pre,
        "decode_fp8": fp8,
        "mixed_step": mixed,
        "prefix_cache": pcache,
        "tiered_block_sizes": tiers,
        "decode_skewed": skewed,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

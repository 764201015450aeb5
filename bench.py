#!/usr/bin/env python3
"""Benchmark: paged decode attention on one MI355X.

One step = the whole hot path over one batch: the cache write of every
sequence's newest token and single-token paged decode attention over the
cache that holds it.  By default one pa_decode_append call does both (the
stream-K kernel stores each new token just before it streams that tile,
then the combine kernel); --step separate runs pa_reshape_and_cache, then
pa_decode.
Default workload: the LLaMA-2-70B-shaped batch (B 64, Hq 64, Hkv 8, D 128,
bf16, 16-token blocks, mixed lengths 50..8000, shuffled physical blocks),
seeded and synthetic, resident in HBM before the timed region starts;
--config picks one of the other parity workloads instead.

Prints one JSON line.  `value` is effective GB/s over the whole step
(algorithmic bytes / step time); `roofline` reports the decode call against
the 8 TB/s HBM peak; `cpu_baseline` times the fp64 oracle on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
def traffic_file(config: str) -> str:
    """Counter-derived HBM traffic record of the decode call on a workload."""
    return os.path.join(ROOT, "profiles", f"traffic_decode_{config}.json")
KERNEL_SOURCES = ["decode_kernels.hip", "device_common.h", "launch.h", "api.hip"]
DECODE_KERNELS = ("decode_mfma_kernel", "decode_streamk_reduce_kernel")
CALIBRATION_BYTES = 1 << 30  # the plain copy run after the profiled decode calls


def workloads_is_kv8(kv_dtype) -> bool:
    """8-bit KV storage types (E4M3 or E5M2 codes)."""
    return kv_dtype in ("fp8_e4m3", "fp8_e5m2")


def algorithmic_bytes(case) -> dict:
    """Bytes the decode must move at minimum: every resident K and V row once,
    query in, output out, block-table entries and lengths."""
    s_act = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
    s_kv = 1 if workloads_is_kv8(getattr(case, "kv_dtype", None)) else s_act
    lens = case.context_lens.astype(np.int64)
    if case.ring is not None:
        lens = np.minimum(lens, case.ring.sink + case.ring.window)
    row = case.num_kv_heads * case.head_dim * 2 * s_kv  # one token's K and V rows, all KV heads
    kv = int(lens.sum()) * row
    # rows that several sequences reach through the same physical block (a
    # shared prefix) are counted once in the unique figure
    seen = set()
    for b, n in enumerate(lens):
        for blk in range(-(-int(n) // case.block_size)):
            rows = min(case.block_size, int(n) - blk * case.block_size)
            seen.add((int(case.block_tables[b, blk]), rows))
    unique_rows = {}
    for phys, rows in seen:
        unique_rows[phys] = max(rows, unique_rows.get(phys, 0))
    kv_unique = sum(unique_rows.values()) * row
    qo = case.num_seqs * case.num_q_heads * case.head_dim * 2 * s_act
    tables = int(sum(-(-int(n) // case.block_size) for n in lens)) * 4 + case.num_seqs * 4
    write = case.num_seqs * case.num_kv_heads * case.head_dim * 2 * (s_act + s_kv)  # K and V rows in + codes out
    # a decode call that also stores the new rows reads them once (from the
    # inputs) and writes them once on top of the decode's own bytes
    write_out = case.num_seqs * case.num_kv_heads * case.head_dim * 2 * s_kv
    return {"decode": kv_unique + qo + tables, "decode_logical": kv + qo + tables, "kv": kv,
            "kv_unique": kv_unique, "write": write, "write_out": write_out, "tokens": int(lens.sum())}


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_145_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(config: str, step: str):
    """Counter-derived HBM bytes per decode call, if taken on the current
    kernels with the same kind of step."""
    try:
        with open(traffic_file(config)) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash() or t.get("step", "separate") != step:
        return None
    return t.get("bytes_per_call")


def _counter_rows(path):
    import csv

    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def summarize_counters(fetch_csv: str, write_csv: str, command: str) -> dict:
    """HBM bytes per decode call from two rocprofv3 --pmc runs of
    ``bench.py --profile-calls N`` (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch).  Each counter is scaled by what it reads for the 1 GiB copy
    that the profiled run ends with."""
    out = {"kernel_hash": kernel_hash(), "command": command,
           "step": "separate" if "--step separate" in command else "fused"}
    per_kernel = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r["Counter_Name"] == counter]
        copies = [r for r in rows if "copy" in r["Kernel_Name"].lower()
                  and float(r["Counter_Value"]) * 1024 > CALIBRATION_BYTES / 4]
        if not copies:
            raise SystemExit(f"{path}: no calibration copy dispatch found")
        cal_kib = float(copies[-1]["Counter_Value"])
        factor = CALIBRATION_BYTES / (cal_kib * 1024.0)
        out[f"{counter.lower()}_copy_kib"] = cal_kib
        out[f"{counter.lower()}_factor"] = round(factor, 4)
        for name in DECODE_KERNELS:
            vals = [float(r["Counter_Value"]) for r in rows if name in r["Kernel_Name"]]
            if vals:
                d = per_kernel.setdefault(name, {"dispatches": len(vals)})
                d[f"{counter.lower()}_kib_mean"] = round(statistics.mean(vals), 1)
                d[f"{counter.lower()}_bytes"] = round(statistics.mean(vals) * 1024.0 * factor)
    out["per_kernel"] = per_kernel
    out["bytes_per_call"] = int(sum(d.get("fetch_size_bytes", 0) + d.get("write_size_bytes", 0)
                                    for d in per_kernel.values()))
    return out


def cpu_baseline(case, min_seconds: float = 8.0, max_repeats: int = 40) -> dict:
    """The fp64 oracle (gather through block tables + naive softmax) on the
    host, with BLAS allowed every core this process may run on, and again
    with one thread; each run repeats the whole workload until about
    ``min_seconds`` of CPU work (at least two calls) and reports the median
    call.  The all-cores run is the reported baseline."""
    allowed = len(os.sched_getaffinity(0))
    wide = _oracle_run(case, allowed, min_seconds, max_repeats)
    one = _oracle_run(case, 1, min_seconds, max_repeats)
    wide["single_thread"] = {k: one[k] for k in ("value", "unit", "cores", "seconds_per_call")}
    wide["threads_allowed"] = allowed
    return wide


def _oracle_run(case, threads: int, min_seconds: float, max_repeats: int) -> dict:
    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    kp, vp, _ = oracle.build_pools(case)
    times, cpu_s = [], []
    ctx = threadpool_limits(limits=threads) if threadpool_limits else None
    try:
        if ctx:
            ctx.__enter__()
        while len(times) < 2 or (sum(times) < min_seconds and len(times) < max_repeats):
            t0 = time.perf_counter()
            c0 = time.process_time()
            oracle.decode(case.query, kp, vp, case.block_tables, case.context_lens, case.scale,
                          case.dtype, case.block_size, ring=case.ring, kv_dtype=case.kv_dtype,
                          k_scale=case.k_scale, v_scale=case.v_scale)
            times.append(time.perf_counter() - t0)
            cpu_s.append(time.process_time() - c0)
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    t = statistics.median(times)
    # threads actually busy: process CPU time over wall time
    cores = max(1, round(sum(cpu_s) / sum(times)))
    ab = algorithmic_bytes(case)
    return {"value": round(ab["decode"] / t / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"whole workload ({case.num_seqs} sequences, {ab['tokens']} cached tokens), "
                      f"decode only (fp64 gather + softmax), BLAS threads {threads}, median of {len(times)} "
                      f"calls ({sum(times):.1f} s); {t:.3f} s per call, cpu/wall {sum(cpu_s) / sum(times):.2f}",
            "seconds_per_call": round(t, 4)}


# Per-wave timeline records of the measurement build (the layout the decode
# kernels write after the workspace's other parts): main kernel 8 uint64 per
# wave for up to 8192 waves, combine kernel 2 uint64 per wave for up to 65536.
TIMELINE_WAVES, TIMELINE_COMBINE_WAVES = 8192, 65536
TIMELINE_BYTES = TIMELINE_WAVES * 64 + TIMELINE_COMBINE_WAVES * 16
TIMELINE_TICK_US = 0.01  # s_memrealtime runs at 100 MHz
TIMELINE_RECORDS = []  # raw records of each call, for callers that analyse them further


def wave_timeline(torch, dev, decode, ws, ws_bytes: int, calls: int, config: str, kernel: str) -> dict:
    """Per-wave timeline of ``calls`` decode calls on the measurement build:
    when the waves enter, have the tile schedule, consume their first tile
    and end streaming, per XCD, and when the combine kernel's waves enter
    and finish merging, all relative to the first wave's entry (µs)."""
    base = ws_bytes - TIMELINE_BYTES
    region = ws[base:ws_bytes]
    scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    per_call = []
    for c in range(calls):
        cold = c < (calls + 1) // 2
        region.zero_()
        if cold:
            scrub.sum()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        decode()
        e1.record()
        e1.synchronize()
        rec = region.view(torch.int64).cpu().numpy().view(np.uint64)
        TIMELINE_RECORDS.append(rec.copy())
        main = rec[: TIMELINE_WAVES * 8].reshape(TIMELINE_WAVES, 8)
        main = main[main[:, 6] == 1]
        comb = rec[TIMELINE_WAVES * 8:].reshape(TIMELINE_COMBINE_WAVES, 2)
        comb = comb[comb[:, 0] != 0]
        t0 = int(main[:, 0].min())

        def us(x):
            return (np.asarray(x, dtype=np.float64) - t0) * TIMELINE_TICK_US

        entry, sched, first, end = us(main[:, 0]), us(main[:, 1]), us(main[:, 2]), us(main[:, 3])
        tiles = (main[:, 4] >> np.uint64(32)).astype(np.int64)
        segs = (main[:, 4] & np.uint64(0xFFFFFFFF)).astype(np.int64)
        xcc = main[:, 5].astype(np.int64)
        merged = (comb[:, 1] >> np.uint64(63)) == 1
        c_entry = us(comb[:, 0])
        c_exit = us(comb[merged, 1] & np.uint64((1 << 63) - 1))
        stream = end - first
        row = {
            "cold": cold, "call_us_events": round(e0.elapsed_time(e1) * 1e3, 2), "waves": int(main.shape[0]),
            "entry_spread_us": round(float(entry.max()), 2),
            "schedule_ready_us": {"median": round(float(np.median(sched)), 2), "max": round(float(sched.max()), 2)},
            "first_tile_us": {"median": round(float(np.median(first)), 2), "max": round(float(first.max()), 2)},
            "stream_end_us": {"p10": round(float(np.percentile(end, 10)), 2), "median": round(float(np.median(end)), 2),
                              "p90": round(float(np.percentile(end, 90)), 2), "max": round(float(end.max()), 2)},
            "xcd_mean_end_us": [round(float(end[xcc == x].mean()), 2) if np.any(xcc == x) else None
                                for x in range(8)],
            "tiles_per_wave": {"min": int(tiles.min()), "max": int(tiles.max())},
            "segments_per_wave": {"median": float(np.median(segs)), "max": int(segs.max())},
            # does a wave that begins more segments end later?
            "corr_end_vs_segments": round(float(np.corrcoef(end, segs)[0, 1]), 3) if segs.std() > 0 else None,
            "corr_stream_vs_segments": (round(float(np.corrcoef(stream, segs)[0, 1]), 3)
                                        if segs.std() > 0 else None),
            "combine": {
                "first_entry_us": round(float(c_entry.min()), 2) if c_entry.size else None,
                "gap_after_last_stream_end_us": round(float(c_entry.min() - end.max()), 2) if c_entry.size else None,
                "merging_waves": int(merged.sum()),
                "merge_end_median_us": round(float(np.median(c_exit)), 2) if c_exit.size else None,
                "merge_end_max_us": round(float(c_exit.max()), 2) if c_exit.size else None,
            },
        }
        per_call.append(row)
    del scrub

    def med(rows, *keys):
        vals = []
        for r in rows:
            v = r
            for k in keys:
                v = v[k]
            vals.append(v)
        return round(float(np.median(vals)), 2)

    summary = {}
    for label, rows in (("cold", [r for r in per_call if r["cold"]]), ("hot", [r for r in per_call if not r["cold"]])):
        if not rows:
            continue
        summary[label] = {
            "calls": len(rows),
            "call_us_events": med(rows, "call_us_events"),
            "schedule_ready_us": med(rows, "schedule_ready_us", "median"),
            "first_tile_median_us": med(rows, "first_tile_us", "median"),
            "stream_end_median_us": med(rows, "stream_end_us", "median"),
            "stream_end_max_us": med(rows, "stream_end_us", "max"),
            "combine_gap_us": med(rows, "combine", "gap_after_last_stream_end_us"),
            "merge_end_max_us": med(rows, "combine", "merge_end_max_us"),
        }
    return {"timeline": config, "kernel": kernel + ", measurement build (PA_WAVE_TIMELINE)",
            "clock": "s_memrealtime, 100 MHz, microseconds from the first wave's entry",
            "summary": summary, "calls": per_call}


def read_ceiling(torch, dev, calls: int = 20) -> dict:
    """Plain streaming-read ceiling of this machine: the library's read probe
    (non-temporal 16-byte loads, four work-groups per CU) over 1 GiB, median
    of ``calls`` event-timed launches."""
    import paged_kv_cache_145_amd as pk

    src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.int32, device=dev)
    sums = torch.empty(pk.READ_PROBE_CHECKSUMS, dtype=torch.int32, device=dev)
    for _ in range(3):
        pk.read_probe(src, sums)
    mean_us, med_us = _event_us(torch, lambda: pk.read_probe(src, sums), calls)
    del src
    return {"gbs": round(CALIBRATION_BYTES / (med_us * 1e-6) / 1e9, 1), "bytes": CALIBRATION_BYTES,
            "kernel": "read_probe_kernel (pa_read_probe: non-temporal 16-byte loads, 1 GiB, median of "
                      f"{calls} launches, {med_us:.1f} us)"}


def _nan_pools(workloads, torch, shape, dtype, dev):
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    ibits = torch.int32 if dtype == "f32" else torch.int16
    raw = np.array(workloads.NAN_BITS[dtype], dtype=np.uint32 if dtype == "f32" else np.uint16)
    bits = int(raw.view(np.int32 if dtype == "f32" else np.int16))
    k = torch.empty(shape, dtype=tdt, device=dev)
    v = torch.empty(shape, dtype=tdt, device=dev)
    k.view(ibits).fill_(bits)
    v.view(ibits).fill_(bits)
    return k, v


def _event_us(torch, fn, calls: int):
    """Mean and median microseconds of ``fn`` bracketed by events on the
    current stream (the stream the library launches on)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) * 1e3 for a, b in evs]
    return statistics.mean(ts), statistics.median(ts)


def prefix_cpu_baseline(prompt, block_size: int, reps: int = 20) -> dict:
    """The oracle's prefix model answering the same 2048-id match."""
    from oracle.allocator import BlockAllocatorModel
    from oracle.prefix import PrefixCacheModel

    ids = [int(x) for x in prompt]
    model = PrefixCacheModel(BlockAllocatorModel(256), block_size)
    model.insert(ids, [model.alloc.alloc() for _ in range(len(ids) // block_size)])
    t0, c0 = time.perf_counter(), time.process_time()
    for _ in range(reps):
        got, _ = model.match(ids, 1 << 20)
        for blk in got:
            model.release(blk)
    wall = (time.perf_counter() - t0) / reps
    cores = max(1, round((time.process_time() - c0) / (wall * reps)))
    return {"value": round(wall * 1e6, 1), "unit": "us per 2048-id match", "cores": cores, "kind": "oracle",
            "sample": f"the oracle's prefix model matching the same 2048-id prompt, {reps} times"}


def measure_prefix(args) -> int:
    """Prefix reuse with copy-on-write, measured on the 70B-head workload of
    a 600-token resident system prompt (37 full 16-token blocks and a tail
    of 8) and 12 requests: host admission through the library's prefix index
    (match, copy-on-write, allocate, list), the tail copies, decode over the
    shared blocks, and the block copy kernel at one admission wave and in
    bulk.  Prints one JSON line; ``roofline`` is the copy kernel's."""
    import torch

    import paged_kv_cache_145_amd as pk
    import workloads

    dev = "cuda:0"
    torch.cuda.set_device(0)
    sc = workloads.config_prefix_unaligned()
    bs, hkv, d = sc.block_size, sc.num_kv_heads, sc.head_dim
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[sc.dtype]
    raw_view = np.int32 if sc.dtype == "f32" else np.int16

    def to_dev(raw):
        return torch.from_numpy(np.ascontiguousarray(raw).view(raw_view)).view(tdt).to(dev)

    k, v = _nan_pools(workloads, torch, (sc.num_blocks, bs, hkv, d), sc.dtype, dev)
    pool = pk.Pool(k, v, bs)
    print("bench: admitting the prefix workload through the prefix index", file=sys.stderr, flush=True)
    p = len(sc.system_tokens)
    sys_blocks = [pool.alloc_block() for _ in range(-(-p // bs))]
    pool.prefix_insert(sc.system_tokens, sys_blocks, tail=True, resident=True)
    for blk in sys_blocks:
        pool.decref(blk)
    tables, covered, copies, admit_us = [], [], [], []
    for r in sc.requests:
        n = len(r.tokens)
        t0 = time.perf_counter()
        blocks, cov = pool.prefix_match(r.tokens)
        if cov % bs and cov < n:
            new, copied = pool.cow_block(blocks[-1])
            if copied:
                copies.append((blocks[-1], new))
            blocks[-1] = new
        while len(blocks) * bs < n:
            blocks.append(pool.alloc_block())
        pool.prefix_insert(r.tokens, blocks)
        admit_us.append((time.perf_counter() - t0) * 1e6)
        tables.append(blocks)
        covered.append(cov)
    if min(min(t) for t in tables) < 0:
        raise SystemExit("pool too small for the prefix workload")

    def write_rows(rows_tables, positions, keys, values):
        bt = np.full((len(rows_tables), max(len(t) for t in rows_tables)), -1, dtype=np.int32)
        for i, t in enumerate(rows_tables):
            bt[i, : len(t)] = t
        sid = np.concatenate([np.full(len(q), i, dtype=np.int32) for i, q in enumerate(positions)])
        pos = np.concatenate([np.asarray(q, dtype=np.int64) for q in positions])
        slots = pk.compute_slot_mapping(pool, bt, sid, pos)
        pk.reshape_and_cache(pool, to_dev(keys), to_dev(values), torch.from_numpy(slots).to(dev))

    write_rows([sys_blocks], [np.arange(p)], sc.system_keys, sc.system_values)
    src = torch.tensor([a for a, _ in copies], dtype=torch.int32, device=dev)
    dst = torch.tensor([b for _, b in copies], dtype=torch.int32, device=dev)
    pk.copy_blocks(pool, src, dst)
    write_rows(tables, [np.arange(c, len(r.tokens)) for c, r in zip(covered, sc.requests)],
               np.concatenate([r.keys[c:] for c, r in zip(covered, sc.requests)]),
               np.concatenate([r.values[c:] for c, r in zip(covered, sc.requests)]))
    bt = np.full((sc.num_seqs, max(len(t) for t in tables)), -1, dtype=np.int32)
    for i, t in enumerate(tables):
        bt[i, : len(t)] = t
    lens = np.array([len(r.tokens) for r in sc.requests], dtype=np.int32)
    query, tables_d, lens_d = to_dev(sc.query), torch.from_numpy(bt).to(dev), torch.from_numpy(lens).to(dev)
    out = torch.empty((sc.num_seqs, sc.num_q_heads, d), dtype=tdt, device=dev)
    mcl = int(lens.max())
    ws = torch.empty(max(pk.decode_workspace_bytes(pool, sc.num_seqs, sc.num_q_heads, mcl), 1),
                     dtype=torch.uint8, device=dev)

    def decode():
        pk.decode(pool, out, query, tables_d, lens_d, mcl, sc.scale, workspace=ws)

    row = hkv * d * 2 * 2  # one token's K and V rows
    unique_blocks = {}
    for t, n in zip(tables, lens):
        for j, blk in enumerate(t):
            unique_blocks[blk] = max(unique_blocks.get(blk, 0), min(bs, int(n) - j * bs))
    dec_bytes = sum(unique_blocks.values()) * row + sc.num_seqs * sc.num_q_heads * d * 2 * 2
    for _ in range(args.warmup):
        decode()
    torch.cuda.synchronize()
    dec_mean, dec_med = _event_us(torch, decode, args.steps)
    block_bytes = bs * hkv * d * 2
    wave = (src, dst)

    def copy_wave():
        pk.copy_blocks(pool, *wave)

    for _ in range(args.warmup):
        copy_wave()
    wave_mean, wave_med = _event_us(torch, copy_wave, args.steps)
    pool.close()

    # bulk: 4096 pairs of 70B-shaped blocks (256 MiB read, 256 MiB written)
    pairs = 4096
    print(f"bench: timing the block copy in bulk ({pairs} pairs)", file=sys.stderr, flush=True)
    bk = torch.zeros((2 * pairs, bs, hkv, d), dtype=tdt, device=dev)
    bv = torch.zeros_like(bk)
    bulk = pk.Pool(bk, bv, bs)
    perm = np.random.default_rng(sc.seed).permutation(2 * pairs).astype(np.int32)
    bsrc, bdst = torch.from_numpy(perm[:pairs]).to(dev), torch.from_numpy(perm[pairs:]).to(dev)

    def copy_bulk():
        pk.copy_blocks(bulk, bsrc, bdst)

    for _ in range(args.warmup):
        copy_bulk()
    bulk_mean, bulk_med = _event_us(torch, copy_bulk, args.steps)
    bulk.close()
    del bk, bv
    bulk_bytes = pairs * block_bytes * 2 * 2  # K and V, read and written
    achieved = bulk_bytes / (bulk_mean * 1e-6) / 1e9

    # host side of the index: keys and a full-prompt match of 2048 ids
    rng = np.random.default_rng(sc.seed + 1)
    prompt = rng.integers(0, 1 << 32, size=2048, dtype=np.uint64).astype(np.uint32)
    hk, hv = torch.zeros((256, bs, hkv, d), dtype=tdt, device=dev), None
    hv = torch.zeros_like(hk)
    host_pool = pk.Pool(hk, hv, bs)
    hb = [host_pool.alloc_block() for _ in range(2048 // bs)]
    host_pool.prefix_insert(prompt, hb)
    long_ids = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    t0 = time.perf_counter()
    pk.block_hashes(long_ids, bs)  # one call over 2^22 ids: the binding's cost is negligible
    hash_ns = (time.perf_counter() - t0) / (long_ids.size // bs) * 1e9
    reps = 2000
    t0 = time.perf_counter()
    for _ in range(reps):  # each match takes a reference per block; all are dropped below
        host_pool.prefix_match(prompt)
    match_us = (time.perf_counter() - t0) / reps * 1e6
    for blk in hb:
        for _ in range(reps):
            host_pool.decref(blk)
    host_pool.close()
    cpu = prefix_cpu_baseline(prompt, bs) if not args.no_cpu_baseline else None

    result = {
        "metric": "prefix reuse: copy-on-write block copy bandwidth (bulk) with admission and shared-prefix decode",
        "value": round(achieved, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(bulk_mean / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sc.dtype,
        "data": "synthetic",
        "config": {
            "workload": ("prefix_unaligned: Hq 64, Hkv 8, D 128, bf16, block 16; 600-token resident system "
                         "prompt (37 full blocks + tail of 8); 12 requests (6 extend it, 2 leave it inside "
                         "the tail, 1 inside a full block, 1 share nothing, 1 prompt only, 1 repeat); bulk "
                         f"copy of {pairs} block pairs"),
            "global_batch": sc.num_seqs,
            "seed": sc.seed,
        },
        "admission": {"host_us_per_request_median": round(statistics.median(admit_us), 2),
                      "covered_tokens": covered, "tail_copies": len(copies)},
        "copy_wave": {"pairs": len(copies), "us_mean": round(wave_mean, 2), "us_median": round(wave_med, 2),
                      "bytes": len(copies) * block_bytes * 2 * 2},
        "decode_shared": {"us_mean": round(dec_mean, 2), "us_median": round(dec_med, 2),
                          "unique_bytes": dec_bytes,
                          "gbs_unique": round(dec_bytes / (dec_mean * 1e-6) / 1e9, 1),
                          "cached_tokens": int(lens.sum())},
        "host_index": {"block_key_ns_per_block16": round(hash_ns, 1),
                       "match_2048_ids_us": round(match_us, 2)},
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_copy_blocks: copy_blocks_kernel (HIP events bracket the call)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "algorithmic_bytes": bulk_bytes,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0


MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16/f16 MFMA peak of MI355X


def multi_costs(case) -> dict:
    """Algorithmic bytes and flops of one pa_decode_multi call: every K/V
    row the longest query row of each sequence sees, once; the queries and
    outputs; table entries.  Flops: 4 * D per (query row, visible key)."""
    s = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
    s_kv = 1 if workloads_is_kv8(case.kv_dtype) else s
    lens = case.context_lens.astype(np.int64)
    row = case.num_kv_heads * case.head_dim * 2 * s_kv
    qo = case.num_seqs * case.q_len * case.num_q_heads * case.head_dim * 2 * s
    if case.ring is not None:
        # ring verification: the resident rows (at most S + W) and the drafts'
        # rows (inputs, query dtype); draft i sees min(n + i + 1, S + W) keys
        cap = case.ring.sink + case.ring.window
        res = np.minimum(lens, cap)
        kv = int(res.sum()) * row + case.num_seqs * case.q_len * case.num_kv_heads * case.head_dim * 2 * s
        tables = int(sum(-(-int(n) // case.block_size) for n in res)) * 4 + case.num_seqs * 4
        keys_seen = sum(min(int(n) + i + 1, cap) for n in lens for i in range(case.q_len))
        flops = 4 * case.head_dim * case.num_q_heads * keys_seen
        return {"bytes": kv + qo + tables, "flops": flops, "tokens": int(res.sum())}
    kv = int(lens.sum()) * row
    tables = int(sum(-(-int(n) // case.block_size) for n in lens)) * 4 + case.num_seqs * 4
    keys_seen = sum(max(0, int(n) - case.q_len + i + 1) for n in lens for i in range(case.q_len))
    flops = 4 * case.head_dim * case.num_q_heads * keys_seen
    return {"bytes": kv + qo + tables, "flops": flops, "tokens": int(lens.sum())}


def measure_multi(args) -> int:
    """Multi-token paged decode (speculative verification, chunked prefill)
    on one of the multi-token workloads; one JSON line."""
    import torch

    import paged_kv_cache_145_amd as pk
    import workloads

    dev = "cuda:0"
    torch.cuda.set_device(0)
    name = args.config if args.config in workloads.MULTI_CONFIGS else "spec_verify_llama70b"
    print(f"bench: generating the seeded workload {name}", file=sys.stderr, flush=True)
    case = workloads.MULTI_CONFIGS[name]()
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]
    raw_view = np.int32 if case.dtype == "f32" else np.int16

    def to_dev(raw):
        return torch.from_numpy(np.ascontiguousarray(raw).view(raw_view)).view(tdt).to(dev)

    shape = (case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim)
    if workloads_is_kv8(case.kv_dtype):
        k = torch.full(shape, workloads.FP8_NAN_CODE, dtype=torch.uint8, device=dev)
        v = torch.full(shape, workloads.FP8_NAN_CODE, dtype=torch.uint8, device=dev)
        pool = pk.Pool(k, v, case.block_size, act_dtype=tdt, k_scale=case.k_scale, v_scale=case.v_scale,
                       kv_format=case.kv_dtype[4:])
    else:
        k, v = _nan_pools(workloads, torch, shape, case.dtype, dev)
        pool = pk.Pool(k, v, case.block_size)
    ring = None
    if case.ring is not None:  # verification over the sink + ring cache (drafts rotated up to q_len - 1 past it)
        cap = case.ring.sink + case.ring.window + case.q_len
        table = torch.empty(pk.rope_table_bytes(cap, case.head_dim) // 4, dtype=torch.float32, device=dev)
        pk.rope_table_init(table, cap, case.head_dim, case.ring.rope_base)
        ring = pk.Ring(case.ring.sink, case.ring.window, case.ring.rope_base, table, capacity=cap)
    for ch in case.writes:
        sid = np.full(ch.positions.shape, ch.seq, dtype=np.int32)
        slots = pk.compute_slot_mapping(pool, case.block_tables, sid, ch.positions, ring)
        pk.reshape_and_cache(pool, to_dev(ch.keys), to_dev(ch.values), torch.from_numpy(slots).to(dev))
    query = to_dev(case.query)
    tables = torch.from_numpy(case.block_tables).to(dev)
    lens = torch.from_numpy(case.context_lens).to(dev)
    mcl = int(case.context_lens.max())
    out = torch.empty(tuple(case.query.shape), dtype=tdt, device=dev)
    if ring is not None:
        dk, dv = to_dev(case.draft_keys), to_dev(case.draft_values)
        ws = torch.empty(max(pk.decode_verify_ring_workspace_bytes(pool, case.num_seqs, case.q_len,
                                                                   case.num_q_heads), 1),
                         dtype=torch.uint8, device=dev)

        def call():
            pk.decode_verify_ring(pool, out, query, dk, dv, tables, lens, mcl, case.scale, ring, workspace=ws)
    else:
        ws = torch.empty(max(pk.decode_multi_workspace_bytes(pool, case.num_seqs, case.q_len, case.num_q_heads,
                                                             mcl), 1), dtype=torch.uint8, device=dev)

        def call():
            pk.decode_multi(pool, out, query, tables, lens, mcl, case.scale, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    if args.timeline > 0:
        print(json.dumps(wave_timeline(torch, dev, call, ws, ws.numel(), args.timeline, args.config,
                                       kernel="decode_multi_kernel + decode_multi_reduce_kernel")), flush=True)
        pool.close()
        return 0
    t0 = time.perf_counter()
    mean_us, med_us = _event_us(torch, call, args.steps)
    wall = time.perf_counter() - t0
    pool.close()
    c = multi_costs(case)
    gbs = c["bytes"] / (mean_us * 1e-6) / 1e9
    tflops = c["flops"] / (mean_us * 1e-6) / 1e12
    # the bound is the resource whose ideal time is longer
    mfma_bound = c["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12) > c["bytes"] / (HBM_PEAK_GBS * 1e9)
    roof = ({"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": c["flops"]}
            if mfma_bound else
            {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": c["bytes"]})
    roof["kernel"] = "pa_decode_multi call: decode_multi_kernel (+ decode_multi_reduce_kernel) (HIP events)"
    roof["traffic"] = None
    new_tokens = case.num_seqs * case.q_len
    result = {
        "metric": "multi-token paged decode: new tokens attended per second",
        "value": round(new_tokens / (mean_us * 1e-6), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {"workload": (f"{name}: B {case.num_seqs}, q_len {case.q_len}, Hq {case.num_q_heads}, "
                                f"Hkv {case.num_kv_heads}, D {case.head_dim}, "
                                f"{case.kv_dtype[4:].upper() + ' KV, ' if case.kv_dtype else ''}{case.dtype}, block {case.block_size}, "
                                f"{c['tokens']} cached tokens (the new ones included)"),
                   "global_batch": case.num_seqs, "q_len": case.q_len, "seed": case.seed},
        "call_us": {"mean": round(mean_us, 2), "median": round(med_us, 2)},
        "effective_gbs": round(gbs, 1),
        "effective_tflops": round(tflops, 2),
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else multi_cpu_baseline(case),
    }
    print(json.dumps(result), flush=True)
    return 0


def multi_cpu_baseline(case, max_rows: int = 800) -> dict:
    """The oracle's decode_multi on a bounded sample: the new tokens of the
    first sequences, up to ``max_rows`` (sequence, token) rows."""
    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    nseq = max(1, min(case.num_seqs, max_rows // case.q_len))
    if case.ring is not None:  # each verified row rebuilds its ring: a smaller sample
        nseq = max(1, min(case.num_seqs, 16))
    kp, vp, _ = oracle.build_pools(case)
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0, c0 = time.perf_counter(), time.process_time()
        if case.ring is not None:
            oracle.decode_verify_ring(case.query[:nseq], case.draft_keys[:nseq], case.draft_values[:nseq], kp, vp,
                                      case.block_tables[:nseq], case.context_lens[:nseq], case.scale, case.dtype,
                                      case.block_size, case.ring)
        else:
            oracle.decode_multi(case.query[:nseq], kp, vp, case.block_tables[:nseq], case.context_lens[:nseq],
                                case.scale, case.dtype, case.block_size, case.q_len)
        wall = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    cores = max(1, round((time.process_time() - c0) / wall))
    rows = nseq * case.q_len
    return {"value": round(rows / wall, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the new tokens of the first {nseq} sequences ({rows} rows), fp64 gather + softmax"
                      f"{' (ring verification)' if case.ring is not None else ''}, "
                      f"{wall:.2f} s"}


def batching_cpu_baseline(reqs, block_size, num_blocks, max_batch, max_blocks, iters: int) -> dict:
    """The oracle's scheduler model driving the same request stream."""
    from oracle.allocator import BlockAllocatorModel
    from oracle.batching import ContinuousBatchingModel

    m = ContinuousBatchingModel(BlockAllocatorModel(num_blocks), block_size, max_batch, max_blocks)
    t0, c0 = time.perf_counter(), time.process_time()
    for it in range(iters):
        for rid, p, g, arrival in reqs:
            if arrival == it:
                m.add(rid, p, g)
        batch, _ = m.schedule()
        for s in batch:
            m.step(s.rid)
    wall = time.perf_counter() - t0
    cores = max(1, round((time.process_time() - c0) / wall))
    return {"value": round(wall / iters * 1e6, 1), "unit": "us per scheduling iteration", "cores": cores,
            "kind": "oracle", "sample": f"the oracle's scheduler model over the first {iters} iterations of the "
                                        f"same request stream (host bookkeeping only, no attention)"}


def measure_batching(args) -> int:
    """Continuous batching driven by the library's batcher over the 70B-head
    pool: every iteration schedules (host C++), writes the new K/V rows and
    decodes the decoding requests.  One JSON line; ``roofline`` is the
    decode calls' (their algorithmic bytes over their event time)."""
    import torch

    import paged_kv_cache_145_amd as pk
    import workloads

    dev = "cuda:0"
    torch.cuda.set_device(0)
    bs, hkv, hq, d, nb, max_batch = 16, 8, 64, 128, 6841, 64
    max_blocks = -(-(2000 + 256) // bs)
    reqs = workloads.batching_requests(145050, 384, bs, max_blocks, prompt_lo=50, prompt_hi=2000,
                                       gen_lo=16, gen_hi=256)
    tdt = torch.bfloat16
    k = torch.zeros((nb, bs, hkv, d), dtype=tdt, device=dev)
    v = torch.zeros_like(k)
    pool = pk.Pool(k, v, bs)
    batcher = pk.Batcher(pool, max_batch, max_blocks)
    gen = torch.Generator(device=dev)
    gen.manual_seed(145050)
    rows_cap = max_batch * 2000
    rows_k = torch.randn((rows_cap, hkv, d), generator=gen, device=dev).to(tdt)
    rows_v = torch.randn((rows_cap, hkv, d), generator=gen, device=dev).to(tdt)
    query = torch.randn((max_batch, hq, d), generator=gen, device=dev).to(tdt)
    out = torch.empty((max_batch, hq, d), dtype=tdt, device=dev)
    ws = torch.empty(max(pk.decode_workspace_bytes(pool, max_batch, hq, max_blocks * bs), 1), dtype=torch.uint8,
                     device=dev)
    scale = 1.0 / np.sqrt(d)
    row_bytes = hkv * d * 2 * 2
    total_iters = args.warmup + args.steps
    host_s, it_s, sched_us = [], [], []
    dec_ev, dec_bytes, dec_tokens = [], [], []
    stats = {"prefill": 0, "preempted": 0, "freed_requests": 0, "written_rows": 0}
    print(f"bench: continuous batching, {total_iters} iterations", file=sys.stderr, flush=True)
    for it in range(total_iters):
        t0 = time.perf_counter()
        for rid, p, g, arrival in reqs:
            if arrival == it:
                batcher.add(rid, p, g)
        ts = time.perf_counter()
        batch, info = batcher.schedule()
        sched_s = time.perf_counter() - ts
        n = info["scheduled"]
        if n == 0:
            continue
        ws_, wc = batch["write_start"], batch["write_count"]
        sid = np.repeat(np.arange(n, dtype=np.int32), wc)
        pos = np.concatenate([np.arange(a, a + c, dtype=np.int64) for a, c in zip(ws_, wc)])
        slots = pk.compute_slot_mapping(pool, batch["tables"], sid, pos)
        dec = np.flatnonzero(~batch["prefill"])
        tables = torch.from_numpy(np.ascontiguousarray(batch["tables"][dec])).to(dev, non_blocking=False)
        lens_np = np.ascontiguousarray(batch["context_lens"][dec])
        lens = torch.from_numpy(lens_np).to(dev)
        slots_d = torch.from_numpy(slots).to(dev)
        t1 = time.perf_counter()
        m = slots.shape[0]
        pk.reshape_and_cache(pool, rows_k[:m], rows_v[:m], slots_d)
        if dec.size:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            pk.decode(pool, out[: dec.size], query[: dec.size], tables, lens, int(lens_np.max()), scale, workspace=ws)
            e1.record()
        for rid in batch["ids"]:
            batcher.step(int(rid))
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        if it >= args.warmup:
            sched_us.append(sched_s * 1e6)
            host_s.append(t1 - t0)
            it_s.append(t2 - t0)
            if dec.size:
                dec_ev.append(e0.elapsed_time(e1) * 1e-3)
                dec_bytes.append(int(lens_np.sum()) * row_bytes + dec.size * hq * d * 2 * 2)
                dec_tokens.append(int(dec.size))
            for key in ("prefill", "preempted", "freed_requests"):
                stats[key] += info[key]
            stats["written_rows"] += m
    batcher.close()
    pool.close()
    wall = sum(it_s)
    achieved = sum(dec_bytes) / sum(dec_ev) / 1e9 if dec_ev else 0.0
    result = {
        "metric": "continuous batching: decoded tokens per second (host scheduling, cache writes and decode)",
        "value": round(sum(dec_tokens) / wall, 1) if wall else 0.0,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": len(it_s),
        "warmup": args.warmup,
        "ms_per_step": round(wall / max(1, len(it_s)) * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"continuous batching over a {nb}-block pool (Hq {hq}, Hkv {hkv}, D {d}, bf16, "
                                f"block {bs}), batch <= {max_batch}, 384 requests: prompts U[50,2000], "
                                f"generations U[16,256], arrivals over the first 96 iterations"),
                   "global_batch": max_batch, "seed": 145050},
        "iteration_ms": {"mean": round(statistics.mean(it_s) * 1e3, 4), "host_mean": round(statistics.mean(host_s) * 1e3, 4),
                         "schedule_call_us": round(statistics.mean(sched_us), 2)},
        "decode_us_mean": round(statistics.mean(dec_ev) * 1e6, 2) if dec_ev else None,
        "decode_batch_mean": round(statistics.mean(dec_tokens), 1) if dec_tokens else 0,
        "scheduler": stats,
        "roofline": {"bound": "hbm", "kernel": "pa_decode calls of the loop (HIP events)", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_call": int(statistics.mean(dec_bytes)) if dec_bytes else 0},
        "cpu_baseline": None if args.no_cpu_baseline else batching_cpu_baseline(reqs, bs, nb, max_batch, max_blocks,
                                                                                 min(total_iters, 200)),
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cold-steps", type=int, default=50,
                    help="extra decode calls each preceded by a 1 GiB read that evicts the caches (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--config", default="llama70b_b64",
                    choices=sorted(list(__import__("workloads").CONFIGS) + list(__import__("workloads").FP8_CONFIGS)
                                   + list(__import__("workloads").MULTI_CONFIGS)),
                    help="workload (default: the 70B-shaped batch the metric is quoted on; the others "
                         "are the parity configurations, timed the same way)")
    ap.add_argument("--launch", choices=("eager", "graph"), default="eager",
                    help="launch eagerly (default) or replay captured HIP graphs of the write and the "
                         "decode call (one replay each per step)")
    ap.add_argument("--step", choices=("fused", "separate"), default="fused",
                    help="fused (default): one pa_decode_append call stores the new tokens and decodes; "
                         "separate: pa_reshape_and_cache, then pa_decode")
    ap.add_argument("--profile-calls", type=int, default=0,
                    help="only run this many decode calls, then a 1 GiB copy (for rocprofv3 counter runs)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 counter_collection.csv files into the traffic record")
    ap.add_argument("--measure", choices=("decode", "prefix", "multi", "batching"), default="decode",
                    help="decode (default): the hot-path step; prefix: prefix reuse with copy-on-write "
                         "(admission, tail copies, shared-prefix decode, bulk block copy); multi: "
                         "multi-token decode on --config spec_verify_llama70b (default) or chunked_prefill; "
                         "batching: the continuous-batching driver looping over schedule, writes and decode")
    ap.add_argument("--timeline", type=int, default=0, metavar="CALLS",
                    help="load the measurement build and print the per-wave timeline of this many decode "
                         "calls (half after a 1 GiB scrub, half back to back) instead of timing steps "
                         "(single-token decode, or --measure multi)")
    ap.add_argument("--traffic-command", default="",
                    help="the profiling command line recorded with --write-traffic")
    args = ap.parse_args()
    if args.write_traffic:
        rec = summarize_counters(args.write_traffic[0], args.write_traffic[1], args.traffic_command)
        with open(traffic_file(args.config), "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps(rec))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path has no multi-GPU mode); got --gpus {args.gpus}",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_145_amd as pk
    import workloads
    from paged_kv_cache_145_amd import _lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.timeline > 0:
        if args.measure not in ("decode", "multi"):
            print("--timeline covers the single- and multi-token decode", file=sys.stderr)
            return 2
        _lib.use_timeline_build()
    _lib.load()
    if args.measure == "prefix":
        return measure_prefix(args)
    if args.measure == "multi":
        return measure_multi(args)
    if args.measure == "batching":
        return measure_batching(args)
    if args.config in workloads.MULTI_CONFIGS:
        print("multi-token workloads run with --measure multi", file=sys.stderr)
        return 2
    dev = "cuda:0"
    torch.cuda.set_device(0)
    print(f"bench: generating the seeded workload {args.config}", file=sys.stderr, flush=True)
    if args.config == "sink_ring":  # timing set: full windows at distinct ring phases near 100k
        case = workloads.config_sink_ring(lengths=workloads.ring_timing_lengths())
    else:
        case = {**workloads.CONFIGS, **workloads.FP8_CONFIGS}[args.config]()
    ab = algorithmic_bytes(case)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]
    ibits = torch.int32 if case.dtype == "f32" else torch.int16
    raw_view = np.int32 if case.dtype == "f32" else np.int16

    def to_dev(raw):
        return torch.from_numpy(np.ascontiguousarray(raw).view(raw_view)).view(tdt).to(dev)

    shape = (case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim)
    if workloads_is_kv8(case.kv_dtype):
        k_cache = torch.full(shape, workloads.FP8_NAN_CODE, dtype=torch.uint8, device=dev)
        v_cache = torch.full(shape, workloads.FP8_NAN_CODE, dtype=torch.uint8, device=dev)
        pool = pk.Pool(k_cache, v_cache, case.block_size, act_dtype=tdt, k_scale=case.k_scale,
                       v_scale=case.v_scale, kv_format=case.kv_dtype[4:])
    else:
        k_cache = torch.empty(shape, dtype=tdt, device=dev)
        v_cache = torch.empty(shape, dtype=tdt, device=dev)
        nan_bits = int(np.array(workloads.NAN_BITS[case.dtype],
                                dtype=np.uint32 if case.dtype == "f32" else np.uint16).view(raw_view))
        k_cache.view(ibits).fill_(nan_bits)
        v_cache.view(ibits).fill_(nan_bits)
        pool = pk.Pool(k_cache, v_cache, case.block_size)
    ring = None
    if case.ring is not None:
        cap = case.ring.sink + case.ring.window
        table = torch.empty(pk.rope_table_bytes(cap, case.head_dim) // 4, dtype=torch.float32, device=dev)
        pk.rope_table_init(table, cap, case.head_dim, case.ring.rope_base)
        ring = pk.Ring(case.ring.sink, case.ring.window, case.ring.rope_base, table)

    # fill the cache through the library's own write path
    for ch in case.writes:
        sid = np.full(ch.positions.shape, ch.seq, dtype=np.int32)
        slots = pk.compute_slot_mapping(pool, case.block_tables, sid, ch.positions, ring)
        pk.reshape_and_cache(pool, to_dev(ch.keys), to_dev(ch.values), torch.from_numpy(slots).to(dev))
    step_chunks = case.step_writes()
    step_slots = np.concatenate([pk.compute_slot_mapping(
        pool, case.block_tables, np.full(1, ch.seq, dtype=np.int32), ch.positions, ring) for ch in step_chunks])
    step_keys = to_dev(np.concatenate([ch.keys for ch in step_chunks]))
    step_vals = to_dev(np.concatenate([ch.values for ch in step_chunks]))
    step_slots_d = torch.from_numpy(step_slots).to(dev)

    query = to_dev(case.query)
    tables = torch.from_numpy(case.block_tables).to(dev)
    lens = torch.from_numpy(case.context_lens).to(dev)
    max_ctx = int(case.context_lens.max())
    out = torch.empty((case.num_seqs, case.num_q_heads, case.head_dim), dtype=tdt, device=dev)
    ws_bytes = pk.decode_workspace_bytes(pool, case.num_seqs, case.num_q_heads, max_ctx, ring)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    group = case.num_q_heads // case.num_kv_heads
    # the one-call step is a single launch on the MFMA path (f16/bf16 or
    # 8-bit pools, groups up to 16); elsewhere the library would run the
    # two calls in turn, so the bench times them as two calls
    mfma = case.dtype != "f32" and 1 <= group <= 16 and os.environ.get("PA_FORCE_VALU", "0") in ("", "0")
    fused = args.step == "fused" and mfma

    def decode():
        if fused:  # stores the step's new tokens and decodes in one call
            pk.decode_append(pool, out, query, step_keys, step_vals, step_slots_d, tables, lens, max_ctx,
                             case.scale, ring=ring, workspace=ws)
        else:
            pk.decode(pool, out, query, tables, lens, max_ctx, case.scale, ring=ring, workspace=ws)

    # algorithmic bytes of the call the events bracket
    call_bytes = ab["decode"] + (ab["write_out"] if fused else 0)

    if args.timeline > 0:
        if not mfma:
            print("--timeline covers the stream-K (MFMA) decode", file=sys.stderr)
            return 2
        for _ in range(args.warmup):
            decode()
        kernel = ("decode_mfma_kernel" + (" (append variant)" if fused else "") +
                  " + decode_streamk_reduce_kernel")
        print(json.dumps(wave_timeline(torch, dev, decode, ws, ws_bytes, args.timeline, args.config, kernel)),
              flush=True)
        pool.close()
        return 0

    if args.profile_calls > 0:
        for _ in range(args.profile_calls):
            decode()
        torch.cuda.synchronize()
        src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
        src.fill_(3)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # calibration: reads and writes exactly 1 GiB
        torch.cuda.synchronize()
        print(f"bench: profiled {args.profile_calls} decode calls and a 1 GiB copy", file=sys.stderr)
        pool.close()
        return 0

    def write():
        if not fused:
            pk.reshape_and_cache(pool, step_keys, step_vals, step_slots_d)

    def step(ev_decode=None):
        write()
        if ev_decode is not None:
            ev_decode[0].record()
        decode()
        if ev_decode is not None:
            ev_decode[1].record()

    print(f"bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.launch == "graph":
        # a decode loop replays captured launches: one graph for the cache
        # write, one for the decode call (both kernels)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g_write, g_decode = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        if not fused:
            with torch.cuda.graph(g_write, stream=side):
                write()
        with torch.cuda.graph(g_decode, stream=side):
            decode()
        torch.cuda.synchronize()
        if not fused:
            write = g_write.replay
        decode = g_decode.replay
        for _ in range(max(1, args.warmup // 4)):
            step()
        torch.cuda.synchronize()

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    decode_ms = [a.elapsed_time(b) for a, b in events]

    cold_ms = []
    if args.cold_steps > 0:
        # read (not write) 1 GiB between calls: the caches end up holding
        # clean unrelated lines, so the call finds neither its data cached
        # nor dirty lines to write back
        scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        for _ in range(args.cold_steps):
            scrub.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            decode()
            e1.record()
            e1.synchronize()
            cold_ms.append(e0.elapsed_time(e1))
        del scrub

    ceiling = read_ceiling(torch, dev)
    ms_per_step = wall / args.steps * 1e3
    step_bytes = ab["decode"] + ab["write"]
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dec_avg_ms = statistics.mean(decode_ms)
    achieved = call_bytes / (dec_avg_ms * 1e-3) / 1e9
    traffic = read_traffic(args.config, "fused" if fused else "separate")
    if fused:
        kernel = ("pa_decode_append call: decode_mfma_kernel (variant that also stores the new tokens) + "
                  "decode_streamk_reduce_kernel")
    elif mfma:
        kernel = "pa_decode call: decode_mfma_kernel + decode_streamk_reduce_kernel"
    else:
        kernel = "pa_decode call: decode_valu_kernel (+ decode_reduce_kernel when a context is split)"

    if args.config == "llama70b_b64":
        workload = ("llama70b_b64: paged decode, B 64, Hq 64, Hkv 8 (GQA 8), D 128, bf16 KV, "
                    "block 16, lengths 32xU[50,500] + 19xU[500,2000] + 13xU[2000,8000], "
                    "shuffled blocks, pool 1.1x need")
    else:
        kv_name = (f"{case.kv_dtype[4:].upper()} (8-bit, per-head scales)" if workloads_is_kv8(case.kv_dtype)
                   else case.dtype)
        workload = (f"{args.config}: paged decode, B {case.num_seqs}, Hq {case.num_q_heads}, "
                    f"Hkv {case.num_kv_heads}, D {case.head_dim}, {kv_name} KV, {case.dtype} query, "
                    f"block {case.block_size}"
                    + (f", sink {case.ring.sink} + ring {case.ring.window}" if case.ring else ""))
    result = {
        "metric": "paged decode attention: effective KV GB/s (% of HBM peak) and tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {
            "workload": workload,
            "global_batch": case.num_seqs,
            "cached_tokens": ab["tokens"],
            "max_context_len": max_ctx,
            "num_blocks": case.num_blocks,
            "seed": case.seed,
            "kv_storage": (f"{case.kv_dtype[4:]} codes, per-head scales" if workloads_is_kv8(case.kv_dtype)
                           else case.dtype),
            "step": ("one pa_decode_append call (stores the new tokens, then attends)" if fused
                     else "pa_reshape_and_cache, then pa_decode"),
            "launch": (("hip graph replay of the call" if fused else
                        "hip graph replay (cache write graph + decode call graph)") if args.launch == "graph"
                       else "eager launches"),
        },
        "tokens_per_s": round(case.num_seqs / (ms_per_step * 1e-3), 1),
        "step_bytes": step_bytes,
        "decode_us": {"mean": round(dec_avg_ms * 1e3, 2),
                      "median": round(statistics.median(decode_ms) * 1e3, 2),
                      "p10": round(float(np.percentile(decode_ms, 10)) * 1e3, 2),
                      "p90": round(float(np.percentile(decode_ms, 90)) * 1e3, 2)},
        "decode_cold_us": ({"median": round(statistics.median(cold_ms) * 1e3, 2),
                            "gbs": round(call_bytes / (statistics.median(cold_ms) * 1e-3) / 1e9, 1)}
                           if cold_ms else None),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel + " (HIP events bracket the call)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "frac_cold": (round(call_bytes / (statistics.median(cold_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                          if cold_ms else None),
            "read_ceiling": ceiling,
            "frac_of_read_ceiling": round(achieved / ceiling["gbs"], 4),
            "traffic": traffic,
            "algorithmic_bytes": call_bytes,
            "algorithmic_bytes_logical": ab["decode_logical"] + (ab["write_out"] if fused else 0),
        },
    }
    pool.close()
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

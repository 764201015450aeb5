#!/usr/bin/env python3
"""Benchmark: paged decode attention on one MI355X.

One step = the whole hot path over one batch: the cache write of every
sequence's newest token (pa_reshape_and_cache) followed by single-token
paged decode attention (pa_decode: split-K partition kernel + reduce).
Workload: the LLaMA-2-70B-shaped batch (B 64, Hq 64, Hkv 8, D 128, bf16,
16-token blocks, mixed lengths 50..8000, shuffled physical blocks), seeded
and synthetic, resident in HBM before the timed region starts.

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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_llama70b_b64.json")
KERNEL_SOURCES = ["decode_kernels.hip", "device_common.h", "launch.h", "api.hip"]


def algorithmic_bytes(case) -> dict:
    """Bytes the decode must move at minimum: every resident K and V row once,
    query in, output out, block-table entries and lengths."""
    s_kv = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
    lens = case.context_lens.astype(np.int64)
    if case.ring is not None:
        lens = np.minimum(lens, case.ring.sink + case.ring.window)
    kv = int(lens.sum()) * case.num_kv_heads * case.head_dim * 2 * s_kv
    qo = case.num_seqs * case.num_q_heads * case.head_dim * 2 * s_kv
    tables = int(sum(-(-int(n) // case.block_size) for n in lens)) * 4 + case.num_seqs * 4
    write = case.num_seqs * case.num_kv_heads * case.head_dim * 2 * s_kv * 2  # read + write, K and V
    return {"decode": kv + qo + tables, "kv": kv, "write": write, "tokens": int(lens.sum())}


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_145_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """Counter-derived HBM bytes per decode call, if taken on the current kernels."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t.get("bytes_per_call")


def cpu_baseline(case, repeats: int = 3) -> dict:
    """The fp64 oracle (gather through block tables + naive softmax) on host cores."""
    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    kp, vp, _ = oracle.build_pools(case)
    times = []
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        if ctx:
            ctx.__enter__()
        for _ in range(repeats):
            t0 = time.perf_counter()
            oracle.decode(case.query, kp, vp, case.block_tables, case.context_lens, case.scale,
                          case.dtype, case.block_size, ring=case.ring)
            times.append(time.perf_counter() - t0)
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    t = statistics.median(times)
    ab = algorithmic_bytes(case)
    return {"value": round(ab["decode"] / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"whole workload ({case.num_seqs} sequences, {ab['tokens']} cached tokens), "
                      f"decode only, median of {repeats}; {t:.3f} s per call",
            "seconds_per_call": round(t, 4)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cold-steps", type=int, default=50,
                    help="extra decode calls each preceded by a 1 GiB cache scrub (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
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
    _lib.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    print("bench: generating the seeded 70B-shaped batch", file=sys.stderr, flush=True)
    case = workloads.config_llama70b()
    ab = algorithmic_bytes(case)
    tdt = torch.bfloat16

    def to_dev(raw):
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(tdt).to(dev)

    shape = (case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim)
    k_cache = torch.empty(shape, dtype=tdt, device=dev)
    v_cache = torch.empty(shape, dtype=tdt, device=dev)
    k_cache.view(torch.int16).fill_(workloads.NAN_BITS["bf16"])
    v_cache.view(torch.int16).fill_(workloads.NAN_BITS["bf16"])
    pool = pk.Pool(k_cache, v_cache, case.block_size)

    # fill the cache through the library's own write path
    for ch in case.writes:
        sid = np.full(ch.positions.shape, ch.seq, dtype=np.int32)
        slots = pk.compute_slot_mapping(pool, case.block_tables, sid, ch.positions)
        pk.reshape_and_cache(pool, to_dev(ch.keys), to_dev(ch.values), torch.from_numpy(slots).to(dev))
    step_chunks = case.step_writes()
    step_slots = np.concatenate([pk.compute_slot_mapping(
        pool, case.block_tables, np.full(1, ch.seq, dtype=np.int32), ch.positions) for ch in step_chunks])
    step_keys = to_dev(np.concatenate([ch.keys for ch in step_chunks]))
    step_vals = to_dev(np.concatenate([ch.values for ch in step_chunks]))
    step_slots_d = torch.from_numpy(step_slots).to(dev)

    query = to_dev(case.query)
    tables = torch.from_numpy(case.block_tables).to(dev)
    lens = torch.from_numpy(case.context_lens).to(dev)
    max_ctx = int(case.context_lens.max())
    out = torch.empty((case.num_seqs, case.num_q_heads, case.head_dim), dtype=tdt, device=dev)
    ws_bytes = pk.decode_workspace_bytes(pool, case.num_seqs, case.num_q_heads, max_ctx)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev_decode=None):
        pk.reshape_and_cache(pool, step_keys, step_vals, step_slots_d)
        if ev_decode is not None:
            ev_decode[0].record()
        pk.decode(pool, out, query, tables, lens, max_ctx, case.scale, workspace=ws)
        if ev_decode is not None:
            ev_decode[1].record()

    print(f"bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
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
        scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        for _ in range(args.cold_steps):
            scrub.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            pk.decode(pool, out, query, tables, lens, max_ctx, case.scale, workspace=ws)
            e1.record()
            e1.synchronize()
            cold_ms.append(e0.elapsed_time(e1))
        del scrub

    ms_per_step = wall / args.steps * 1e3
    step_bytes = ab["decode"] + ab["write"]
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dec_avg_ms = statistics.mean(decode_ms)
    achieved = ab["decode"] / (dec_avg_ms * 1e-3) / 1e9
    traffic = read_traffic()
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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama70b_b64: paged decode, B 64, Hq 64, Hkv 8 (GQA 8), D 128, bf16 KV, "
                        "block 16, lengths 32xU[50,500] + 19xU[500,2000] + 13xU[2000,8000], "
                        "shuffled blocks, pool 1.1x need",
            "global_batch": case.num_seqs,
            "cached_tokens": ab["tokens"],
            "max_context_len": max_ctx,
            "num_blocks": case.num_blocks,
            "seed": case.seed,
        },
        "tokens_per_s": round(case.num_seqs / (ms_per_step * 1e-3), 1),
        "step_bytes": step_bytes,
        "decode_us": {"mean": round(dec_avg_ms * 1e3, 2),
                      "median": round(statistics.median(decode_ms) * 1e3, 2),
                      "p10": round(float(np.percentile(decode_ms, 10)) * 1e3, 2),
                      "p90": round(float(np.percentile(decode_ms, 90)) * 1e3, 2)},
        "decode_cold_us": ({"median": round(statistics.median(cold_ms) * 1e3, 2),
                            "gbs": round(ab["decode"] / (statistics.median(cold_ms) * 1e-3) / 1e9, 1)}
                           if cold_ms else None),
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_decode (decode_mfma_kernel + decode_reduce_kernel)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": ab["decode"],
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

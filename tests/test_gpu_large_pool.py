"""Pools larger than 4 GiB: the 64-bit offsets of the cache write, the
decode tile loads, the one-call step's stores and the block copy.  A small
workload's blocks are relabelled to ids straddling the 4 GiB byte offset of
4.6 GiB pools (bf16, 32 KiB blocks) and 4.4 GiB pools (E4M3, 16 KiB blocks);
writes must be bit-exact, decode within the oracle's tolerance."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_145_amd as pk
import workloads
from gpu_support import INT_VIEW, DeviceCase, assert_parity, oracle_reference, raw_to_torch, torch_bits

pytestmark = pytest.mark.gpu

GiB = 1 << 30


def _big(case, kv8=False):
    """The case on a pool of more than 4 GiB per K/V, its blocks shifted to
    ids whose byte offsets straddle 4 GiB."""
    block_bytes = case.block_size * case.num_kv_heads * case.head_dim * (1 if kv8 else 2)
    boundary = (4 * GiB) // block_bytes  # first block id past 4 GiB
    shift = boundary - case.num_blocks // 2
    num_blocks = boundary + (GiB // 2) // block_bytes
    tables = np.where(case.block_tables >= 0, case.block_tables + shift, case.block_tables).astype(np.int32)
    big = dataclasses.replace(case, num_blocks=num_blocks, block_tables=tables,
                              pad_block=case.pad_block + shift if case.pad_block >= 0 else -1)
    assert num_blocks * block_bytes > 4 * GiB and (shift + case.num_blocks) * block_bytes > 4 * GiB
    return big, shift


def _pool_slice(t, shift, n):
    return t[shift:shift + n]


@pytest.mark.parametrize("kind", ["bf16", "e4m3"])
def test_pool_past_4gib_write_decode_step_and_copy(kind):
    base = workloads.make_paged_case("big", 9301, "bf16", [1, 17, 100, 1000, 3000, 5003], 64, 8, 128, 16)
    if kind == "e4m3":
        base = workloads.config_fp8(lambda: base, kv_format="e4m3")
    kv8 = kind != "bf16"
    case, shift = _big(base, kv8)
    print(f"large pool {kind}: {case.num_blocks} blocks, shift {shift}", flush=True)
    dc = DeviceCase(case)
    dc.write_all()
    torch.cuda.synchronize()
    # 1. cache write: the used blocks equal the oracle's pools, byte for byte
    kp, vp, _ = oracle.build_pools(base)
    view = torch.uint8 if kv8 else INT_VIEW[base.dtype]
    got_k = _pool_slice(dc.k_cache, shift, base.num_blocks).view(view).cpu().numpy()
    got_v = _pool_slice(dc.v_cache, shift, base.num_blocks).view(view).cpu().numpy()
    ref_k = kp if kv8 else kp.view(np.int16)
    ref_v = vp if kv8 else vp.view(np.int16)
    assert np.array_equal(got_k, ref_k) and np.array_equal(got_v, ref_v)
    # 2. decode over blocks past 4 GiB
    _, _, _, ref = oracle_reference(base)
    out = dc.decode()
    assert_parity(out, ref, base.dtype)
    # 3. the one-call step: rewrite every newest token through the decode launch
    step = {ch.seq: ch for ch in base.step_writes()}
    b_count = base.num_seqs
    keys = workloads.nan_array((b_count, base.num_kv_heads, base.head_dim), base.dtype)
    vals = workloads.nan_array((b_count, base.num_kv_heads, base.head_dim), base.dtype)
    slots = np.full(b_count, -1, dtype=np.int32)
    for b, ch in step.items():
        slots[b] = dc.slots_for(ch)[0]
        keys[b], vals[b] = ch.keys[0], ch.values[0]
    assert int(slots.min()) * base.num_kv_heads * base.head_dim * (1 if kv8 else 2) > 2 * GiB
    mcl = int(base.context_lens.max())
    ws = torch.empty(pk.decode_workspace_bytes(dc.pool, b_count, base.num_q_heads, mcl), dtype=torch.uint8,
                     device="cuda:0")
    out2 = torch.empty_like(out)
    pk.decode_append(dc.pool, out2, dc.query, raw_to_torch(keys, base.dtype).cuda(),
                     raw_to_torch(vals, base.dtype).cuda(), torch.from_numpy(slots).cuda(), dc.block_tables,
                     dc.context_lens, mcl, base.scale, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(torch_bits(out2, base.dtype), torch_bits(out, base.dtype))
    assert np.array_equal(_pool_slice(dc.k_cache, shift, base.num_blocks).view(view).cpu().numpy(), ref_k)
    # 4. block copies between ids on both sides of the 4 GiB offset
    n_used = base.num_blocks
    src = np.arange(shift, shift + 8, dtype=np.int32)
    dst = np.arange(shift + n_used - 8, shift + n_used, dtype=np.int32)
    before = dc.k_cache[src.tolist()].clone()
    pk.copy_blocks(dc.pool, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    assert torch.equal(dc.k_cache[dst.tolist()].view(view), before.view(view))
    assert torch.equal(dc.v_cache[dst.tolist()].view(view), dc.v_cache[src.tolist()].view(view))
    dc.close()
    del dc
    torch.cuda.empty_cache()

"""GPU parity of speculative verification over the sink + ring cache
(pa_decode_verify_ring) against the oracle: draft rows are inputs, the cache
is only read, and each draft's output is the ring decode after drafts 0..i
would have been written.  Covers streams that have not wrapped, that wrap
during the step, and long past the wrap (the edge lengths of the sink + ring
workload, plus an empty stream), f16 and bf16, D 64, small windows where
drafts evict drafts, the cache left byte-for-byte unchanged, accept-then-
write giving the oracle's last-writer state, and block relabelling."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_145_amd as pk
import workloads
from gpu_support import INT_VIEW, TORCH_DTYPES, DeviceCase, assert_parity, options, raw_to_torch, torch_bits

pytestmark = pytest.mark.gpu

DRAFT_ROPE = 16  # RoPE table positions beyond sink + window (up to 16 drafts)


def _ref(case):
    k, v, _ = oracle.build_pools(case)
    return oracle.decode_verify_ring(case.query, case.draft_keys, case.draft_values, k, v, case.block_tables,
                                     case.context_lens, case.scale, case.dtype, case.block_size, case.ring)


def _verify(dc, case, tables=None):
    dt = case.dtype
    out = torch.full(case.query.shape, float("nan"), dtype=TORCH_DTYPES[dt], device=dc.device)
    mcl = max(int(case.context_lens.max()), 1)
    nbytes = pk.decode_verify_ring_workspace_bytes(dc.pool, case.num_seqs, case.q_len, case.num_q_heads)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=dc.device)
    pk.decode_verify_ring(dc.pool, out, dc.query, raw_to_torch(case.draft_keys, dt).to(dc.device),
                          raw_to_torch(case.draft_values, dt).to(dc.device),
                          dc.block_tables if tables is None else tables, dc.context_lens, mcl, case.scale,
                          dc.ring, workspace=ws)
    torch.cuda.synchronize()
    return out


CASES = {
    "workload_f16": lambda: workloads.config_ring_verify(),
    "workload_bf16": lambda: workloads.config_ring_verify(dtype="bf16", lengths=[0, 1, 5, 1019, 1020, 1023,
                                                                                  1024, 1028, 99_999]),
    "d64_q8": lambda: workloads.config_ring_verify(lengths=[0, 3, 1020, 1021, 1030, 7777], q_len=8, head_dim=64,
                                                   num_q_heads=8, num_kv_heads=2),
    "mha_q1": lambda: workloads.config_ring_verify(lengths=[0, 2, 1023, 1024, 3000], q_len=1, num_q_heads=4,
                                                   num_kv_heads=4),
    # windows shorter than the step: drafts evict earlier drafts
    "s2_w3_q4": lambda: workloads.config_ring_verify(lengths=[0, 1, 2, 4, 5, 6, 11, 50], q_len=4, sink=2,
                                                     window=3),
    "s0_w5_q7": lambda: workloads.config_ring_verify(lengths=[0, 3, 5, 6, 13], q_len=7, sink=0, window=5),
    "s20_w40_q16": lambda: workloads.config_ring_verify(lengths=[0, 10, 19, 20, 45, 59, 60, 61, 500], q_len=16,
                                                        sink=20, window=40, num_q_heads=16, num_kv_heads=2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_ring_verify_parity(name):
    case = CASES[name]()
    print(f"ring verify {name}: B {case.num_seqs} q_len {case.q_len}", flush=True)
    ref = _ref(case)
    dc = DeviceCase(case, rope_extra=DRAFT_ROPE)
    dc.write_all()
    view = INT_VIEW[case.dtype]
    k0, v0 = dc.k_cache.view(view).clone(), dc.v_cache.view(view).clone()
    out = _verify(dc, case)
    assert_parity(out.reshape(case.num_seqs * case.q_len, case.num_q_heads, case.head_dim),
                  ref.reshape(-1, case.num_q_heads, case.head_dim), case.dtype)
    # the cache is only read
    assert torch.equal(dc.k_cache.view(view), k0) and torch.equal(dc.v_cache.view(view), v0)
    again = _verify(dc, case)
    assert np.array_equal(torch_bits(out, case.dtype), torch_bits(again, case.dtype))
    dc.close()


def test_ring_verify_accept_then_write_gives_last_writer_state():
    """After verification, stream b accepts a_b drafts (0..q_len) and stores
    them at their ring slots: the pools equal the oracle's pools of the same
    writes, and a single-token decode over them matches the oracle."""
    case = workloads.config_ring_verify(lengths=[0, 3, 1019, 1022, 1024, 5000, 99_998])
    dc = DeviceCase(case, rope_extra=DRAFT_ROPE)
    dc.write_all()
    _verify(dc, case)
    accepted = [b % (case.q_len + 1) for b in range(case.num_seqs)]
    chunks = []
    for b, a_b in enumerate(accepted):
        n = int(case.context_lens[b])
        if a_b:
            chunks.append(workloads.WriteChunk(b, np.arange(n, n + a_b, dtype=np.int64),
                                               case.draft_keys[b, :a_b], case.draft_values[b, :a_b]))
    dc.write_all(chunks)
    # oracle: the same committed writes, then the accepted drafts
    k_ref, v_ref, _ = oracle.build_pools(case)
    s, w = case.ring.sink, case.ring.window
    for ch in chunks:
        slots = [oracle.slot_of(case.block_tables[ch.seq], oracle.ring_slot(int(p), s, w), case.block_size)
                 for p in ch.positions]
        oracle.reshape_and_cache_(k_ref, v_ref, ch.keys, ch.values, slots, case.block_size)
    view = INT_VIEW[case.dtype]
    got_k = dc.k_cache.view(view).cpu().numpy()
    assert np.array_equal(got_k, k_ref.view(np.int16)) and np.array_equal(dc.v_cache.view(view).cpu().numpy(),
                                                                           v_ref.view(np.int16))
    # decode the next token over the committed cache (context n + a)
    lens = case.context_lens + np.array(accepted, dtype=np.int32)
    q = case.query[:, 0]
    ref = oracle.decode(q, k_ref, v_ref, case.block_tables, lens, case.scale, case.dtype, case.block_size,
                        ring=case.ring)
    out = torch.empty((case.num_seqs, case.num_q_heads, case.head_dim), dtype=TORCH_DTYPES[case.dtype],
                      device="cuda:0")
    nbytes = pk.decode_workspace_bytes(dc.pool, case.num_seqs, case.num_q_heads, int(lens.max()), dc.ring)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda:0")
    pk.decode(dc.pool, out, raw_to_torch(np.ascontiguousarray(q), case.dtype).to("cuda:0"), dc.block_tables,
              torch.from_numpy(lens).to("cuda:0"), int(lens.max()), case.scale, ring=dc.ring, workspace=ws)
    torch.cuda.synchronize()
    assert_parity(out, ref, case.dtype)
    dc.close()


def test_ring_verify_block_relabelling_bit_identical():
    case = workloads.config_ring_verify(lengths=[0, 17, 1023, 1025, 5000])
    dc = DeviceCase(case, rope_extra=DRAFT_ROPE)
    dc.write_all()
    base = torch_bits(_verify(dc, case), case.dtype)
    perm = torch.from_numpy(np.random.default_rng(7).permutation(case.num_blocks)).to("cuda:0")
    k2, v2 = torch.empty_like(dc.k_cache), torch.empty_like(dc.v_cache)
    k2[perm], v2[perm] = dc.k_cache, dc.v_cache
    dc.k_cache.copy_(k2)
    dc.v_cache.copy_(v2)
    tables = torch.where(dc.block_tables >= 0, perm[dc.block_tables.clamp(min=0).long()].int(), dc.block_tables)
    assert np.array_equal(torch_bits(_verify(dc, case, tables.contiguous()), case.dtype), base)
    dc.close()


def test_ring_verify_rejects_a_short_rope_table():
    case = workloads.config_ring_verify(lengths=[5, 2000])
    dc = DeviceCase(case)  # table holds only sink + window positions
    with pytest.raises(pk.PaError, match="INVAL"):
        _verify(dc, case)
    dc.close()


@pytest.mark.parametrize("cost", [2, 9])
def test_ring_verify_cost_weighted_ranges(cost):
    """Ring verification under cost-weighted stream-K ranges (short ranges,
    so the edge lengths are cut and merged)."""
    case = CASES[list(CASES)[0]]()
    ref = _ref(case)
    dc = DeviceCase(case, rope_extra=DRAFT_ROPE)
    dc.write_all()
    with options(PA_MULTI_SEQ_COST=cost + 1, PA_MULTI_MIN_RANGE=1):
        out = _verify(dc, case)
    assert_parity(out.reshape(case.num_seqs * case.q_len, case.num_q_heads, case.head_dim),
                  ref.reshape(-1, case.num_q_heads, case.head_dim), case.dtype)
    dc.close()

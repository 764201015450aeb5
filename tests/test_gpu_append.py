"""GPU parity of the decode step that also stores the step's new token
(pa_decode_append) against the oracle's write-then-decode: every cached
token but the newest is written beforehand, the newest one's slot holds a
NaN sentinel, and one call must both store the new rows (bit for bit, as
pa_reshape_and_cache would) and attend over the full context, giving the
same bits as pa_reshape_and_cache followed by pa_decode.  Covers the fused
single-launch path (16-bit and 8-bit pools, GQA groups up to 16) on ragged,
short, long and shared-prefix batches and on batches larger than one launch
slice, and the two-step path (fp32 pools, wider groups).
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_145_amd as pk
import workloads
from gpu_support import (TORCH_DTYPES, DeviceCase, INT_VIEW, assert_parity, options, oracle_reference,
                         raw_to_torch, torch_bits)

pytestmark = pytest.mark.gpu


def _prepare(case):
    """Pools holding every write, then NaN rows at the newest token of each
    sequence; returns the device case and the step's (slots, key, value)."""
    dc = DeviceCase(case)
    dc.write_all()
    full = DeviceCase(case)
    full.write_all()
    step = {ch.seq: ch for ch in case.step_writes()}
    hkv, d, dt = case.num_kv_heads, case.head_dim, case.dtype
    keys = workloads.nan_array((case.num_seqs, hkv, d), dt)
    vals = workloads.nan_array((case.num_seqs, hkv, d), dt)
    slots = np.full(case.num_seqs, -1, dtype=np.int32)
    for b, ch in step.items():
        slots[b] = dc.slots_for(ch)[0]
        keys[b] = ch.keys[0]
        vals[b] = ch.values[0]
    live = slots >= 0
    if live.any():  # overwrite the newest tokens with the sentinel
        nan = workloads.nan_array((int(live.sum()), hkv, d), dt)
        pk.reshape_and_cache(dc.pool, raw_to_torch(nan, dt).to(dc.device), raw_to_torch(nan, dt).to(dc.device),
                             torch.from_numpy(slots[live]).to(dc.device))
    return dc, full, slots, keys, vals


def _append(dc, case, slots, keys, vals, max_ctx=None):
    dt = case.dtype
    mcl = int(case.context_lens.max()) if max_ctx is None else max_ctx
    out = torch.full((case.num_seqs, case.num_q_heads, case.head_dim), float("nan"), dtype=TORCH_DTYPES[dt],
                     device=dc.device)
    nbytes = pk.decode_workspace_bytes(dc.pool, case.num_seqs, case.num_q_heads, mcl, dc.ring)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dc.device)
    ws.fill_(0xFF)  # the workspace needs no initialisation
    pk.decode_append(dc.pool, out, dc.query, raw_to_torch(keys, dt).to(dc.device),
                     raw_to_torch(vals, dt).to(dc.device), torch.from_numpy(slots).to(dc.device),
                     dc.block_tables, dc.context_lens, mcl, case.scale, ring=dc.ring, workspace=ws)
    torch.cuda.synchronize()
    return out


def _same_pools(a, b, dtype):
    view = torch.uint8 if workloads.is_kv8(a.case.kv_dtype) else INT_VIEW[dtype]
    assert torch.equal(a.k_cache.view(view), b.k_cache.view(view)), "key pool differs"
    assert torch.equal(a.v_cache.view(view), b.v_cache.view(view)), "value pool differs"


def _check(case):
    _, _, _, ref = oracle_reference(case)
    dc, full, slots, keys, vals = _prepare(case)
    out = _append(dc, case, slots, keys, vals)
    assert_parity(out, ref, case.dtype)
    _same_pools(dc, full, case.dtype)
    two_step = full.decode()  # the pool already holds the new rows
    assert np.array_equal(torch_bits(out, case.dtype), torch_bits(two_step, case.dtype))
    dc.close()
    full.close()
    return out


SHAPES = [
    # dtype, Hq, Hkv, D, bs, lengths
    ("bf16", 32, 4, 128, 16, [0, 1, 2, 15, 16, 17, 33, 700, 2900]),
    ("f16", 8, 8, 64, 64, [1, 64, 65, 1500, 33]),        # G 1
    ("bf16", 16, 1, 128, 16, [3, 20000]),                # G 16, many stream-K segments
    ("f16", 24, 8, 128, 16, [17, 18, 40000, 2]),         # G 3
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}-G{s[1] // s[2]}-D{s[3]}-bs{s[4]}")
def test_append_parity_shapes(shape):
    dtype, hq, hkv, d, bs, lens = shape
    print(f"append shape {shape}", flush=True)
    _check(workloads.make_paged_case("append", 8100 + hq + d + len(lens), dtype, lens, hq, hkv, d, bs))


def test_append_llama70b_batch():
    print("append llama70b b64", flush=True)
    case = workloads.config_llama70b()
    out = _check(case)
    # repeated calls (the new rows rewritten in place) give the same bits
    dc, full, slots, keys, vals = _prepare(case)
    again = _append(dc, case, slots, keys, vals)
    assert np.array_equal(torch_bits(out, case.dtype), torch_bits(again, case.dtype))
    dc.close()
    full.close()


def test_append_shared_prefix_bit_identical_to_private_copies():
    """The newest token lives in each sequence's own block; the result over
    shared prefix blocks equals, bit for bit, that over private copies."""
    print("append shared prefix", flush=True)
    outs = []
    for private in (False, True):
        case = workloads.config_shared_prefix(private_copies=private)
        outs.append(torch_bits(_check(case), case.dtype))
    assert np.array_equal(outs[0], outs[1])


def test_append_padding_slot_writes_nothing():
    """A sequence whose slot is -1 stores nothing (its row keeps the NaN
    sentinel); every output row, that one included, has the bits of the
    two-step path with the same slots."""
    case = workloads.make_paged_case("append_pad", 8200, "bf16", [40, 5, 300, 17], 16, 2, 128, 16)
    print("append padding slot", flush=True)
    _, _, _, ref = oracle_reference(case)
    dc, full, slots, keys, vals = _prepare(case)
    before_k = dc.k_cache.clone()
    pad = 2
    pad_slot = int(slots[pad])
    slots[pad] = -1
    out = _append(dc, case, slots, keys, vals)
    keep = [b for b in range(case.num_seqs) if b != pad]
    assert_parity(out[keep], ref[keep], case.dtype)
    blk, row = divmod(pad_slot, case.block_size)
    view = INT_VIEW[case.dtype]
    assert torch.equal(dc.k_cache[blk, row].view(view), before_k[blk, row].view(view))
    dc2, full2, _, _, _ = _prepare(case)
    dt = case.dtype
    pk.reshape_and_cache(dc2.pool, raw_to_torch(keys, dt).to(dc2.device), raw_to_torch(vals, dt).to(dc2.device),
                         torch.from_numpy(slots).to(dc2.device))
    two_step = dc2.decode()
    assert np.array_equal(torch_bits(out, dt), torch_bits(two_step, dt))
    _same_pools(dc, dc2, dt)
    for x in (dc, full, dc2, full2):
        x.close()


def test_append_sink_ring():
    """Ring mode: the newest token's ring slot picks the tile that stores it
    (not the last tile once a context has wrapped), lengths from 1 to 100,000
    around every wrap boundary."""
    print("append sink ring", flush=True)
    _check(workloads.config_sink_ring())


def test_append_more_sequences_than_one_launch_slice():
    rng = np.random.default_rng(78)
    lens = [int(x) for x in rng.integers(1, 41, size=1300)]
    print("append slices: 1300 sequences", flush=True)
    _check(workloads.make_paged_case("append_slices", 8300, "bf16", lens, 16, 2, 64, 16))


FALLBACK = [
    ("f32", 8, 2, 64, 16, [0, 1, 17, 300]),                   # no fp32 MFMA kernel
    ("bf16", 64, 2, 128, 16, [1, 2, 900, 33]),                # G 32: VALU kernel
]


@pytest.mark.parametrize("shape", FALLBACK, ids=lambda s: f"{s[0]}-G{s[1] // s[2]}")
def test_append_two_step_paths(shape):
    dtype, hq, hkv, d, bs, lens = shape
    print(f"append fallback {shape}", flush=True)
    _check(workloads.make_paged_case("append_fb", 8400 + hq, dtype, lens, hq, hkv, d, bs))


@pytest.mark.parametrize("kv_format", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", [("bf16", 32, 4, 128, [1, 2, 16, 17, 1000, 0, 5000]),
                                   ("f16", 8, 8, 64, [3, 64, 65, 2000])], ids=["bf16-G8-D128", "f16-G1-D64"])
def test_append_fp8_pool(kv_format, shape):
    """8-bit pools: the launch quantises the new rows as the cache write does
    (bit-exact pools) and attends over them."""
    dtype, hq, hkv, d, lens = shape
    print(f"append {kv_format} {shape}", flush=True)
    case = workloads.config_fp8(lambda: workloads.make_paged_case("append_fp8", 8500 + hq, dtype, lens, hq, hkv, d,
                                                                  16), kv_format=kv_format)
    _check(case)


def test_append_fp8_llama70b():
    print("append llama70b e4m3", flush=True)
    _check(workloads.config_llama70b_fp8())


def test_append_rejects_misaligned_inputs():
    case = workloads.make_paged_case("append_bad", 8600, "bf16", [5, 9], 8, 2, 64, 16)
    dc, full, slots, keys, vals = _prepare(case)
    k = raw_to_torch(keys, "bf16").to(dc.device)
    kbuf = torch.empty(k.numel() + 8, dtype=k.dtype, device=dc.device)
    kmis = kbuf[1 : 1 + k.numel()].view(k.shape)  # 2-byte offset
    out = torch.empty((2, 8, 64), dtype=torch.bfloat16, device=dc.device)
    with pytest.raises(pk.PaError) as e:
        pk.decode_append(dc.pool, out, dc.query, kmis, raw_to_torch(vals, "bf16").to(dc.device),
                         torch.from_numpy(slots).to(dc.device), dc.block_tables, dc.context_lens, 9, case.scale,
                         workspace=dc.workspace())
    assert e.value.status == -1
    dc.close()
    full.close()


@pytest.mark.parametrize("cost", [2, 6])
def test_append_cost_weighted_ranges(cost):
    """The one-call step with cost-weighted stream-K ranges equals the two
    calls bit for bit (both under the same ranges) and the oracle."""
    print(f"append llama70b b64, sequence cost {cost}", flush=True)
    with options(PA_DECODE_SEQ_COST=cost + 1):
        _check(workloads.config_llama70b())
        _check(workloads.make_paged_case("append_cost", 8700 + cost, "bf16", [0, 1, 2, 15, 16, 17, 33, 700],
                                         32, 4, 128, 16))

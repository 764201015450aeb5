"""Pins for the fp64 oracle: it is checked against things other than itself.

* dense special case against torch's scaled_dot_product_attention (a library
  routine, float64 on the CPU) with K/V expanded per GQA group;
* pure-Python brute force with math.exp on the tiny fp32 workload;
* closed forms: n = 1 gives V_0, identical keys give the mean of V;
* invariances the paging method implies: relabelling physical blocks and
  sharing prefix blocks leave the output bit-identical; table padding and
  unwritten (NaN) rows are never read;
* ring mapping against hand-worked values from the slot equation, a
  brute-force last-writer simulation, and a survivor-order formulation;
* RoPE against complex multiplication, norm and relative-position invariance;
* write side: write-then-gather round trip, untouched rows keep their bytes.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import oracle
import workloads
from oracle.allocator import AllocatorError, BlockAllocatorModel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers (test-side, independent of the oracle's addressing)
# --------------------------------------------------------------------------

def logical_kv(case, b):
    """K/V of sequence b in logical order, straight from the generator's writes."""
    n = int(case.context_lens[b])
    hkv, d = case.num_kv_heads, case.head_dim
    k = np.full((n, hkv, d), np.nan)
    v = np.full((n, hkv, d), np.nan)
    for ch in case.writes:
        if ch.seq != b:
            continue
        for j, p in enumerate(ch.positions):
            k[int(p)] = oracle.to_f64(ch.keys[j], case.dtype)
            v[int(p)] = oracle.to_f64(ch.values[j], case.dtype)
    # shared-prefix cases write the prefix once, through sequence 0
    if np.isnan(k).any() and case.notes.get("prefix_blocks"):
        pk, pv = logical_kv_prefix(case)
        k[: pk.shape[0]] = pk
        v[: pv.shape[0]] = pv
    assert not np.isnan(k).any()
    return k, v


def logical_kv_prefix(case):
    ch = case.writes[0]
    return oracle.to_f64(ch.keys, case.dtype), oracle.to_f64(ch.values, case.dtype)


def sdpa_reference(q, k, v, scale):
    """q [Hq, D], k/v [n, Hkv, D] (float64) via torch SDPA with K/V repeated per group."""
    hq, hkv = q.shape[0], k.shape[1]
    g = hq // hkv
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    out = F.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return out[0, :, 0, :].numpy()


def decode_case(case, pools=None, tables=None):
    if pools is None:
        kp, vp, _ = oracle.build_pools(case)
    else:
        kp, vp = pools
    return oracle.decode(case.query, kp, vp, case.block_tables if tables is None else tables,
                         case.context_lens, case.scale, case.dtype, case.block_size, ring=case.ring)


# --------------------------------------------------------------------------
# dense special case and brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("maker", [workloads.config_tiny_fp32, workloads.config_embedded_1p1b])
def test_matches_library_attention_on_workload(maker):
    case = maker()
    out = decode_case(case)
    q = oracle.to_f64(case.query, case.dtype)
    for b in range(case.num_seqs):
        k, v = logical_kv(case, b)
        ref = sdpa_reference(q[b], k, v, case.scale)
        assert np.max(np.abs(out[b] - ref)) <= 1e-12


@settings(max_examples=40, deadline=None)
@given(
    hkv=st.sampled_from([1, 2, 3]),
    group=st.sampled_from([1, 2, 4, 6, 8]),
    d=st.sampled_from([8, 16, 64]),
    bs=st.sampled_from([1, 4, 16]),
    n=st.integers(min_value=1, max_value=70),
    seed=st.integers(min_value=0, max_value=2**31 - 1),
)
def test_identity_table_equals_dense_attention(hkv, group, d, bs, n, seed):
    """Contiguous pool + identity block table == textbook attention (GQA groups contiguous)."""
    rng = np.random.default_rng(seed)
    hq = hkv * group
    nblk = -(-n // bs)
    kp = rng.standard_normal((nblk, bs, hkv, d))
    vp = rng.standard_normal((nblk, bs, hkv, d))
    q = rng.standard_normal((1, hq, d))
    table = np.arange(nblk, dtype=np.int32)[None]
    scale = 1 / math.sqrt(d)
    out = oracle.decode(q, kp, vp, table, [n], scale, "f32", bs)
    k = kp.reshape(nblk * bs, hkv, d)[:n]
    v = vp.reshape(nblk * bs, hkv, d)[:n]
    ref = sdpa_reference(q[0], k, v, scale)
    assert np.max(np.abs(out[0] - ref)) <= 1e-12


def brute_force_decode(case):
    """Pure-Python loops with math.exp; addressing by T // bs, T % bs."""
    hq, d, hkv, bs = case.num_q_heads, case.head_dim, case.num_kv_heads, case.block_size
    g = hq // hkv
    out = [[[0.0] * d for _ in range(hq)] for _ in range(case.num_seqs)]
    kp, vp, _ = oracle.build_pools(case)
    kp = kp.astype(np.float64).tolist()
    vp = vp.astype(np.float64).tolist()
    q = case.query.astype(np.float64).tolist()
    for b in range(case.num_seqs):
        n = int(case.context_lens[b])
        table = [int(x) for x in case.block_tables[b]]
        for h in range(hq):
            kv = h // g
            scores = []
            for t in range(n):
                row = kp[table[t // bs]][t % bs][kv]
                scores.append(case.scale * sum(q[b][h][i] * row[i] for i in range(d)))
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for i in range(d):
                out[b][h][i] = sum(w[t] * vp[table[t // bs]][t % bs][kv][i] for t in range(n)) / tot
    return np.array(out)


def test_brute_force_tiny():
    case = workloads.config_tiny_fp32()
    assert list(case.context_lens) == [37, 70]
    out = decode_case(case)
    ref = brute_force_decode(case)
    assert np.max(np.abs(out - ref)) <= 1e-12


# --------------------------------------------------------------------------
# closed-form special cases
# --------------------------------------------------------------------------

def test_single_token_returns_v0_exactly():
    case = workloads.make_paged_case("n1", 7, "bf16", [1, 1, 1], 8, 2, 64, 16)
    out = decode_case(case)
    for b in range(3):
        v0 = oracle.to_f64(case.writes[b].values[0], "bf16")  # [Hkv, D]
        for h in range(8):
            assert np.array_equal(out[b, h], v0[h // 4])


def test_identical_keys_give_mean_of_values():
    case = workloads.make_paged_case("constk", 8, "f16", [45], 4, 1, 64, 16)
    k0 = case.writes[0].keys[0].copy()
    case.writes[0].keys[:] = k0
    out = decode_case(case)
    v = oracle.to_f64(case.writes[0].values, "f16")[:, 0, :]
    assert np.max(np.abs(out[0] - v.mean(axis=0))) <= 1e-13


def test_zero_length_gives_zeros():
    case = workloads.make_paged_case("n0", 9, "f16", [0, 5], 4, 2, 64, 16)
    out = decode_case(case)
    assert np.all(out[0] == 0.0)
    assert np.all(np.isfinite(out[1]))


def test_gqa_group_mapping_is_contiguous():
    """Head h must read KV head h // G: swapping KV heads changes exactly the matching q heads."""
    case = workloads.make_paged_case("gqa", 10, "f32", [33], 6, 2, 16, 4)
    base = decode_case(case)
    for ch in case.writes:
        ch.keys[:] = ch.keys[:, ::-1].copy()
        ch.values[:] = ch.values[:, ::-1].copy()
    swapped = decode_case(case)
    q = oracle.to_f64(case.query, "f32")
    k, v = logical_kv(case, 0)  # swapped content
    ref = sdpa_reference(q[0], k, v, case.scale)
    assert np.max(np.abs(swapped[0] - ref)) <= 1e-12
    assert not np.allclose(base[0, :3], swapped[0, :3])


# --------------------------------------------------------------------------
# invariances of the paging method
# --------------------------------------------------------------------------

def relabel_blocks(kp, vp, tables, perm):
    """Move physical block i to perm[i] and remap the tables (padding -1 stays)."""
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], tables).astype(np.int32)
    return kp2, vp2, t2


@pytest.mark.parametrize("maker", [workloads.config_tiny_fp32, workloads.config_embedded_1p1b])
def test_block_relabelling_is_bit_identical(maker):
    case = maker()
    kp, vp, _ = oracle.build_pools(case)
    base = decode_case(case, (kp, vp))
    perm = np.random.default_rng(3).permutation(case.num_blocks)
    kp2, vp2, t2 = relabel_blocks(kp, vp, case.block_tables, perm)
    moved = decode_case(case, (kp2, vp2), t2)
    assert np.array_equal(base, moved)


def test_shared_prefix_equals_private_copies_bit_identical():
    shared = workloads.config_shared_prefix(private_copies=False, batch=4)
    private = workloads.config_shared_prefix(private_copies=True, batch=4)
    assert np.array_equal(shared.context_lens, private.context_lens)
    ids = shared.notes["shared_prefix_ids"]
    for b in range(4):
        assert list(shared.block_tables[b, :4]) == ids
    a = decode_case(shared)
    b = decode_case(private)
    assert np.array_equal(a, b)
    q = oracle.to_f64(shared.query, "f16")
    for s in range(4):
        k, v = logical_kv(shared, s)
        assert np.max(np.abs(a[s] - sdpa_reference(q[s], k, v, shared.scale))) <= 1e-12


def test_table_padding_is_never_read():
    a = workloads.config_embedded_1p1b(pad_with_minus_one=False)
    b = workloads.config_embedded_1p1b(pad_with_minus_one=True)
    assert np.array_equal(decode_case(a), decode_case(b))


def test_unwritten_rows_are_nan_and_unread():
    case = workloads.config_tiny_fp32()
    kp, vp, _ = oracle.build_pools(case)
    written = 37 + 70
    assert np.isnan(kp).any(axis=(2, 3)).sum() == case.num_blocks * case.block_size - written
    assert np.all(np.isfinite(decode_case(case, (kp, vp))))


# --------------------------------------------------------------------------
# exact widening of stored 16-bit values
# --------------------------------------------------------------------------

def test_bf16_widening_every_bit_pattern():
    """bf16 bits widen as torch's own bfloat16 -> float64 conversion does,
    for all 65,536 patterns (NaN payloads compared as NaN)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.to_f64(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -133), (0x7F80, math.inf),
    (0xFF80, -math.inf), (0x8000, -0.0), (0x4049, 3.140625), (0x0080, 2.0 ** -126),
    (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127),
])
def test_bf16_widening_hand_values(bits, value):
    """bf16 is the top half of a binary32: sign, 8 exponent bits (bias 127),
    7 fraction bits; values worked by hand from that layout."""
    got = float(oracle.to_f64(np.array([bits], dtype=np.uint16), "bf16")[0])
    assert got == value and math.copysign(1.0, got) == math.copysign(1.0, value)


def test_f16_widening_hand_values():
    """binary16: 5 exponent bits (bias 15), 10 fraction bits."""
    for bits, value in [(0x3C00, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -24), (0x7BFF, 65504.0),
                        (0x3555, 0.333251953125)]:
        raw = np.array([bits], dtype=np.uint16).view(np.float16)
        assert float(oracle.to_f64(raw, "f16")[0]) == value


# --------------------------------------------------------------------------
# ring mapping
# --------------------------------------------------------------------------

def read_pairs(name):
    rows = []
    with open(f"{GOLDEN}/{name}") as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                rows.append([int(x) for x in line.split()])
    return rows


def test_ring_slot_hand_values():
    for pos, slot in read_pairs("ring_slots_s4_w1020.txt"):
        assert oracle.ring_slot(pos, 4, 1020) == slot


def test_ring_cache_order_hand_values():
    for row in read_pairs("ring_cache_order_s2_w3.txt"):
        n, slots = row[0], row[1:]
        assert oracle.ring_cache_order(n, 2, 3) == slots


@pytest.mark.parametrize("sink", [0, 1, 2, 4])
@pytest.mark.parametrize("window", [1, 2, 3, 5, 12])
def test_ring_last_writer_simulation(sink, window):
    """Appending positions 0..n-1 and keeping each slot's last writer leaves
    exactly the cache-order list, oldest surviving position first."""
    holder = {}
    for n in range(1, 120):
        p = n - 1
        holder[oracle.ring_slot(p, sink, window)] = p
        by_age = sorted(holder.items(), key=lambda kv: kv[1])
        assert [slot for slot, _ in by_age] == oracle.ring_cache_order(n, sink, window)
        survivors = [pos for _, pos in by_age]
        assert survivors == list(workloads.ring_survivor_positions(n, sink, window))
        # each slot's last writer, as the simulation kept it
        for slot, pos in holder.items():
            assert oracle.ring_writer(slot, n, sink, window) == pos
        for slot in range(sink + window):
            if slot not in holder:
                assert oracle.ring_writer(slot, n, sink, window) == -1
        # closed-form inverse: cache index of ring slot r
        for j, (slot, _) in enumerate(by_age):
            if n <= sink + window or slot < sink:
                expect = slot
            else:
                expect = sink + ((slot - sink) - (n - window - sink)) % window
            assert j == expect == oracle.ring_cache_index(slot, n, sink, window)


# --------------------------------------------------------------------------
# RoPE (rotate-half pairing is a reading; see the header of the oracle)
# --------------------------------------------------------------------------

def test_rope_equals_complex_multiplication():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 16))
    pos = np.array([0, 1, 7, 1000, 99_999])
    out = oracle.rope_rotate_half(x, pos, 10000.0)
    z = x[:, :8] + 1j * x[:, 8:]
    theta = 10000.0 ** (-np.arange(8) / 8.0)
    zr = z * np.exp(1j * pos[:, None] * theta[None, :])
    assert np.max(np.abs(out[:, :8] - zr.real)) < 1e-12
    assert np.max(np.abs(out[:, 8:] - zr.imag)) < 1e-12
    assert np.array_equal(oracle.rope_rotate_half(x, 0, 10000.0), x)


def test_rope_norm_and_relative_invariance():
    rng = np.random.default_rng(12)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, j, c in [(10, 3, 5), (1023, 0, 77), (5, 5, 1000)]:
        a = oracle.rope_rotate_half(q, m, 1e4) @ oracle.rope_rotate_half(k, j, 1e4)
        b = oracle.rope_rotate_half(q, m + c, 1e4) @ oracle.rope_rotate_half(k, j + c, 1e4)
        assert abs(a - b) < 1e-12
        assert abs(np.linalg.norm(oracle.rope_rotate_half(q, m, 1e4)) - np.linalg.norm(q)) < 1e-12


def test_ring_decode_equals_survivors_in_position_order():
    """Ring decode == attention over the resident positions sorted by age,
    keys rotated by their rank, query by the last rank.  Built without the
    slot mapping, straight from the generator's survivors."""
    lens = [1, 5, 17, 40, 41, 42, 100]
    case = workloads.config_sink_ring(lengths=lens, sink=2, window=37, block_size=4,
                                      num_q_heads=6, num_kv_heads=2, head_dim=16)
    out = decode_case(case)
    q = oracle.to_f64(case.query, "f16")
    for b, ch in enumerate(case.writes):
        order = np.argsort(ch.positions)
        k = oracle.to_f64(ch.keys[order], "f16")
        v = oracle.to_f64(ch.values[order], "f16")
        m = k.shape[0]
        kr = oracle.rope_rotate_half(k, np.arange(m)[:, None], 1e4)
        qr = oracle.rope_rotate_half(q[b], m - 1, 1e4)
        ref = sdpa_reference(qr, kr, v, case.scale)
        assert np.max(np.abs(out[b] - ref)) <= 1e-12


def test_ring_without_wrap_is_plain_paging_with_absolute_rope():
    case = workloads.config_sink_ring(lengths=[30, 39], sink=2, window=37, block_size=4,
                                      num_q_heads=4, num_kv_heads=2, head_dim=16)
    kp, vp, _ = oracle.build_pools(case)
    ring_out = decode_case(case, (kp, vp))
    # same pools, plain paging with keys/query pre-rotated by absolute position
    q = oracle.to_f64(case.query, "f16")
    for b in range(2):
        n = int(case.context_lens[b])
        k = oracle.to_f64(oracle.gather_rows(kp, case.block_tables[b], np.arange(n), 4), "f16")
        v = oracle.to_f64(oracle.gather_rows(vp, case.block_tables[b], np.arange(n), 4), "f16")
        kr = oracle.rope_rotate_half(k, np.arange(n)[:, None], 1e4)
        qr = oracle.rope_rotate_half(q[b], n - 1, 1e4)
        assert np.max(np.abs(ring_out[b] - sdpa_reference(qr, kr, v, case.scale))) <= 1e-12


# --------------------------------------------------------------------------
# write side
# --------------------------------------------------------------------------

def test_write_then_gather_round_trip_and_untouched_rows():
    case = workloads.config_embedded_1p1b()
    kp, vp, slots = oracle.build_pools(case)
    for b in range(case.num_seqs):
        n = int(case.context_lens[b])
        k = oracle.gather_rows(kp, case.block_tables[b], np.arange(n), case.block_size)
        assert np.array_equal(k.view(np.uint16), case.writes[b].keys.view(np.uint16))
    written = np.zeros(kp.shape[:2], dtype=bool)
    for s in np.concatenate(slots):
        written[s // 16, s % 16] = True
    assert np.all(kp.view(np.uint16)[~written] == workloads.NAN_BITS["f16"])
    # negative slots are skipped; duplicates rejected
    k2, _ = oracle.reshape_and_cache(kp, vp, case.writes[0].keys[:2], case.writes[0].values[:2],
                                     [-1, -5], 16)
    assert np.array_equal(k2.view(np.uint16), kp.view(np.uint16))
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(kp, vp, case.writes[0].keys[:2], case.writes[0].values[:2], [3, 3], 16)


def test_out_of_pool_ids_raise():
    pool = np.zeros((4, 2, 1, 8))
    with pytest.raises(IndexError):
        oracle.gather_rows(pool, np.array([0, 7]), [3], 2)


# --------------------------------------------------------------------------
# allocator model
# --------------------------------------------------------------------------

def test_allocator_lowest_free_first_and_exhaustion():
    a = BlockAllocatorModel(70)
    got = [a.alloc() for _ in range(70)]
    assert got == list(range(70))
    assert a.alloc() == -1
    a.decref(5)
    a.decref(40)
    assert a.alloc() == 5
    assert a.alloc() == 40
    assert a.alloc() == -1


def test_allocator_refcounts_and_stats():
    a = BlockAllocatorModel(8)
    ids = [a.alloc() for _ in range(4)]
    for _ in range(3):
        a.incref(ids[0])
    assert a.stats() == {"total": 8, "used": 4, "shared": 1, "free": 4}
    for _ in range(3):
        a.decref(ids[0])
    assert a.stats()["shared"] == 0 and a.stats()["used"] == 4
    a.decref(ids[0])
    assert a.stats()["used"] == 3
    with pytest.raises(AllocatorError) as e:
        a.decref(ids[0])
    assert e.value.kind == "state"
    with pytest.raises(AllocatorError) as e:
        a.incref(99)
    assert e.value.kind == "inval"


# --------------------------------------------------------------------------
# closed forms against the printed numbers
# --------------------------------------------------------------------------

def read_sizes():
    out = {}
    with open(f"{GOLDEN}/kv_sizes_printed.txt") as fh:
        for line in fh:
            line = line.split("|")[0].split("#")[0].strip()
            if line:
                key, val, unit, tol = line.split()
                out[key] = (float(val), unit, float(tol))
    return out


def test_closed_forms_match_printed_sizes():
    s = read_sizes()
    sz = oracle.sizes
    per_layer = sz.kv_bytes_per_token(1, 2, 128, 2)
    per_token = sz.kv_bytes_per_token(24, 2, 128, 2)
    assert per_layer == s["per_layer_per_token_bytes"][0]
    assert per_token == s["per_token_all_layers_bytes"][0]
    assert abs(512 * per_token / 1024 / 1000 - s["tokens512_KiBk"][0]) <= s["tokens512_KiBk"][2]
    assert abs(2048 * per_token / 1024 / 1000 - s["tokens2048_KiBk"][0]) <= s["tokens2048_KiBk"][2]
    blk = sz.block_bytes(16, per_token)
    assert blk == s["block_bytes"][0]
    assert 512 * blk / 2**20 == s["pool512_MiB"][0]
    one = sz.kv_cache_bytes(80, 4096, 8, 128, 2)
    assert one == 1_342_177_280
    assert abs(one / 1e9 - s["llama70b_4096_GB"][0]) <= s["llama70b_4096_GB"][2]
    b16 = sz.kv_cache_bytes(80, 4096, 8, 128, 2, batch=16)
    assert 0 <= b16 / 1e9 - s["llama70b_4096_b16_GB"][0] <= s["llama70b_4096_b16_GB"][2]
    assert abs(100 * sz.preallocation_waste(50, 4096) - s["waste_50_of_4096_pct"][0]) <= 0.05
    assert abs(100 * sz.preallocation_waste(200, 4096) - s["waste_200_of_4096_pct"][0]) <= 0.05
    assert sz.preallocation_waste(8000, 4096) == 0.0
    assert [sz.blocks_needed(n, 16) for n in (0, 1, 16, 17, 8000)] == [0, 1, 1, 2, 500]


# ---------------------------------------------------------------------------
# FP8 (E4M3) KV storage
# ---------------------------------------------------------------------------

def _e4m3_golden():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_codes.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            x, code, value = line.split()[:3]
            rows.append((float(x), int(code, 16), float(value)))
    return rows


def test_e4m3_codes_worked_by_hand():
    from oracle import fp8

    rows = _e4m3_golden()
    assert len(rows) >= 20
    for x, code, value in rows:
        assert fp8.e4m3_encode_one(np.float32(x)) == code, (x, hex(code))
        got = fp8.e4m3_value(code)
        assert got == value or (got == 0.0 and value == 0.0 and np.signbit(got) == np.signbit(value)), (x, got)
    assert np.isnan(fp8.e4m3_value(0x7F)) and np.isnan(fp8.e4m3_value(0xFF))
    assert fp8.e4m3_encode_one(np.float32("nan")) == 0x7F


def test_e4m3_every_finite_code_round_trips_and_order_is_kept():
    from oracle import fp8

    finite = [c for c in range(256) if not np.isnan(fp8.e4m3_value(c))]
    assert len(finite) == 254
    for c in finite:
        assert fp8.e4m3_value(fp8.e4m3_encode_one(np.float32(fp8.e4m3_value(c)))) == fp8.e4m3_value(c)
    # the positive codes 0x00..0x7e are strictly increasing in value
    pos = [fp8.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))
    rng = np.random.default_rng(7)
    xs = np.sort(rng.uniform(-500, 500, 4000).astype(np.float32))
    dec = fp8.e4m3_decode(fp8.e4m3_encode(xs))
    assert np.all(np.diff(dec) >= 0)


def test_e4m3_array_encoder_equals_the_scalar_search():
    from oracle import fp8

    rng = np.random.default_rng(9)
    xs = np.concatenate([rng.uniform(-500, 500, 3000), rng.normal(0, 0.02, 3000),
                         fp8.E4M3_TABLE[np.isfinite(fp8.E4M3_TABLE)],
                         (fp8._MAGNITUDES[:-1] + fp8._MAGNITUDES[1:]) / 2,  # every midpoint (ties)
                         [0.0, -0.0, 448.0, 449.0, -1e9, np.nan]]).astype(np.float32)
    got = fp8.e4m3_encode(xs)
    want = np.array([fp8.e4m3_encode_one(v) for v in xs], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_rounding_is_to_a_neighbour_within_half_a_step():
    """Independent of the encoder's search: the result must be one of the two
    representable neighbours, within half their spacing."""
    from oracle import fp8

    rng = np.random.default_rng(8)
    xs = np.concatenate([rng.uniform(-448, 448, 3000), rng.normal(0, 0.01, 1000)]).astype(np.float32)
    for x in xs:
        a = abs(float(x))
        # neighbours from the format: exponent of a, step 2^(e-3), subnormal step 2^-9
        if a < 2.0 ** -6:
            step = 2.0 ** -9
        else:
            step = 2.0 ** (np.floor(np.log2(a)) - 3)
        lo = np.floor(a / step) * step
        got = abs(fp8.e4m3_value(fp8.e4m3_encode_one(x)))
        assert got in (lo, lo + step) or (a >= 448 and got == 448.0)
        assert abs(got - a) <= step / 2 + 1e-300


# ---------------------------------------------------------------------------
# FP8 (E5M2) KV storage
# ---------------------------------------------------------------------------

def _e5m2_golden():
    rows = []
    with open(os.path.join(GOLDEN, "e5m2_codes.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            x, code, value = line.split()[:3]
            rows.append((float(x), int(code, 16), float(value)))
    return rows


def test_e5m2_codes_worked_by_hand():
    from oracle import fp8

    rows = _e5m2_golden()
    assert len(rows) >= 25
    for x, code, value in rows:
        assert fp8.e5m2_encode_one(np.float32(x)) == code, (x, hex(code))
        got = fp8.e5m2_value(code)
        assert got == value or (got == 0.0 and value == 0.0 and np.signbit(got) == np.signbit(value)), (x, got)
    for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF):
        assert np.isnan(fp8.e5m2_value(c))
    assert fp8.e5m2_value(0x7C) == np.inf and fp8.e5m2_value(0xFC) == -np.inf
    assert fp8.e5m2_encode_one(np.float32("nan")) == 0x7F


def test_e5m2_is_the_top_byte_of_ieee_half():
    """E5M2 shares binary16's sign, exponent width and bias; its 2 mantissa
    bits are binary16's top 2.  So code c is the half-precision number with
    bits c << 8 (numpy's float16, an independent implementation of IEEE
    binary16), for every code: zeros, subnormals, normals, infinities, NaN."""
    from oracle import fp8

    halves = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    for c in range(256):
        h, v = halves[c], fp8.e5m2_value(c)
        assert (np.isnan(h) and np.isnan(v)) or (h == v and np.signbit(h) == np.signbit(v)), (hex(c), h, v)


def test_e5m2_every_finite_code_round_trips_and_order_is_kept():
    from oracle import fp8

    finite = [c for c in range(256) if np.isfinite(fp8.e5m2_value(c))]
    assert len(finite) == 248  # 256 - 2 infinities - 6 NaNs
    for c in finite:
        assert fp8.e5m2_value(fp8.e5m2_encode_one(np.float32(fp8.e5m2_value(c)))) == fp8.e5m2_value(c)
    pos = [fp8.e5m2_value(c) for c in range(0x7C)]
    assert all(a < b for a, b in zip(pos, pos[1:]))
    rng = np.random.default_rng(17)
    xs = np.sort(rng.uniform(-60000, 60000, 4000).astype(np.float32))
    dec = fp8.e5m2_decode(fp8.e5m2_encode(xs))
    assert np.all(np.diff(dec) >= 0)


def test_e5m2_array_encoder_equals_the_scalar_search():
    from oracle import fp8

    rng = np.random.default_rng(19)
    mags = fp8._E5M2_MAGNITUDES
    xs = np.concatenate([rng.uniform(-60000, 60000, 3000), rng.normal(0, 0.02, 3000),
                         rng.normal(0, 1e-4, 1000),
                         fp8.E5M2_TABLE[np.isfinite(fp8.E5M2_TABLE)],
                         (mags[:-1] + mags[1:]) / 2,  # every midpoint (ties)
                         [0.0, -0.0, 57344.0, 61440.0, -1e9, np.inf, -np.inf, np.nan]]).astype(np.float32)
    got = fp8.e5m2_encode(xs)
    want = np.array([fp8.e5m2_encode_one(v) for v in xs], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e5m2_rounding_is_to_a_neighbour_within_half_a_step():
    """Independent of the encoder's search: one of the two representable
    neighbours (spacing 2^(e-2), subnormal spacing 2^-16), within half a
    step; the tie goes to the even code."""
    from oracle import fp8

    rng = np.random.default_rng(18)
    xs = np.concatenate([rng.uniform(-57344, 57344, 3000), rng.normal(0, 0.01, 1000),
                         rng.normal(0, 3e-5, 1000)]).astype(np.float32)
    for x in xs:
        a = abs(float(x))
        step = 2.0 ** -16 if a < 2.0 ** -14 else 2.0 ** (np.floor(np.log2(a)) - 2)
        lo = np.floor(a / step) * step
        code = fp8.e5m2_encode_one(x)
        got = abs(fp8.e5m2_value(code))
        assert got in (lo, lo + step), (x, got)
        assert abs(got - a) <= step / 2
        if abs(got - a) == step / 2:
            assert code % 2 == 0, (x, hex(code))


@pytest.mark.parametrize("kv_format", ["e4m3", "e5m2"])
def test_fp8_decode_equals_attention_on_dequantised_pools(kv_format):
    """The fp8 path of decode is attention on scale[h] * value(code): build a
    float64 pool from the codes by hand and compare (E5M2 values through
    numpy's binary16, of which E5M2 is the top byte)."""
    from oracle import fp8

    case = workloads.config_fp8(workloads.config_tiny_fp32, kv_format=kv_format)
    kp, vp, _ = oracle.build_pools(case)
    assert kp.dtype == np.uint8
    if kv_format == "e4m3":
        table = fp8.E4M3_TABLE
        encode_one = fp8.e4m3_encode_one
    else:
        table = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
        encode_one = fp8.e5m2_encode_one
    ref_k = table[kp] * case.k_scale.astype(np.float64)[None, None, :, None]
    ref_v = table[vp] * case.v_scale.astype(np.float64)[None, None, :, None]
    got = oracle.decode(case.query, kp, vp, case.block_tables, case.context_lens, case.scale, case.dtype,
                        case.block_size, kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale)
    q = oracle.to_f64(case.query, case.dtype)
    g = case.num_q_heads // case.num_kv_heads
    for b in range(case.num_seqs):
        n = int(case.context_lens[b])
        rows_k = np.stack([ref_k[case.block_tables[b, t // case.block_size], t % case.block_size] for t in range(n)])
        rows_v = np.stack([ref_v[case.block_tables[b, t // case.block_size], t % case.block_size] for t in range(n)])
        for h in range(case.num_q_heads):
            s = case.scale * rows_k[:, h // g, :] @ q[b, h]
            p = np.exp(s - s.max())
            np.testing.assert_allclose(got[b, h], (p / p.sum()) @ rows_v[:, h // g, :], rtol=0, atol=1e-12)
    # the quantisation is a float32 product with 1/scale, then the nearest
    # code (ties to even) of the format
    ch = case.writes[0]
    x = oracle.to_f64(ch.keys, case.dtype).astype(np.float32)
    inv = (np.float32(1) / case.k_scale.astype(np.float32)).astype(np.float32)
    codes = oracle.quantize_for_cache(ch.keys, case.dtype, case.k_scale, case.kv_dtype)
    for idx in [(0, 0, 0), (3, 1, 17), (10, 1, 63)]:
        prod = np.float32(x[idx] * inv[idx[1]])
        assert codes[idx] == encode_one(prod)

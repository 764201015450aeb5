"""Pins for the oracle's speculative verification over the sink + ring
cache (``oracle.decode_verify_ring``), each from outside the function:

* sequential decoding: row i equals the single-token ring decode after the
  drafts 0..i are written into a copy of the cache (the verification must
  reproduce what decoding the drafts one at a time gives);
* a position formulation written here from the Slot(pos) equation and
  rotate-half RoPE, sharing nothing with the oracle's ring code: token i at
  position p sees the sinks and positions max(S, p + 1 - W) .. p; a window
  key sits at its true distance p - pos from the query, a sink key at
  min(p, S + W - 1) - pos (the query's cache index is capped at S + W - 1);
* no wrap (n + q_len <= S + W): dense causal attention with absolute RoPE
  positions, by torch's scaled_dot_product_attention in float64;
* relabelling physical blocks leaves the result bit-identical; the oracle
  does not modify the pools (rejected drafts leave nothing to undo).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads


def _pools(case):
    k, v, _ = oracle.build_pools(case)
    return k, v


def _verify(case, k=None, v=None, tables=None):
    if k is None:
        k, v = _pools(case)
    return oracle.decode_verify_ring(case.query, case.draft_keys, case.draft_values, k, v,
                                     case.block_tables if tables is None else tables, case.context_lens,
                                     case.scale, case.dtype, case.block_size, case.ring, kv_dtype=case.kv_dtype,
                                     k_scale=case.k_scale, v_scale=case.v_scale)


def _rows_by_position(case, b):
    """K/V rows of stream b keyed by logical position (committed survivors
    and this step's drafts), straight from the generator."""
    rows = {}
    for ch in case.writes:
        if ch.seq == b:
            for j, p in enumerate(ch.positions):
                rows[int(p)] = (oracle.to_f64(ch.keys[j], case.dtype), oracle.to_f64(ch.values[j], case.dtype))
    n = int(case.context_lens[b])
    for i in range(case.q_len):
        rows[n + i] = (oracle.to_f64(case.draft_keys[b, i], case.dtype),
                       oracle.to_f64(case.draft_values[b, i], case.dtype))
    return rows


def _rotate(x, angle_steps, base):
    """Rotate-half RoPE as complex multiplication: (x_k + i x_{k+D/2}) e^{i m theta_k}."""
    d = x.shape[-1]
    theta = base ** (-2.0 * np.arange(d // 2) / d)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * angle_steps * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def _by_positions(case):
    s, w, base = case.ring.sink, case.ring.window, case.ring.rope_base
    hq, hkv = case.num_q_heads, case.num_kv_heads
    g_size = hq // hkv
    out = np.zeros((case.num_seqs, case.q_len, hq, case.head_dim))
    for b in range(case.num_seqs):
        rows = _rows_by_position(case, b)
        n = int(case.context_lens[b])
        for i in range(case.q_len):
            p = n + i
            visible = [pos for pos in range(p + 1) if pos < s or pos >= p + 1 - w]
            q = oracle.to_f64(case.query[b, i], case.dtype)
            for h in range(hq):
                g = h // g_size
                scores, vals = [], []
                for pos in visible:
                    dist = (min(p, s + w - 1) - pos) if pos < s else (p - pos)
                    k, v = rows[pos]
                    scores.append(case.scale * float(np.dot(_rotate(q[h], dist, base), k[g])))
                    vals.append(v[g])
                sc = np.array(scores)
                wts = np.exp(sc - sc.max())
                out[b, i, h] = (wts / wts.sum()) @ np.array(vals)
    return out


SMALL = [
    # (S, W, block size, committed lengths, q_len): wraps before, during and after the step
    (4, 12, 4, [0, 1, 3, 4, 9, 12, 15, 16, 17, 40, 41], 5),
    (2, 3, 4, [0, 1, 2, 4, 5, 6, 11], 4),     # q_len > W: drafts evict drafts
    (0, 5, 4, [0, 3, 5, 6, 13], 3),           # no sinks
    (3, 1, 4, [0, 2, 3, 4, 9], 2),            # a one-slot window
]


def _small(spec, seed_offset=40, dtype="f16"):
    s, w, bs, lens, ql = spec
    return workloads.config_ring_verify(lengths=lens, q_len=ql, seed_offset=seed_offset, sink=s, window=w,
                                        block_size=bs, num_q_heads=4, num_kv_heads=2, head_dim=16, dtype=dtype)


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: f"S{s[0]}-W{s[1]}-q{s[4]}")
def test_verify_equals_the_position_formulation(spec):
    case = _small(spec)
    np.testing.assert_allclose(_verify(case), _by_positions(case), rtol=0, atol=1e-12)


def test_verify_equals_the_position_formulation_on_the_workload_shape():
    case = workloads.config_ring_verify(lengths=[0, 5, 1020, 1022, 1024, 1030, 3000])
    np.testing.assert_allclose(_verify(case), _by_positions(case), rtol=0, atol=1e-12)


@pytest.mark.parametrize("spec", SMALL[:2], ids=lambda s: f"S{s[0]}-W{s[1]}-q{s[4]}")
@pytest.mark.parametrize("kv_dtype", [None, "fp8_e4m3"])
def test_verify_equals_sequential_decode(spec, kv_dtype):
    """Row i = single-token ring decode after writing drafts 0..i (8-bit
    pools: the write stores their codes)."""
    case = _small(spec, seed_offset=41, dtype="bf16")
    if kv_dtype is not None:
        case.kv_dtype = kv_dtype
        case.k_scale = np.full(case.num_kv_heads, 5.0 / 448, dtype=np.float32)
        case.v_scale = np.full(case.num_kv_heads, 4.0 / 448, dtype=np.float32)
    k, v = _pools(case)
    got = _verify(case, k, v)
    s, w = case.ring.sink, case.ring.window
    for b in range(case.num_seqs):
        n = int(case.context_lens[b])
        kk, vv = k.copy(), v.copy()
        for i in range(case.q_len):
            slot = oracle.slot_of(case.block_tables[b], oracle.ring_slot(n + i, s, w), case.block_size)
            rk, rv = case.draft_keys[b, i:i + 1], case.draft_values[b, i:i + 1]
            if kv_dtype is not None:
                rk = oracle.quantize_for_cache(rk, case.dtype, case.k_scale, kv_dtype)
                rv = oracle.quantize_for_cache(rv, case.dtype, case.v_scale, kv_dtype)
            oracle.reshape_and_cache_(kk, vv, rk, rv, [slot], case.block_size)
            ref = oracle.decode(case.query[b:b + 1, i], kk, vv, case.block_tables[b:b + 1],
                                np.array([n + i + 1]), case.scale, case.dtype, case.block_size, ring=case.ring,
                                kv_dtype=kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale)
            assert np.array_equal(got[b, i], ref[0])


def test_verify_without_wrap_is_dense_causal_rope_attention():
    """n + q_len <= S + W: nothing is evicted and cache order is position
    order, so each draft attends causally over positions 0..p with
    absolute RoPE."""
    case = workloads.config_ring_verify(lengths=[0, 1, 7, 300, 1019], q_len=5)
    got = _verify(case)
    base = case.ring.rope_base
    g = case.num_q_heads // case.num_kv_heads
    for b in range(case.num_seqs):
        rows = _rows_by_position(case, b)
        n = int(case.context_lens[b])
        total = n + case.q_len
        k = np.stack([rows[p][0] for p in range(total)])  # [T, Hkv, D]
        v = np.stack([rows[p][1] for p in range(total)])
        k = oracle.rope_rotate_half(k, np.arange(total)[:, None], base)
        q = oracle.rope_rotate_half(oracle.to_f64(case.query[b], case.dtype), np.arange(n, total)[:, None], base)
        qt = torch.from_numpy(q).permute(1, 0, 2)  # [Hq, q_len, D]
        kt = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)
        vt = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)
        mask = torch.from_numpy(np.arange(total)[None, :] <= np.arange(n, total)[:, None])
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=case.scale)
        np.testing.assert_allclose(got[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_verify_is_invariant_under_block_relabelling_and_leaves_pools():
    case = workloads.config_ring_verify(lengths=[0, 17, 1023, 1025, 5000])
    k, v = _pools(case)
    k0, v0 = k.copy(), v.copy()
    base = _verify(case, k, v)
    assert np.array_equal(k, k0, equal_nan=True) and np.array_equal(v, v0, equal_nan=True)
    perm = np.random.default_rng(5).permutation(case.num_blocks)
    k2, v2 = np.empty_like(k), np.empty_like(v)
    k2[perm], v2[perm] = k, v
    tables = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], case.block_tables)
    assert np.array_equal(_verify(case, k2, v2, tables), base)

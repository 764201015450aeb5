"""Pins for the oracle's multi-token decode (several new tokens per
sequence attending causally over the paged cache).

* q_len = 1 is exactly single-token ``decode``;
* new token i equals single-token ``decode`` over its own prefix
  (context p + 1), for every token of every sequence;
* dense causal attention: an identity block table over a dense pool against
  torch's scaled_dot_product_attention (float64 on the CPU) with an explicit
  mask that lets token i see keys 0 .. L - q_len + i;
* causality: rewriting keys and values after a token's position leaves its
  row bit-identical; rewriting the key at its own position changes it;
* tokens whose position is negative (context shorter than q_len) are zeros.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads


def _pools(case):
    kp, vp, _ = oracle.build_pools(case)
    return kp, vp


def test_q_len_one_is_decode():
    case = workloads.make_multi_case("m1", 7001, "f32", [1, 16, 17, 40], 1, 6, 2, 64, 16)
    kp, vp = _pools(case)
    got = oracle.decode_multi(case.query, kp, vp, case.block_tables, case.context_lens, case.scale,
                              case.dtype, case.block_size, 1)
    want = oracle.decode(case.query[:, 0], kp, vp, case.block_tables, case.context_lens, case.scale,
                         case.dtype, case.block_size)
    assert np.array_equal(got[:, 0], want)


def test_each_token_is_decode_over_its_prefix():
    case = workloads.config_spec_verify_tiny()
    kp, vp = _pools(case)
    q = case.q_len
    got = oracle.decode_multi(case.query, kp, vp, case.block_tables, case.context_lens, case.scale,
                              case.dtype, case.block_size, q)
    for i in range(q):
        lens_i = np.maximum(case.context_lens - q + i + 1, 0).astype(np.int32)
        want = oracle.decode(case.query[:, i], kp, vp, case.block_tables, lens_i, case.scale,
                             case.dtype, case.block_size)
        assert np.array_equal(got[:, i], want), i


def test_dense_causal_attention_against_sdpa():
    rng = np.random.default_rng(3)
    hq, hkv, d, bs, q = 8, 2, 64, 16, 7
    L = 45
    nblk = -(-L // bs)
    k = rng.standard_normal((nblk * bs, hkv, d)).astype(np.float32)
    v = rng.standard_normal((nblk * bs, hkv, d)).astype(np.float32)
    kp = k.reshape(nblk, bs, hkv, d)
    vp = v.reshape(nblk, bs, hkv, d)
    query = rng.standard_normal((1, q, hq, d)).astype(np.float32)
    table = np.arange(nblk, dtype=np.int32)[None]
    scale = 0.125
    got = oracle.decode_multi(query, kp, vp, table, np.array([L], dtype=np.int32), scale, "f32", bs, q)
    g = hq // hkv
    kk = torch.from_numpy(k[:L].astype(np.float64)).repeat_interleave(g, dim=1).permute(1, 0, 2)  # [Hq, L, D]
    vv = torch.from_numpy(v[:L].astype(np.float64)).repeat_interleave(g, dim=1).permute(1, 0, 2)
    qq = torch.from_numpy(query[0].astype(np.float64)).permute(1, 0, 2)  # [Hq, q, D]
    mask = torch.arange(L)[None, :] <= (L - q + torch.arange(q))[:, None]  # token i sees 0 .. L-q+i
    want = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)  # [Hq, q, D]
    assert np.max(np.abs(got[0] - want.permute(1, 0, 2).numpy())) < 1e-12


def test_later_keys_never_reach_a_token():
    case = workloads.make_multi_case("m2", 7002, "f32", [30, 50], 6, 4, 2, 64, 16)
    kp, vp = _pools(case)
    args = (case.block_tables, case.context_lens, case.scale, case.dtype, case.block_size, 6)
    base = oracle.decode_multi(case.query, kp, vp, *args)
    b, i = 1, 2
    pos = int(case.context_lens[b]) - 6 + i
    k2, v2 = kp.copy(), vp.copy()
    for p in range(pos + 1, int(case.context_lens[b])):  # every key after token i's position
        blk, off = case.block_tables[b, p // 16], p % 16
        k2[blk, off] = 9.0
        v2[blk, off] = -9.0
    after = oracle.decode_multi(case.query, k2, v2, *args)
    assert np.array_equal(after[b, : i + 1], base[b, : i + 1])
    assert not np.array_equal(after[b, i + 1], base[b, i + 1])
    k3 = kp.copy()
    blk, off = case.block_tables[b, pos // 16], pos % 16
    k3[blk, off] = 3.0  # the key at token i's own position is visible to it
    assert not np.array_equal(oracle.decode_multi(case.query, k3, vp, *args)[b, i], base[b, i])


def test_tokens_before_position_zero_are_zero():
    case = workloads.config_spec_verify_tiny()  # first sequence: 3 tokens, q_len 5
    kp, vp = _pools(case)
    got = oracle.decode_multi(case.query, kp, vp, case.block_tables, case.context_lens, case.scale,
                              case.dtype, case.block_size, case.q_len)
    assert np.all(got[0, :2] == 0.0)
    assert np.all(np.abs(got[0, 2:]).max(axis=-1) > 0)

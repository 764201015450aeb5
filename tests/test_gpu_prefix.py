"""GPU parity of the copy-on-write block copy and of decode over prefixes
shared through the prefix index.

* pa_copy_blocks against the oracle's copy, byte for byte, for every pool
  dtype (8-bit codes included), single- and multi-segment blocks, a ragged
  last segment, padding and out-of-pool pairs;
* the prefix-sharing workloads: a resident system prompt that ends inside a
  block, requests that extend it (copy-on-write of its tail), leave it inside
  the tail or inside a full block, share nothing, or repeat an earlier
  request.  Tables come from the library's index (and equal the oracle
  model's); the pools after the writes and copies equal the oracle's bit for
  bit; decode is within the parity tolerance of the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_145_amd as pk
import workloads
from gpu_support import TORCH_DTYPES, assert_parity, raw_to_torch
from oracle.prefix import copy_blocks as oracle_copy_blocks
from prefix_support import LibApi, ModelApi, admit, padded_tables

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _pool_tensors(shape, dtype, rng):
    """Pools of random bytes (every bit pattern, NaNs included)."""
    nbytes = int(np.prod(shape)) * (1 if dtype == "fp8" else 4 if dtype == "f32" else 2)
    raw_k = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    raw_v = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    tdt = torch.uint8 if dtype == "fp8" else TORCH_DTYPES[dtype]
    k = torch.from_numpy(raw_k).to(DEV).view(tdt).view(shape)
    v = torch.from_numpy(raw_v).to(DEV).view(tdt).view(shape)
    return raw_k.reshape(shape[0], -1), raw_v.reshape(shape[0], -1), k, v


def _make_pool(k, v, bs, dtype, hkv):
    if dtype == "fp8":
        ks, vs = workloads.fp8_scales(hkv)
        return pk.Pool(k, v, bs, act_dtype=torch.bfloat16, k_scale=ks, v_scale=vs)
    return pk.Pool(k, v, bs)


@pytest.mark.parametrize("dtype,nb,bs,hkv,d", [
    ("f32", 20, 64, 16, 128),   # 512 KiB blocks: 32 full segments
    ("f16", 33, 16, 3, 64),     # 6 KiB blocks: one ragged segment
    ("bf16", 17, 16, 10, 128),  # 40 KiB blocks: three segments, the last ragged
    ("bf16", 300, 16, 8, 128),  # 70B-shaped blocks
    ("fp8", 40, 64, 8, 128),    # 64 KiB blocks of E4M3 codes
])
def test_copy_blocks_bit_exact(dtype, nb, bs, hkv, d):
    print(f"copy_blocks {dtype} nb={nb} bs={bs} hkv={hkv} d={d}", flush=True)
    rng = np.random.default_rng(nb * 7 + bs)
    shape = (nb, bs, hkv, d)
    raw_k, raw_v, k, v = _pool_tensors(shape, dtype, rng)
    pool = _make_pool(k, v, bs, dtype, hkv)
    perm = rng.permutation(nb)
    half = nb // 2
    src = [int(x) for x in perm[:half]]
    dst = [int(x) for x in perm[half:2 * half]]
    src += [-1, nb + 3, 0]  # padding, outside the pool, and a pair whose destination is outside
    dst += [int(perm[-1]), int(perm[-1]), nb]
    s_t = torch.tensor(src, dtype=torch.int32, device=DEV)
    d_t = torch.tensor(dst, dtype=torch.int32, device=DEV)
    pk.copy_blocks(pool, s_t, d_t)
    torch.cuda.synchronize()
    oracle_copy_blocks(raw_k, raw_v, src, dst)
    got_k = k.contiguous().view(torch.uint8).view(nb, -1).cpu().numpy()
    got_v = v.contiguous().view(torch.uint8).view(nb, -1).cpu().numpy()
    assert np.array_equal(got_k, raw_k)
    assert np.array_equal(got_v, raw_v)
    # zero pairs: nothing changes
    pk.copy_blocks(pool, s_t[:0], d_t[:0])
    torch.cuda.synchronize()
    assert np.array_equal(k.contiguous().view(torch.uint8).view(nb, -1).cpu().numpy(), raw_k)
    pool.close()


def _write(pool, table_rows, positions_per_row, keys, values, sc):
    """Device writes through the library's slot mapping."""
    if not positions_per_row:
        return
    bt = padded_tables_from_rows(table_rows)
    sid = np.concatenate([np.full(len(p), i, dtype=np.int32) for i, p in enumerate(positions_per_row)])
    pos = np.concatenate([np.asarray(p, dtype=np.int64) for p in positions_per_row])
    if sid.size == 0:
        return
    slots = pk.compute_slot_mapping(pool, bt, sid, pos)
    pk.reshape_and_cache(pool, raw_to_torch(keys, sc.dtype).to(DEV), raw_to_torch(values, sc.dtype).to(DEV),
                         torch.from_numpy(slots).to(DEV))
    return slots


def padded_tables_from_rows(rows):
    width = max(1, max(len(r) for r in rows))
    out = np.full((len(rows), width), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        out[i, : len(r)] = r
    return out


def _oracle_rows(rows, sc, which):
    if sc.kv_dtype == "fp8_e4m3":
        return oracle.quantize_for_cache(rows, sc.dtype, sc.k_scale if which == "k" else sc.v_scale)
    return rows


def _oracle_write(kp, vp, table, positions, keys, values, sc):
    slots = [oracle.slot_of(np.asarray(table), int(p), sc.block_size) for p in positions]
    oracle.reshape_and_cache_(kp, vp, _oracle_rows(keys, sc, "k"), _oracle_rows(values, sc, "v"),
                              np.asarray(slots, dtype=np.int64), sc.block_size)


@pytest.mark.parametrize("name", ["prefix_unaligned", "prefix_unaligned_fp8", "prefix_unaligned_small"])
def test_shared_unaligned_prefix_decode(name):
    print(f"prefix decode {name}", flush=True)
    sc = workloads.PREFIX_CONFIGS[name]()
    shape = (sc.num_blocks, sc.block_size, sc.num_kv_heads, sc.head_dim)
    fp8 = sc.kv_dtype == "fp8_e4m3"
    if fp8:
        k = torch.full(shape, workloads.FP8_NAN_CODE, dtype=torch.uint8, device=DEV)
        v = torch.full_like(k, workloads.FP8_NAN_CODE)
        pool = pk.Pool(k, v, sc.block_size, act_dtype=TORCH_DTYPES[sc.dtype], k_scale=sc.k_scale,
                       v_scale=sc.v_scale)
    else:
        nan = torch.from_numpy(workloads.nan_array((1,), sc.dtype).view(
            np.int32 if sc.dtype == "f32" else np.int16)).to(DEV)
        k = torch.empty(shape, dtype=TORCH_DTYPES[sc.dtype], device=DEV)
        v = torch.empty_like(k)
        ib = torch.int32 if sc.dtype == "f32" else torch.int16
        k.view(ib).copy_(nan.expand(shape))
        v.view(ib).copy_(nan.expand(shape))
        pool = pk.Pool(k, v, sc.block_size)
    from paged_kv_cache_145_amd import _lib

    adm = admit(LibApi(_lib.load(), pool.handle, sc.block_size), sc)
    ref_adm = admit(ModelApi(sc.num_blocks, sc.block_size), sc)
    assert adm == ref_adm
    assert adm.copies, "the workload must exercise copy-on-write"

    # device: system prompt once, then the tail copies, then every request's own rows
    p = len(sc.system_tokens)
    _write(pool, [adm.system_blocks], [np.arange(p)], sc.system_keys, sc.system_values, sc)
    src = torch.tensor([s for s, _ in adm.copies], dtype=torch.int32, device=DEV)
    dst = torch.tensor([d for _, d in adm.copies], dtype=torch.int32, device=DEV)
    pk.copy_blocks(pool, src, dst)
    own_pos = [np.arange(cov, len(r.tokens)) for cov, r in zip(adm.covered, sc.requests)]
    own_k = np.concatenate([r.keys[cov:] for cov, r in zip(adm.covered, sc.requests)])
    own_v = np.concatenate([r.values[cov:] for cov, r in zip(adm.covered, sc.requests)])
    _write(pool, adm.tables, own_pos, own_k, own_v, sc)

    # oracle: the same steps on host pools
    kp, vp = sc.empty_pool(), sc.empty_pool()
    _oracle_write(kp, vp, adm.system_blocks, np.arange(p), sc.system_keys, sc.system_values, sc)
    oracle.prefix.copy_blocks(kp, vp, [s for s, _ in adm.copies], [d for _, d in adm.copies])
    for t, cov, r in zip(adm.tables, adm.covered, sc.requests):
        _oracle_write(kp, vp, t, np.arange(cov, len(r.tokens)), r.keys[cov:], r.values[cov:], sc)
    torch.cuda.synchronize()
    view = torch.uint8
    assert np.array_equal(k.contiguous().view(view).cpu().numpy().reshape(-1),
                          np.ascontiguousarray(kp).view(np.uint8).reshape(-1))
    assert np.array_equal(v.contiguous().view(view).cpu().numpy().reshape(-1),
                          np.ascontiguousarray(vp).view(np.uint8).reshape(-1))

    # shared blocks really are shared at decode time
    first_tables = [t[0] for t, r in zip(adm.tables, sc.requests) if r.shared >= sc.block_size]
    assert len(set(first_tables)) == 1 and pool.refcount(first_tables[0]) > 2

    tables = padded_tables(adm, -1)
    lens = np.array([len(r.tokens) for r in sc.requests], dtype=np.int32)
    ref = oracle.decode(sc.query, kp, vp, tables, lens, sc.scale, sc.dtype, sc.block_size,
                        kv_dtype=sc.kv_dtype, k_scale=sc.k_scale, v_scale=sc.v_scale)
    # the oracle over each request's logical rows gives the same answer
    for b, r in enumerate(sc.requests):
        if fp8:
            kk = oracle.fp8.dequantize_rows(_oracle_rows(r.keys, sc, "k"), sc.k_scale)
            vv = oracle.fp8.dequantize_rows(_oracle_rows(r.values, sc, "v"), sc.v_scale)
        else:
            kk, vv = oracle.to_f64(r.keys, sc.dtype), oracle.to_f64(r.values, sc.dtype)
        q = oracle.to_f64(sc.query[b], sc.dtype)
        g = sc.num_q_heads // sc.num_kv_heads
        for h in range(sc.num_kv_heads):
            want = oracle.attention_one_group(q[h * g:(h + 1) * g], kk[:, h], vv[:, h], sc.scale)
            assert np.array_equal(want, ref[b, h * g:(h + 1) * g])

    out = torch.empty((sc.num_seqs, sc.num_q_heads, sc.head_dim), dtype=TORCH_DTYPES[sc.dtype], device=DEV)
    mcl = int(lens.max())
    nbytes = pk.decode_workspace_bytes(pool, sc.num_seqs, sc.num_q_heads, mcl)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    pk.decode(pool, out, raw_to_torch(sc.query, sc.dtype).to(DEV), torch.from_numpy(tables).to(DEV),
              torch.from_numpy(lens).to(DEV), mcl, sc.scale, workspace=ws)
    torch.cuda.synchronize()
    assert_parity(out, ref, sc.dtype)
    pool.close()

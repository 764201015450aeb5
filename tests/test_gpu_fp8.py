"""8-bit (E4M3 and E5M2) KV pools on the GPU against the oracle.

The cache write quantises each activation row with the pool's per-head
inverse scales and must store exactly the oracle's codes; decode
dequantises in the kernel and must match the oracle's attention over
scale[h] * value(code) to the 16-bit tolerance.  The format and scaling
follow the reading of "大模型推理内存优化：从 KV Cache 分页到连续批处理的工程实践",
section "工程边界与架构取舍" (FP8 storage of the KV cache) described in the
oracle's fp8 module.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_145_amd as pk
import workloads
from gpu_support import DeviceCase, assert_parity, options, oracle_reference, torch_bits

pytestmark = pytest.mark.gpu

FP8_CASES = ["tiny_fp8", "embedded_1p1b_fp8", "llama70b_b64_fp8", "llama70b_b64_e5m2",
             "tiny_e5m2", "embedded_1p1b_e5m2"]


def _case(name):
    if name in workloads.FP8_CONFIGS:
        return workloads.FP8_CONFIGS[name]()
    base = {"tiny_e5m2": workloads.config_tiny_fp32, "embedded_1p1b_e5m2": workloads.config_embedded_1p1b}[name]
    return workloads.config_fp8(base, kv_format="e5m2")


@pytest.mark.parametrize("name", FP8_CASES)
def test_fp8_cache_write_bit_exact(name):
    case = _case(name)
    dc = DeviceCase(case)
    dc.write_all()
    torch.cuda.synchronize()
    kp, vp, _ = oracle.build_pools(case)
    assert np.array_equal(dc.k_cache.cpu().numpy(), kp)
    assert np.array_equal(dc.v_cache.cpu().numpy(), vp)
    dc.close()


@pytest.mark.parametrize("name", FP8_CASES)
def test_fp8_decode_parity(name):
    case = _case(name)
    dc = DeviceCase(case)
    dc.write_all()
    out = dc.decode()
    _, _, _, ref = oracle_reference(case)
    assert_parity(out, ref, case.dtype)
    dc.close()


def _act_bits(x: np.ndarray, act: str) -> np.ndarray:
    """Raw 16-bit rows of float64 values in the activation dtype (nearest-even)."""
    if act == "f16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    raw = workloads.round_f32_to_bf16_bits(np.where(np.isfinite(x), x, 0).astype(np.float32)).astype(np.uint16)
    raw[np.isnan(x)] = 0x7FC0
    raw[x == np.inf] = 0x7F80
    raw[x == -np.inf] = 0xFF80
    return raw


@pytest.mark.parametrize("kv_format", ["e4m3", "e5m2"])
def test_fp8_write_special_values(kv_format):
    """The cache write's encoder on values chosen to hit its branches: zeros
    of both signs, subnormals, every tie between neighbouring codes (to the
    even code), every code's value, values between, the largest finite
    value and values past it, both infinities, NaN; scales of 1, so the
    quantised product is the value itself."""
    from oracle import fp8

    if kv_format == "e4m3":
        mags, top, act = fp8._MAGNITUDES, 448.0, "f16"
    else:
        mags, top, act = fp8._E5M2_MAGNITUDES, 57344.0, "bf16"
    mids = (mags[:-1] + mags[1:]) / 2
    special = np.array([0.0, -0.0, top, -top, 1.1 * top, 1e30, -1e30, np.inf, -np.inf, np.nan])
    vals = np.concatenate([special, mids, -mids, mags, -mags, 1.3 * mags, 0.9 * mags])
    hkv, d = 2, 128
    per_row = hkv * d
    rows = -(-vals.size // per_row)
    x = np.zeros(rows * per_row)
    x[: vals.size] = vals
    raw = _act_bits(x, act)
    # the ties survive the activation dtype exactly (4 / 3 significant bits)
    back = raw.view(np.float16).astype(np.float64) if act == "f16" else \
        (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    n_sp = special.size
    assert np.array_equal(back[n_sp: n_sp + mids.size], mids)
    raw = raw.reshape(rows, hkv, d)
    if act == "f16":  # raw f16 rows are float16 arrays, bf16 rows their uint16 bits
        raw = raw.view(np.float16)
    base = workloads.make_paged_case("special", 145_095, act, [rows], 4, hkv, d, 16)
    base.writes = [workloads.WriteChunk(0, np.arange(rows, dtype=np.int64), raw.copy(), raw[::-1].copy())]
    case = workloads.config_fp8(lambda: base, kv_format=kv_format)
    case.k_scale = np.ones(hkv, dtype=np.float32)
    case.v_scale = np.ones(hkv, dtype=np.float32)
    dc = DeviceCase(case)
    dc.write_all()
    torch.cuda.synchronize()
    kp, vp, _ = oracle.build_pools(case)
    assert np.array_equal(dc.k_cache.cpu().numpy(), kp)
    assert np.array_equal(dc.v_cache.cpu().numpy(), vp)
    dc.close()


@pytest.mark.parametrize("kv_format", ["e4m3", "e5m2"])
def test_fp8_ragged_and_empty_sequences(kv_format):
    """Empty sequences, one token, every tail length, 64-token blocks, D 64."""
    base = workloads.make_paged_case("ragged", 145_077, "f16", [0, 1, 15, 16, 17, 33, 250, 0, 1000],
                                     8, 2, 64, 64)
    case = workloads.config_fp8(lambda: base, kv_format=kv_format)
    dc = DeviceCase(case)
    dc.write_all()
    out = dc.decode()
    _, _, _, ref = oracle_reference(case)
    assert_parity(out, ref, case.dtype)
    got = out.float().cpu().numpy()
    assert np.all(got[0] == 0) and np.all(got[7] == 0)
    dc.close()


def test_fp8_relabelling_bit_identical():
    case = workloads.FP8_CONFIGS["tiny_fp8"]()
    a = DeviceCase(case)
    a.write_all()
    out_a = a.decode().cpu()
    perm = np.random.default_rng(3).permutation(case.num_blocks).astype(np.int32)
    case_b = workloads.FP8_CONFIGS["tiny_fp8"]()
    case_b.block_tables = np.where(case_b.block_tables >= 0, perm[np.maximum(case_b.block_tables, 0)], -1)
    b = DeviceCase(case_b)
    b.write_all()
    out_b = b.decode().cpu()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    a.close()
    b.close()


def test_fp8_unsupported_combinations_are_rejected():
    case = workloads.FP8_CONFIGS["tiny_fp8"]()
    dc = DeviceCase(case)
    # a group above 16 has no 8-bit kernel
    q1 = torch.zeros((case.num_seqs, 32 * case.num_kv_heads, case.head_dim), dtype=torch.bfloat16, device="cuda")
    o1 = torch.empty_like(q1)
    with pytest.raises(pk.PaError) as e:
        pk.decode(dc.pool, o1, q1, dc.block_tables, dc.context_lens, int(case.context_lens.max()), 0.1)
    assert e.value.status == -5
    dc.close()


@pytest.mark.parametrize("kv_format", ["e4m3", "e5m2"])
@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 128), (4, 2, 64), (6, 2, 128)], ids=["G1-D128", "G2-D64", "G3-D128"])
def test_fp8_small_groups(hq, hkv, d, kv_format):
    """GQA groups below 4 (MHA included) on 8-bit pools, several tile ranges."""
    base = workloads.make_paged_case("small_group", 145_090 + hq + d, "bf16", [700, 3, 2100, 64, 0, 1300],
                                     hq, hkv, d, 16)
    case = workloads.config_fp8(lambda: base, kv_format=kv_format)
    dc = DeviceCase(case)
    dc.write_all()
    out = dc.decode()
    _, _, _, ref = oracle_reference(case)
    assert_parity(out, ref, case.dtype)
    assert np.all(out.float().cpu().numpy()[4] == 0)
    dc.close()


RING_FP8 = [("e4m3", 128, 12, 2), ("e5m2", 128, 12, 2), ("e4m3", 64, 8, 2), ("e5m2", 64, 4, 4)]


@pytest.mark.parametrize("kv_format,d,hq,hkv", RING_FP8, ids=lambda v: str(v))
@pytest.mark.parametrize("lengths", ["parity", "timing"])
def test_fp8_ring_parity(kv_format, d, hq, hkv, lengths):
    """8-bit pools in sink + ring mode: codes widened, then rotated by cache
    order (D 64 rotates across lanes, D 128 within a lane)."""
    lens = None if lengths == "parity" else workloads.ring_timing_lengths()
    case = workloads.config_sink_ring_fp8(kv_format, lens, d, hq, hkv)
    print(f"fp8 ring {kv_format} D{d} Hq{hq} Hkv{hkv} {lengths}", flush=True)
    _, _, _, ref = oracle_reference(case)
    dc = DeviceCase(case)
    dc.write_all()
    out = dc.decode()
    assert_parity(out, ref, case.dtype)
    dc.close()


@pytest.mark.parametrize("kv_format", ["e4m3", "e5m2"])
def test_fp8_ring_append_step(kv_format):
    """The one-call step on 8-bit ring pools: the staging wave quantises the
    newest token into its ring slot and the call equals write-then-decode."""
    from test_gpu_append import _check

    _check(workloads.config_sink_ring_fp8(kv_format, [1, 4, 5, 1023, 1024, 1025, 2045, 99_999]))


@pytest.mark.parametrize("cost", [2, 6])
@pytest.mark.parametrize("name", ["llama70b_b64_fp8", "llama70b_b64_e5m2"])
def test_fp8_decode_cost_weighted_ranges(name, cost):
    """8-bit pools under cost-weighted stream-K ranges: the oracle's result,
    repeated bit for bit."""
    case = _case(name)
    dc = DeviceCase(case)
    dc.write_all()
    with options(PA_DECODE_SEQ_COST=cost + 1):
        out = dc.decode()
        again = dc.decode()
    _, _, _, ref = oracle_reference(case)
    assert_parity(out, ref, case.dtype)
    assert np.array_equal(torch_bits(out, case.dtype), torch_bits(again, case.dtype))
    dc.close()


@pytest.mark.parametrize("share", [400, 900])
def test_fp8_decode_young_share_ranges(share):
    """8-bit pools run two work-groups per CU; the second one's shorter
    ranges give the oracle's result, repeated bit for bit, also on ragged
    lengths with empty sequences."""
    for case in (_case("llama70b_b64_fp8"),
                 workloads.config_fp8(lambda: workloads.make_paged_case("young", 8800, "bf16",
                                                                        [0, 1, 17, 300, 0, 5000, 2], 32, 4,
                                                                        128, 16))):
        dc = DeviceCase(case)
        dc.write_all()
        with options(PA_YOUNG_SHARE=share, PA_DECODE_SEQ_COST=4):
            out = dc.decode()
            again = dc.decode()
        _, _, _, ref = oracle_reference(case)
        assert_parity(out, ref, case.dtype)
        assert np.array_equal(torch_bits(out, case.dtype), torch_bits(again, case.dtype))
        dc.close()

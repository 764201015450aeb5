"""GPU parity of multi-token paged decode (pa_decode_multi) against the
oracle's ``decode_multi``: speculative verification (q_len 5), ragged and
short contexts, every supported GQA width and head size, stream-K cuts
(the merge kernel, through the shortest stream-K range), q_len = 1 against single-token decode, the 70B-shaped
verification batch in full, chunked prefill on sampled rows, and a
rejected-draft rollback followed by new writes.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_145_amd as pk
import workloads
from gpu_support import TORCH_DTYPES, DeviceCase, assert_parity, options, raw_to_torch, torch_to_f64

pytestmark = pytest.mark.gpu


def _run(dc, case, max_ctx=None, tables=None):
    mcl = int(case.context_lens.max()) if max_ctx is None else max_ctx
    out = torch.empty((case.num_seqs, case.q_len, case.num_q_heads, case.head_dim),
                      dtype=TORCH_DTYPES[case.dtype], device=dc.device)
    out.fill_(float("nan"))
    nbytes = pk.decode_multi_workspace_bytes(dc.pool, case.num_seqs, case.q_len, case.num_q_heads, mcl)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dc.device)
    pk.decode_multi(dc.pool, out, dc.query, dc.block_tables if tables is None else tables, dc.context_lens,
                    mcl, case.scale, workspace=ws)
    torch.cuda.synchronize()
    return out


def _ref(case, kp=None, vp=None):
    if kp is None:
        kp, vp, _ = oracle.build_pools(case)
    return oracle.decode_multi(case.query, kp, vp, case.block_tables, case.context_lens, case.scale,
                               case.dtype, case.block_size, case.q_len, kv_dtype=case.kv_dtype,
                               k_scale=case.k_scale, v_scale=case.v_scale)


def test_spec_verify_tiny():
    case = workloads.config_spec_verify_tiny()
    print(f"multi {case.name}", flush=True)
    dc = DeviceCase(case)
    dc.write_all()
    out = _run(dc, case)
    ref = _ref(case)
    assert_parity(out, ref, case.dtype)
    got = torch_to_f64(out)
    assert np.all(got[0, :2] == 0.0)  # positions before 0 attend to nothing
    dc.close()


SHAPES = [
    # dtype, lens, q_len, Hq, Hkv, D, bs
    ("bf16", [0, 1, 2, 17, 64, 65, 300], 2, 8, 2, 128, 16),
    ("f16", [4, 16, 33, 129, 700], 4, 16, 4, 128, 16),
    ("bf16", [8, 40, 511, 1025], 8, 8, 8, 64, 64),      # MHA-like G = 1: 8 rows per head
    ("f16", [33, 34, 100, 2000], 33, 12, 2, 128, 16),    # G 6: 198 rows, several passes
    ("bf16", [3, 90, 257], 3, 32, 2, 64, 16),           # G 16: 48 rows
    ("bf16", [1, 5, 9, 1000], 1, 64, 8, 128, 16),       # q_len 1
]


@pytest.mark.parametrize("min_range", [None, 1, 64])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"s{i}" for i in range(len(SHAPES))])
def test_multi_parity_shapes(shape, min_range):
    """min_range sets the shortest stream-K range: 1 cuts sequences into
    many merged pieces, 64 leaves most of them whole."""
    dtype, lens, q, hq, hkv, d, bs = shape
    print(f"multi shape {shape} min_range={min_range}", flush=True)
    case = workloads.make_multi_case("multi_shape", 7100 + len(lens) + q, dtype, lens, q, hq, hkv, d, bs)
    dc = DeviceCase(case)
    dc.write_all()
    with options(PA_MULTI_MIN_RANGE=min_range):
        out = _run(dc, case)
    assert_parity(out, _ref(case), dtype)
    dc.close()


@pytest.mark.parametrize("waves", [1, 2])
@pytest.mark.parametrize("pass_group", [1, 2, 4])
@pytest.mark.parametrize("shape", SHAPES[:5], ids=[f"s{i}" for i in range(5)])
def test_multi_parity_pass_groups(shape, pass_group, waves):
    """Several passes of one head per work-group (sharing K/V tiles through
    L2), including pass groups with fewer real passes than waves, in both
    kernel configurations (one and two waves per SIMD)."""
    dtype, lens, q, hq, hkv, d, bs = shape
    print(f"multi shape {shape} pass_group={pass_group} waves={waves}", flush=True)
    case = workloads.make_multi_case("multi_shape", 7100 + len(lens) + q, dtype, lens, q, hq, hkv, d, bs)
    dc = DeviceCase(case)
    dc.write_all()
    with options(PA_MULTI_PASS_GROUP=pass_group, PA_MULTI_MIN_RANGE=1, PA_MULTI_WAVES=waves):
        out = _run(dc, case)
    assert_parity(out, _ref(case), dtype)
    dc.close()


def test_q_len_one_matches_single_token_decode():
    case = workloads.make_multi_case("multi_q1", 7200, "bf16", [1, 50, 333, 4000], 1, 64, 8, 128, 16)
    dc = DeviceCase(case)
    dc.write_all()
    out = _run(dc, case)
    ref = _ref(case)
    assert_parity(out, ref, case.dtype)
    single = torch.empty((case.num_seqs, case.num_q_heads, case.head_dim), dtype=torch.bfloat16, device=dc.device)
    mcl = int(case.context_lens.max())
    ws = torch.empty(max(pk.decode_workspace_bytes(dc.pool, case.num_seqs, case.num_q_heads, mcl), 1),
                     dtype=torch.uint8, device=dc.device)
    pk.decode(dc.pool, single, dc.query[:, 0].contiguous(), dc.block_tables, dc.context_lens, mcl, case.scale,
              workspace=ws)
    torch.cuda.synchronize()
    assert_parity(single, ref[:, 0], case.dtype)
    dc.close()


def test_spec_verify_llama70b_full():
    case = workloads.config_spec_verify_llama70b()
    print("multi spec_verify_llama70b", flush=True)
    dc = DeviceCase(case)
    dc.write_all()
    out = _run(dc, case)
    assert_parity(out, _ref(case), case.dtype)
    dc.close()


def test_chunked_prefill_every_row():
    """All 256 rows of each sequence's chunk (4 x 256 x 64 heads) against the
    oracle, element by element."""
    case = workloads.config_chunked_prefill()
    print("multi chunked_prefill", flush=True)
    dc = DeviceCase(case)
    dc.write_all()
    out = _run(dc, case)
    assert_parity(out, _ref(case), case.dtype)
    dc.close()


def test_rejected_drafts_roll_back():
    """Verify 5 tokens, reject the last 2 (lengths drop by 2), write 2 other
    tokens at those positions and verify again: the result is the oracle's
    over the rewritten cache, with no trace of the rejected rows."""
    case = workloads.config_spec_verify_tiny()
    dc = DeviceCase(case)
    dc.write_all()
    _run(dc, case)
    rng = np.random.default_rng(9)
    new_rows = []
    for b in range(case.num_seqs):
        n = int(case.context_lens[b])
        if n < 2:
            continue
        pos = np.array([n - 2, n - 1], dtype=np.int64)
        k = workloads.draw_values(rng, (2, case.num_kv_heads, case.head_dim), case.dtype)
        v = workloads.draw_values(rng, (2, case.num_kv_heads, case.head_dim), case.dtype)
        new_rows.append(workloads.WriteChunk(b, pos, k, v))
    dc.write_all(new_rows)
    case.writes = case.writes + new_rows  # the oracle replays every write in order
    out = _run(dc, case)
    assert_parity(out, _ref(case), case.dtype)
    dc.close()


@pytest.mark.parametrize("waves", [None, 2])
@pytest.mark.parametrize("min_range", [None, 1])
@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[1], SHAPES[3], SHAPES[4]], ids=["s0", "s1", "s3", "s4"])
def test_multi_parity_fp8_pools(shape, min_range, waves):
    """8-bit (E4M3) pools: codes widened in registers, per-head scales."""
    dtype, lens, q, hq, hkv, d, bs = shape
    print(f"multi fp8 shape {shape} min_range={min_range} waves={waves}", flush=True)
    case = workloads.config_fp8(lambda: workloads.make_multi_case("multi_fp8", 7400 + len(lens) + q, dtype, lens,
                                                                  q, hq, hkv, d, bs))
    dc = DeviceCase(case)
    dc.write_all()
    with options(PA_MULTI_MIN_RANGE=min_range, PA_MULTI_WAVES=waves):
        out = _run(dc, case)
    assert_parity(out, _ref(case), dtype)
    dc.close()


@pytest.mark.parametrize("min_range", [None, 1])
@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[3], SHAPES[5]], ids=["s0", "s3", "s5"])
def test_multi_parity_e5m2_pools(shape, min_range):
    """8-bit pools in the E5M2 format: the same kernels with the other
    widening."""
    dtype, lens, q, hq, hkv, d, bs = shape
    print(f"multi e5m2 shape {shape} min_range={min_range}", flush=True)
    case = workloads.config_fp8(lambda: workloads.make_multi_case("multi_e5m2", 7450 + len(lens) + q, dtype, lens,
                                                                  q, hq, hkv, d, bs), kv_format="e5m2")
    dc = DeviceCase(case)
    dc.write_all()
    with options(PA_MULTI_MIN_RANGE=min_range):
        out = _run(dc, case)
    assert_parity(out, _ref(case), dtype)
    dc.close()


def test_spec_verify_llama70b_fp8():
    case = workloads.config_fp8(workloads.config_spec_verify_llama70b)
    print("multi spec_verify_llama70b fp8", flush=True)
    dc = DeviceCase(case)
    dc.write_all()
    out = _run(dc, case)
    assert_parity(out, _ref(case), case.dtype)
    dc.close()


def test_unsupported_pools():
    case = workloads.make_multi_case("m32", 7300, "f32", [10], 2, 4, 2, 64, 16)
    dc = DeviceCase(case)
    out = torch.empty((1, 2, case.num_q_heads, case.head_dim), dtype=TORCH_DTYPES[case.dtype], device=dc.device)
    with pytest.raises(pk.PaError) as e:
        pk.decode_multi(dc.pool, out, dc.query, dc.block_tables, dc.context_lens, 10, case.scale)
    assert e.value.status == -5
    dc.close()


def test_more_sequences_than_one_launch_slice():
    """1,300 sequences: the single-token decode schedules at most 1,024
    sequences per launch and the multi-token decode at most 1,024 (sequence,
    pass group) pairs, so both run as consecutive slices."""
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(1, 41, size=1300)]
    print("slices: 1300 sequences", flush=True)
    for q in (1, 9):
        case = workloads.make_multi_case("slices", 7500 + q, "bf16", lens, q, 16, 2, 64, 16)
        dc = DeviceCase(case)
        dc.write_all()
        out = _run(dc, case)
        assert_parity(out, _ref(case), case.dtype)
        if q == 1:
            single = torch.empty((case.num_seqs, 16, 64), dtype=torch.bfloat16, device=dc.device)
            mcl = int(case.context_lens.max())
            ws = torch.empty(max(pk.decode_workspace_bytes(dc.pool, case.num_seqs, 16, mcl), 1), dtype=torch.uint8,
                             device=dc.device)
            pk.decode(dc.pool, single, dc.query[:, 0].contiguous(), dc.block_tables, dc.context_lens, mcl,
                      case.scale, workspace=ws)
            torch.cuda.synchronize()
            kp, vp, _ = oracle.build_pools(case)
            ref = oracle.decode(case.query[:, 0], kp, vp, case.block_tables, case.context_lens, case.scale,
                                case.dtype, case.block_size)
            assert_parity(single, ref, case.dtype)
        dc.close()


@pytest.mark.parametrize("cost", [1, 4, 30])
@pytest.mark.parametrize("pass_group", [1, 4])
@pytest.mark.parametrize("shape", SHAPES[:5], ids=[f"s{i}" for i in range(5)])
def test_multi_cost_weighted_ranges(shape, pass_group, cost):
    """Stream-K ranges that weigh each (sequence, pass group) as `cost` extra
    tiles: the oracle's result, repeated bit for bit, with short ranges so
    that many pieces are merged."""
    dtype, lens, q, hq, hkv, d, bs = shape
    print(f"multi shape {shape} pass_group={pass_group} cost={cost}", flush=True)
    case = workloads.make_multi_case("multi_shape", 7100 + len(lens) + q, dtype, lens, q, hq, hkv, d, bs)
    dc = DeviceCase(case)
    dc.write_all()
    with options(PA_MULTI_SEQ_COST=cost + 1, PA_MULTI_PASS_GROUP=pass_group, PA_MULTI_MIN_RANGE=1):
        out = _run(dc, case)
        again = _run(dc, case)
    assert_parity(out, _ref(case), dtype)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    dc.close()


@pytest.mark.parametrize("share", [300, 700, 950])
@pytest.mark.parametrize("shape", SHAPES[:5], ids=[f"s{i}" for i in range(5)])
def test_multi_young_share_ranges(shape, share):
    """Two waves per SIMD (two work-groups per CU) with the second
    work-group's ranges shortened: the oracle's result, repeated bit for
    bit."""
    dtype, lens, q, hq, hkv, d, bs = shape
    print(f"multi shape {shape} young share {share}", flush=True)
    case = workloads.make_multi_case("multi_shape", 7100 + len(lens) + q, dtype, lens, q, hq, hkv, d, bs)
    dc = DeviceCase(case)
    dc.write_all()
    with options(PA_YOUNG_SHARE=share, PA_MULTI_WAVES=2, PA_MULTI_MIN_RANGE=1):
        out = _run(dc, case)
        again = _run(dc, case)
    assert_parity(out, _ref(case), dtype)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    dc.close()


@pytest.mark.parametrize("share", [500, 850])
def test_chunked_prefill_young_share(share):
    case = workloads.config_chunked_prefill()
    print(f"chunked prefill young share {share}", flush=True)
    dc = DeviceCase(case)
    dc.write_all()
    with options(PA_YOUNG_SHARE=share):
        out = _run(dc, case)
    ref = _ref(case)
    assert_parity(out, ref, case.dtype)
    dc.close()

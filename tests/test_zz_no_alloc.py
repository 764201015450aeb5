"""GPU test of pa_decode_append_noalloc, the decode step for callers that
cannot allocate: it must give the bits of pa_decode_append (with a workspace
the caller allocates) for the output and the cache, on two calls in a row
that share the library's scratch array, the second on a smaller batch, and
refuse a batch whose partials exceed the scratch size before launching
anything."""
import numpy as np
import pytest
import torch

import paged_kv_cache_145_amd as pk
import workloads
from gpu_support import TORCH_DTYPES, assert_parity, oracle_reference, raw_to_torch, torch_bits
from test_gpu_append import _append, _prepare, _same_pools

pytestmark = pytest.mark.gpu


def _noalloc(dc, case, slots, keys, vals):
    dt = case.dtype
    mcl = int(case.context_lens.max())
    out = torch.full((case.num_seqs, case.num_q_heads, case.head_dim), float("nan"), dtype=TORCH_DTYPES[dt],
                     device=dc.device)
    pk.decode_append_noalloc(dc.pool, out, dc.query, raw_to_torch(keys, dt).to(dc.device),
                             raw_to_torch(vals, dt).to(dc.device), torch.from_numpy(slots).to(dc.device),
                             dc.block_tables, dc.context_lens, mcl, case.scale, ring=dc.ring)
    torch.cuda.synchronize()
    return out


def _pair(case):
    """noalloc vs the workspace form on twin pools: equal outputs and pools,
    and within the oracle's tolerance."""
    print(f"noalloc case {case.name}: B {case.num_seqs}, max len {int(case.context_lens.max())}", flush=True)
    _, _, _, ref = oracle_reference(case)
    dc_a, _, slots, keys, vals = _prepare(case)
    dc_b, _, _, _, _ = _prepare(case)
    got = _noalloc(dc_a, case, slots, keys, vals)
    want = _append(dc_b, case, slots, keys, vals)
    assert np.array_equal(torch_bits(got, case.dtype), torch_bits(want, case.dtype))
    _same_pools(dc_a, dc_b, case.dtype)
    assert_parity(got, ref, case.dtype)
    dc_a.close()
    dc_b.close()


def test_noalloc_matches_workspace_form_on_two_calls():
    # the 70B-shaped batch (cut sequences write partials to the scratch),
    # then a smaller ragged batch that reuses the scratch left by the first
    _pair(workloads.config_llama70b())
    _pair(workloads.make_paged_case("noalloc_small", 9201, "bf16", [0, 1, 17, 300, 2049], 16, 2, 128, 16))


def test_noalloc_ring_and_fp8():
    _pair(workloads.config_sink_ring(lengths=[1, 1024, 1025, 99_999]))
    _pair(workloads.FP8_CONFIGS["llama70b_b64_fp8"]())


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    case = workloads.make_paged_case("noalloc_big", 9202, "bf16", [16] * 1000, 128, 8, 128, 16)
    dc, _, slots, keys, vals = _prepare(case)
    need = pk.decode_workspace_bytes(dc.pool, case.num_seqs, case.num_q_heads, 16, dc.ring)
    limit = pk.decode_noalloc_scratch_bytes()
    assert limit == 32 << 20
    if need <= limit:
        pytest.skip(f"workspace {need} fits the scratch on this device")
    out = torch.zeros((case.num_seqs, case.num_q_heads, case.head_dim), dtype=torch.bfloat16, device=dc.device)
    with pytest.raises(pk.PaError, match="NOMEM"):
        pk.decode_append_noalloc(dc.pool, out, dc.query, raw_to_torch(keys, "bf16").to(dc.device),
                                 raw_to_torch(vals, "bf16").to(dc.device), torch.from_numpy(slots).to(dc.device),
                                 dc.block_tables, dc.context_lens, 16, case.scale)
    dc.close()

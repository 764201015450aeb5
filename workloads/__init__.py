"""Seeded synthetic workloads for paged decode attention.

This module only draws inputs: sequence lengths, physical block placement
(block tables), query and key/value values, and the list of logical
positions that each sequence writes into the cache.  It contains none of the
method's arithmetic: no slot computation, no gather, no softmax, no RoPE.
Both the CPU oracle (``oracle/``) and the HIP path consume what it returns,
and each side computes slots, writes the cache and attends on its own.

Value storage ("raw") conventions, shared by both sides as plain data:

* ``f32``  -> numpy float32
* ``f16``  -> numpy float16
* ``bf16`` -> numpy uint16 holding the bfloat16 bit pattern (numpy has no
  bfloat16); values are drawn in float32 and rounded to nearest-even.

Every pool row that no write covers is NaN (f32 0x7FC00000, f16 0x7E00,
bf16 0x7FC0), so any read outside a sequence's context poisons the result.
Block-table entries past a sequence's last block point at a never-written
(NaN) block, or hold -1 when ``pad_with_minus_one`` is set.

Workload shapes follow the five configurations of the paged decode
problem: a tiny fp32 case, one layer of a 1.1B embedded model
(12 q heads / 2 KV heads, D 128, 16-token blocks, 680-block pool), a
LLaMA-2-70B-shaped batch (64 q / 8 KV heads, bf16, mixed lengths 50..8000),
a 32-sequence MHA batch sharing a 256-token prefix in 64-token blocks, and a
sink + ring streaming cache (4 sink + 1020 ring slots, positions to 100k).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

SEED_BASE = 145_000

RAW_DTYPES = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
FP8_NAN_CODE = 0x7F  # NaN in both 8-bit formats (E4M3 S.1111.111, E5M2 S.11111.11)
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}


KV8_DTYPES = ("fp8_e4m3", "fp8_e5m2")


def is_kv8(kv_dtype) -> bool:
    """True for the 8-bit KV storage types."""
    return kv_dtype in KV8_DTYPES


def round_f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest-even); return bits.

    For finite inputs bits + 0x8000 stays below 2**32, so uint32 suffices.
    """
    bits = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    bits += np.uint32(0x7FFF)
    bits += lsb
    bits >>= np.uint32(16)
    return bits.astype(np.uint16)


def draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) draws in float32, stored in ``dtype``'s raw form."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return round_f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def nan_array(shape, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.full(shape, NAN_BITS["f32"], dtype=np.uint32).view(np.float32)
    if dtype == "f16":
        return np.full(shape, NAN_BITS["f16"], dtype=np.uint16).view(np.float16)
    return np.full(shape, NAN_BITS["bf16"], dtype=np.uint16)


@dataclass
class RingSpec:
    sink: int
    window: int
    rope_base: float = 10000.0


@dataclass
class WriteChunk:
    """Logical positions of sequence ``seq`` and the K/V rows written there."""

    seq: int
    positions: np.ndarray  # int64 [m]
    keys: np.ndarray  # raw [m, Hkv, D]
    values: np.ndarray  # raw [m, Hkv, D]


@dataclass
class DecodeCase:
    name: str
    seed: int
    dtype: str
    num_blocks: int
    block_size: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    scale: float
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B, max_blocks]
    query: np.ndarray  # raw [B, Hq, D]
    writes: List[WriteChunk]  # everything that fills the cache, in order
    ring: Optional[RingSpec] = None
    pad_block: int = -1  # block id used for table padding (-1: none)
    notes: dict = field(default_factory=dict)
    # 8-bit KV storage: "fp8_e4m3" / "fp8_e5m2" pools hold codes, dequantised per KV head
    # by k_scale / v_scale (float32 [Hkv]); ``dtype`` is then the dtype of
    # the query, the output and the key/value rows handed to the cache write
    kv_dtype: Optional[str] = None
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    # several new tokens per sequence (speculative verification, chunked
    # prefill): query is then [B, q_len, Hq, D] and the last q_len positions
    # of each sequence are its new tokens; None for single-token decode
    q_len: Optional[int] = None
    # speculative verification over the sink + ring cache: the q_len draft
    # rows [B, q_len, Hkv, D] (raw, the query dtype) of positions
    # context_lens[b] .. context_lens[b] + q_len - 1, which are not in the
    # cache (context_lens counts the committed positions only)
    draft_keys: Optional[np.ndarray] = None
    draft_values: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    def empty_pool(self) -> np.ndarray:
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        if is_kv8(self.kv_dtype):
            return np.full(shape, FP8_NAN_CODE, dtype=np.uint8)
        return nan_array(shape, self.dtype)

    def step_writes(self) -> List[WriteChunk]:
        """The newest token of every sequence: what one decode step writes."""
        out = []
        last = {}
        for ci, ch in enumerate(self.writes):
            for j, p in enumerate(ch.positions):
                last[ch.seq] = (ci, j, int(p))
        for b in range(self.num_seqs):
            n = int(self.context_lens[b])
            if n == 0 or b not in last:
                continue
            ci, j, p = last[b]
            ch = self.writes[ci]
            out.append(
                WriteChunk(b, np.array([p], dtype=np.int64), ch.keys[j : j + 1], ch.values[j : j + 1])
            )
        return out


def _placement_tables(
    rng: np.random.Generator,
    blocks_per_seq: List[int],
    num_blocks: int,
    max_blocks: int,
    pad_with_minus_one: bool,
):
    """Assign physical ids from one seeded permutation, in sequence order."""
    perm = rng.permutation(num_blocks).astype(np.int32)
    used = int(sum(blocks_per_seq))
    if used > num_blocks:
        raise ValueError("pool too small for placement")
    spare = perm[used:]
    pad = -1 if (pad_with_minus_one or spare.size == 0) else int(spare[0])
    tables = np.full((len(blocks_per_seq), max_blocks), pad, dtype=np.int32)
    cur = 0
    for b, nb in enumerate(blocks_per_seq):
        tables[b, :nb] = perm[cur : cur + nb]
        cur += nb
    return tables, pad


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _dense_writes(rng, lens, num_kv_heads, head_dim, dtype) -> List[WriteChunk]:
    writes = []
    for b, n in enumerate(lens):
        n = int(n)
        if n == 0:
            continue
        k = draw_values(rng, (n, num_kv_heads, head_dim), dtype)
        v = draw_values(rng, (n, num_kv_heads, head_dim), dtype)
        writes.append(WriteChunk(b, np.arange(n, dtype=np.int64), k, v))
    return writes


def make_paged_case(
    name: str,
    seed: int,
    dtype: str,
    lens,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    num_blocks: Optional[int] = None,
    pool_slack: float = 1.1,
    max_blocks: Optional[int] = None,
    pad_with_minus_one: bool = False,
) -> DecodeCase:
    """A generic plain-paging case: shuffled placement, N(0,1) values."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(lens, dtype=np.int32)
    bps = [_ceil_div(int(n), block_size) for n in lens]
    need = int(sum(bps))
    if num_blocks is None:
        num_blocks = max(1, math.ceil(pool_slack * need))
    if max_blocks is None:
        max_blocks = max(1, max(bps) if bps else 1)
    tables, pad = _placement_tables(rng, bps, num_blocks, max_blocks, pad_with_minus_one)
    query = draw_values(rng, (len(lens), num_q_heads, head_dim), dtype)
    writes = _dense_writes(rng, lens, num_kv_heads, head_dim, dtype)
    return DecodeCase(
        name=name, seed=seed, dtype=dtype, num_blocks=num_blocks, block_size=block_size,
        num_kv_heads=num_kv_heads, num_q_heads=num_q_heads, head_dim=head_dim,
        scale=1.0 / math.sqrt(head_dim), context_lens=lens, block_tables=tables,
        query=query, writes=writes, pad_block=pad,
    )


# ---------------------------------------------------------------------------
# The five workload configurations
# ---------------------------------------------------------------------------

def config_tiny_fp32(pad_with_minus_one: bool = False) -> DecodeCase:
    """B 2, lengths {37, 70}, Hq 4, Hkv 2, D 64, fp32, 16-token blocks, 16-block pool."""
    seed = SEED_BASE + 1
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.array([37, 70], dtype=np.int32)
    bs, nblk = 16, 16
    tables, pad = _placement_tables(rng, [3, 5], nblk, 5, pad_with_minus_one)
    query = draw_values(rng, (2, 4, 64), "f32")
    writes = _dense_writes(rng, lens, 2, 64, "f32")
    return DecodeCase(
        name="tiny_fp32", seed=seed, dtype="f32", num_blocks=nblk, block_size=bs,
        num_kv_heads=2, num_q_heads=4, head_dim=64, scale=1.0 / 8.0,
        context_lens=lens, block_tables=tables, query=query, writes=writes, pad_block=pad,
    )


def config_embedded_1p1b(pad_with_minus_one: bool = False) -> DecodeCase:
    """One layer of the 1.1B embedded shape: Hq 12, Hkv 2, D 128, fp16, bs 16, 680 blocks, B 8.

    Lengths are uniform in [16, 2048] and redrawn (same seeded stream) until
    the batch fits the 680-block pool.
    """
    seed = SEED_BASE + 2
    rng = np.random.Generator(np.random.PCG64(seed))
    bs, nblk = 16, 680
    redraws = 0
    while True:
        lens = rng.integers(16, 2048, size=8, endpoint=True).astype(np.int32)
        bps = [_ceil_div(int(n), bs) for n in lens]
        if sum(bps) <= nblk:
            break
        redraws += 1
    tables, pad = _placement_tables(rng, bps, nblk, max(bps), pad_with_minus_one)
    query = draw_values(rng, (8, 12, 128), "f16")
    writes = _dense_writes(rng, lens, 2, 128, "f16")
    case = DecodeCase(
        name="embedded_1p1b", seed=seed, dtype="f16", num_blocks=nblk, block_size=bs,
        num_kv_heads=2, num_q_heads=12, head_dim=128, scale=1.0 / math.sqrt(128),
        context_lens=lens, block_tables=tables, query=query, writes=writes, pad_block=pad,
    )
    case.notes["length_redraws"] = redraws
    return case


def llama70b_lengths(rng: np.random.Generator, batch: int = 64) -> np.ndarray:
    """Mixed decode lengths: 50% U[50,500], 30% U[500,2000], 20% U[2000,8000].

    The mixture is taken as fixed counts (32/19/13 of 64, rounded so they sum
    to the batch), each length an inclusive integer draw, then shuffled.
    """
    n_short = int(round(0.5 * batch))
    n_mid = int(round(0.3 * batch))
    n_long = batch - n_short - n_mid
    lens = np.concatenate([
        rng.integers(50, 500, size=n_short, endpoint=True),
        rng.integers(500, 2000, size=n_mid, endpoint=True),
        rng.integers(2000, 8000, size=n_long, endpoint=True),
    ]).astype(np.int32)
    rng.shuffle(lens)
    return lens


def config_llama70b(pad_with_minus_one: bool = False, batch: int = 64) -> DecodeCase:
    """LLaMA-2-70B-shaped decode on one GPU: Hq 64, Hkv 8, D 128, bf16, bs 16, B 64."""
    seed = SEED_BASE + 3
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = llama70b_lengths(rng, batch)
    bs = 16
    bps = [_ceil_div(int(n), bs) for n in lens]
    need = int(sum(bps))
    nblk = math.ceil(1.1 * need)
    tables, pad = _placement_tables(rng, bps, nblk, max(bps), pad_with_minus_one)
    query = draw_values(rng, (batch, 64, 128), "bf16")
    writes = _dense_writes(rng, lens, 8, 128, "bf16")
    return DecodeCase(
        name="llama70b_b64", seed=seed, dtype="bf16", num_blocks=nblk, block_size=bs,
        num_kv_heads=8, num_q_heads=64, head_dim=128, scale=1.0 / math.sqrt(128),
        context_lens=lens, block_tables=tables, query=query, writes=writes, pad_block=pad,
    )


def config_shared_prefix(private_copies: bool = False, pad_with_minus_one: bool = False,
                         batch: int = 32, prefix_tokens: int = 256) -> DecodeCase:
    """MHA (Hq = Hkv = 32), D 128, fp16, bs 64; B sequences share a 256-token prefix.

    With ``private_copies`` the same logical content is laid out with a
    private copy of the prefix blocks per sequence (the twin layout); values,
    lengths and queries are identical between the two layouts.
    """
    seed = SEED_BASE + 4
    rng = np.random.Generator(np.random.PCG64(seed))
    bs, hkv, d = 64, 32, 128
    pblk = prefix_tokens // bs
    suffix = rng.integers(16, 1024, size=batch, endpoint=True).astype(np.int32)
    lens = (prefix_tokens + suffix).astype(np.int32)
    sblk = [_ceil_div(int(s), bs) for s in suffix]
    shared_need = pblk + int(sum(sblk))
    private_need = pblk * batch + int(sum(sblk))
    perm_shared = rng.permutation(math.ceil(1.1 * shared_need)).astype(np.int32)
    perm_private = rng.permutation(math.ceil(1.1 * private_need)).astype(np.int32)
    query = draw_values(rng, (batch, hkv, d), "f16")
    prefix_k = draw_values(rng, (prefix_tokens, hkv, d), "f16")
    prefix_v = draw_values(rng, (prefix_tokens, hkv, d), "f16")
    suf = []
    for b in range(batch):
        s = int(suffix[b])
        suf.append((draw_values(rng, (s, hkv, d), "f16"), draw_values(rng, (s, hkv, d), "f16")))
    max_blocks = pblk + max(sblk)
    perm = perm_private if private_copies else perm_shared
    nblk = perm.size
    used = private_need if private_copies else shared_need
    spare = perm[used:]
    pad = -1 if (pad_with_minus_one or spare.size == 0) else int(spare[0])
    tables = np.full((batch, max_blocks), pad, dtype=np.int32)
    cur = 0
    if not private_copies:
        prefix_ids = perm[:pblk]
        cur = pblk
    writes: List[WriteChunk] = []
    for b in range(batch):
        if private_copies:
            tables[b, :pblk] = perm[cur : cur + pblk]
            cur += pblk
            writes.append(WriteChunk(b, np.arange(prefix_tokens, dtype=np.int64), prefix_k, prefix_v))
        else:
            tables[b, :pblk] = prefix_ids
            if b == 0:
                writes.append(WriteChunk(0, np.arange(prefix_tokens, dtype=np.int64), prefix_k, prefix_v))
        tables[b, pblk : pblk + sblk[b]] = perm[cur : cur + sblk[b]]
        cur += sblk[b]
        k, v = suf[b]
        writes.append(WriteChunk(b, np.arange(prefix_tokens, int(lens[b]), dtype=np.int64), k, v))
    case = DecodeCase(
        name="shared_prefix_private" if private_copies else "shared_prefix",
        seed=seed, dtype="f16", num_blocks=nblk, block_size=bs, num_kv_heads=hkv,
        num_q_heads=hkv, head_dim=d, scale=1.0 / math.sqrt(d), context_lens=lens,
        block_tables=tables, query=query, writes=writes, pad_block=pad,
    )
    case.notes["prefix_blocks"] = pblk
    case.notes["shared_prefix_ids"] = None if private_copies else [int(x) for x in perm[:pblk]]
    return case


RING_PARITY_LENGTHS = [1, 3, 4, 5, 17, 1000, 1023, 1024, 1025, 1026, 2044, 2045, 4096,
                       50_000, 99_999, 100_000]


def ring_survivor_positions(n: int, sink: int, window: int) -> np.ndarray:
    """Logical positions still resident in a sink + ring cache after n appends.

    This is the cache's retention policy (the first ``sink`` positions stay,
    plus the newest ``window``), not its slot arithmetic.
    """
    if n <= sink + window:
        return np.arange(n, dtype=np.int64)
    return np.concatenate([np.arange(sink), np.arange(n - window, n)]).astype(np.int64)


def config_sink_ring(lengths=None, seed_offset: int = 5, pad_with_minus_one: bool = False,
                     sink: int = 4, window: int = 1020, block_size: int = 16,
                     num_q_heads: int = 12, num_kv_heads: int = 2, head_dim: int = 128) -> DecodeCase:
    """Sink + ring streaming cache: S 4 + W 1020 slots, bs 16, fp16, Hq 12, Hkv 2, D 128.

    The K/V of logical position p of stream b are drawn from
    ``default_rng([seed, b, p])`` so any survivor can be regenerated alone.
    Only survivors are written (with distinct slots).  ``lengths`` defaults to
    the 16 parity positions; the timing set is ``100_000 - 61 * b``.
    """
    seed = SEED_BASE + seed_offset
    if lengths is None:
        lengths = RING_PARITY_LENGTHS
    lens = np.asarray(lengths, dtype=np.int64)
    batch = lens.size
    cap = sink + window
    bps_cap = _ceil_div(cap, block_size)
    rng = np.random.Generator(np.random.PCG64(seed))
    nblk = math.ceil(1.1 * bps_cap * batch)
    tables, pad = _placement_tables(rng, [bps_cap] * batch, nblk, bps_cap, pad_with_minus_one)
    query = draw_values(rng, (batch, num_q_heads, head_dim), "f16")
    writes = []
    for b in range(batch):
        pos = ring_survivor_positions(int(lens[b]), sink, window)
        ks = np.empty((pos.size, num_kv_heads, head_dim), dtype=np.float16)
        vs = np.empty_like(ks)
        for i, p in enumerate(pos):
            r = np.random.default_rng([seed, b, int(p)])
            ks[i] = draw_values(r, (num_kv_heads, head_dim), "f16")
            vs[i] = draw_values(r, (num_kv_heads, head_dim), "f16")
        writes.append(WriteChunk(b, pos, ks, vs))
    return DecodeCase(
        name="sink_ring", seed=seed, dtype="f16", num_blocks=nblk, block_size=block_size,
        num_kv_heads=num_kv_heads, num_q_heads=num_q_heads, head_dim=head_dim,
        scale=1.0 / math.sqrt(head_dim), context_lens=lens.astype(np.int32),
        block_tables=tables, query=query, writes=writes,
        ring=RingSpec(sink, window, 10000.0), pad_block=pad,
    )


RING_VERIFY_LENGTHS = [0] + RING_PARITY_LENGTHS


def config_ring_verify(lengths=None, q_len: int = 5, seed_offset: int = 15, sink: int = 4, window: int = 1020,
                       block_size: int = 16, num_q_heads: int = 12, num_kv_heads: int = 2,
                       head_dim: int = 128, dtype: str = "f16", pad_with_minus_one: bool = False) -> DecodeCase:
    """Speculative verification over the sink + ring cache (the sink + ring
    workload's shape): each stream has committed positions 0..n-1 (only the
    survivors written), and q_len draft tokens at positions n..n+q_len-1
    whose K/V rows are inputs, not cache contents.  Committed rows and
    drafts come from ``default_rng([seed, b, p])`` for position p, so any of
    them can be regenerated alone.  The query holds the drafts' q_len query
    rows.  Default q_len 5: a step of 4 drafts plus the last accepted token."""
    seed = SEED_BASE + seed_offset
    lens = np.asarray(RING_VERIFY_LENGTHS if lengths is None else lengths, dtype=np.int64)
    batch = lens.size
    cap = sink + window
    bps_cap = _ceil_div(cap, block_size)
    rng = np.random.Generator(np.random.PCG64(seed))
    nblk = math.ceil(1.1 * bps_cap * batch)
    tables, pad = _placement_tables(rng, [bps_cap] * batch, nblk, bps_cap, pad_with_minus_one)
    query = draw_values(rng, (batch, q_len, num_q_heads, head_dim), dtype)
    writes = []
    dk = np.empty((batch, q_len, num_kv_heads, head_dim), dtype=query.dtype)
    dv = np.empty_like(dk)
    for b in range(batch):
        n = int(lens[b])
        pos = ring_survivor_positions(n, sink, window)
        ks = np.empty((pos.size, num_kv_heads, head_dim), dtype=query.dtype)
        vs = np.empty_like(ks)
        for i, p in enumerate(pos):
            r = np.random.default_rng([seed, b, int(p)])
            ks[i] = draw_values(r, (num_kv_heads, head_dim), dtype)
            vs[i] = draw_values(r, (num_kv_heads, head_dim), dtype)
        writes.append(WriteChunk(b, pos, ks, vs))
        for i in range(q_len):
            r = np.random.default_rng([seed, b, n + i])
            dk[b, i] = draw_values(r, (num_kv_heads, head_dim), dtype)
            dv[b, i] = draw_values(r, (num_kv_heads, head_dim), dtype)
    return DecodeCase(
        name="ring_verify", seed=seed, dtype=dtype, num_blocks=nblk, block_size=block_size,
        num_kv_heads=num_kv_heads, num_q_heads=num_q_heads, head_dim=head_dim,
        scale=1.0 / math.sqrt(head_dim), context_lens=lens.astype(np.int32),
        block_tables=tables, query=query, writes=writes,
        ring=RingSpec(sink, window, 10000.0), pad_block=pad, q_len=q_len,
        draft_keys=dk, draft_values=dv,
    )


def ring_timing_lengths(batch: int = 16) -> List[int]:
    return [100_000 - 61 * b for b in range(batch)]


def fp8_scales(num_kv_heads: int):
    """Per-KV-head K and V scales: N(0,1) rows reach |x| ~ 5, so
    (5 + h/4) / 448 keeps them inside the E4M3 range; distinct per head so a
    wrong head mapping shows."""
    h = np.arange(num_kv_heads, dtype=np.float64)
    k = ((5.0 + h / 4.0) / 448.0).astype(np.float32)
    v = ((4.0 + h / 3.0) / 448.0).astype(np.float32)
    return k, v


def _requantise_f32(case: DecodeCase) -> DecodeCase:
    """fp32 draws re-stored as bf16 raw rows (8-bit pools take 16-bit rows)."""
    conv = lambda a: round_f32_to_bf16_bits(np.asarray(a, dtype=np.float32))
    case.query = conv(case.query)
    for ch in case.writes:
        ch.keys, ch.values = conv(ch.keys), conv(ch.values)
    case.dtype = "bf16"
    return case


def config_fp8(base=None, kv_format: str = "e4m3", **kw) -> DecodeCase:
    """A workload with 8-bit KV storage (``kv_format`` "e4m3" or "e5m2"):
    the base configuration's lengths, placement and values, the pools
    holding scaled codes of that format."""
    if kv_format not in ("e4m3", "e5m2"):
        raise ValueError(f"unknown 8-bit format {kv_format!r}")
    case = (base or config_llama70b)(**kw)
    if case.dtype == "f32":
        case = _requantise_f32(case)
    case.kv_dtype = "fp8_" + kv_format
    case.k_scale, case.v_scale = fp8_scales(case.num_kv_heads)
    case.name = case.name + ("_fp8" if kv_format == "e4m3" else "_e5m2")
    return case


def config_tiny_fp8() -> DecodeCase:
    """The tiny case (B 2, lengths 37 / 70, Hq 8, Hkv 2) with E4M3 pools and
    bf16 activations; GQA 4 so the MFMA kernel serves it."""
    seed = SEED_BASE + 11
    case = make_paged_case("tiny", seed, "bf16", [37, 70], 8, 2, 128, 16)
    return config_fp8(lambda: case)


def config_llama70b_fp8() -> DecodeCase:
    return config_fp8(config_llama70b)


def config_embedded_1p1b_fp8() -> DecodeCase:
    return config_fp8(config_embedded_1p1b)


def config_llama70b_e5m2() -> DecodeCase:
    return config_fp8(config_llama70b, kv_format="e5m2")


def make_multi_case(name: str, seed: int, dtype: str, lens, q_len: int, num_q_heads: int,
                    num_kv_heads: int, head_dim: int, block_size: int, **kw) -> DecodeCase:
    """A plain-paging case whose sequences each end with ``q_len`` new tokens
    (already written); the query holds one row per new token."""
    case = make_paged_case(name, seed, dtype, lens, num_q_heads, num_kv_heads, head_dim, block_size, **kw)
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    case.query = draw_values(rng, (case.num_seqs, q_len, num_q_heads, head_dim), dtype)
    case.q_len = q_len
    return case


def config_spec_verify_tiny() -> DecodeCase:
    """Speculative verification, small: q_len 5 (four drafts and the last
    accepted token), B 4 with lengths 3 (shorter than q_len), 5, 37, 70;
    Hq 8, Hkv 2, D 128, bf16, 16-token blocks."""
    return make_multi_case("spec_verify_tiny", SEED_BASE + 30, "bf16", [3, 5, 37, 70], 5, 8, 2, 128, 16)


def config_spec_verify_llama70b() -> DecodeCase:
    """Speculative verification on the 70B-shaped batch: the lengths,
    placement and K/V of the single-token workload, q_len 5 per sequence."""
    case = config_llama70b()
    rng = np.random.Generator(np.random.PCG64([case.seed, 5]))
    case.query = draw_values(rng, (case.num_seqs, 5, case.num_q_heads, case.head_dim), case.dtype)
    case.q_len = 5
    case.name = "spec_verify_llama70b"
    return case


def config_chunked_prefill() -> DecodeCase:
    """Chunked prefill with 70B heads: four sequences with 0, 1000, 3000 and
    7000 earlier tokens each take a 256-token chunk (q_len 256, Hq 64,
    Hkv 8, D 128, bf16, 16-token blocks)."""
    return make_multi_case("chunked_prefill", SEED_BASE + 31, "bf16", [256, 1256, 3256, 7256], 256,
                           64, 8, 128, 16)


MULTI_CONFIGS = {
    "spec_verify_tiny": config_spec_verify_tiny,
    "spec_verify_llama70b": config_spec_verify_llama70b,
    "chunked_prefill": config_chunked_prefill,
    # resolved at call time: config_fp8 is defined further down
    "spec_verify_llama70b_fp8": lambda: config_fp8(config_spec_verify_llama70b),
    "spec_verify_llama70b_e5m2": lambda: config_fp8(config_spec_verify_llama70b, kv_format="e5m2"),
    # verification over the sink + ring cache: the edge lengths, and the
    # timing set (16 full windows at distinct ring phases near 100k)
    "ring_verify": lambda: config_ring_verify(),
    "ring_verify_timing": lambda: config_ring_verify(lengths=ring_timing_lengths()),
}


def config_sink_ring_fp8(kv_format: str = "e4m3", lengths=None, head_dim: int = 128,
                         num_q_heads: int = 12, num_kv_heads: int = 2) -> DecodeCase:
    """The sink + ring workload on 8-bit pools (f16 activations written as
    E4M3 or E5M2 codes with per-head scales)."""
    case = config_sink_ring(lengths=lengths, head_dim=head_dim, num_q_heads=num_q_heads,
                            num_kv_heads=num_kv_heads)
    case.kv_dtype = "fp8_" + kv_format
    case.k_scale, case.v_scale = fp8_scales(case.num_kv_heads)
    case.name = f"sink_ring_{kv_format}"
    return case


FP8_CONFIGS = {
    "tiny_fp8": config_tiny_fp8,
    "embedded_1p1b_fp8": config_embedded_1p1b_fp8,
    "llama70b_b64_fp8": config_llama70b_fp8,
    "llama70b_b64_e5m2": config_llama70b_e5m2,
    "sink_ring_fp8": config_sink_ring_fp8,
}


CONFIGS = {
    "tiny_fp32": config_tiny_fp32,
    "embedded_1p1b": config_embedded_1p1b,
    "llama70b_b64": config_llama70b,
    "shared_prefix": config_shared_prefix,
    "sink_ring": config_sink_ring,
}


# ---------------------------------------------------------------------------
# Prefix reuse: a resident system prompt that does not end on a block
# boundary, and requests that share all of it, part of it or none of it
# ---------------------------------------------------------------------------

@dataclass
class PrefixRequest:
    """A request's prompt ids and the K/V rows of every position.  The first
    ``shared`` ids (and rows) are the system prompt's; the rest are its own."""

    tokens: np.ndarray  # uint32 [n]
    shared: int
    keys: np.ndarray  # raw [n, Hkv, D]
    values: np.ndarray


@dataclass
class PrefixScenario:
    name: str
    seed: int
    dtype: str
    num_blocks: int
    block_size: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    scale: float
    system_tokens: np.ndarray  # uint32 [P]
    system_keys: np.ndarray  # raw [P, Hkv, D]
    system_values: np.ndarray
    requests: List[PrefixRequest]
    query: np.ndarray  # raw [B, Hq, D]
    kv_dtype: Optional[str] = None
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return len(self.requests)

    def empty_pool(self) -> np.ndarray:
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        if is_kv8(self.kv_dtype):
            return np.full(shape, FP8_NAN_CODE, dtype=np.uint8)
        return nan_array(shape, self.dtype)


def prefix_scenario(name: str, seed: int, dtype: str, system_len: int, shares, own_lens,
                    num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                    duplicate_of: Optional[int] = None, kv_fp8: bool = False) -> PrefixScenario:
    """Requests b take ``shares[b]`` leading ids of the system prompt and then
    ``own_lens[b]`` ids of their own (the first differing from the system
    prompt's next id); ``duplicate_of`` appends a copy of that request."""
    rng = np.random.Generator(np.random.PCG64(seed))
    hkv, d = num_kv_heads, head_dim
    sys_tok = rng.integers(0, 1 << 32, size=system_len, dtype=np.uint64).astype(np.uint32)
    sys_k = draw_values(rng, (system_len, hkv, d), dtype)
    sys_v = draw_values(rng, (system_len, hkv, d), dtype)
    reqs = []
    for share, own in zip(shares, own_lens):
        share, own = int(share), int(own)
        own_tok = rng.integers(0, 1 << 32, size=own, dtype=np.uint64).astype(np.uint32)
        if own and share < system_len and own_tok[0] == sys_tok[share]:
            own_tok[0] ^= np.uint32(1)
        k = np.concatenate([sys_k[:share], draw_values(rng, (own, hkv, d), dtype)])
        v = np.concatenate([sys_v[:share], draw_values(rng, (own, hkv, d), dtype)])
        reqs.append(PrefixRequest(np.concatenate([sys_tok[:share], own_tok]), share, k, v))
    if duplicate_of is not None:
        r = reqs[duplicate_of]
        reqs.append(PrefixRequest(r.tokens.copy(), r.shared, r.keys.copy(), r.values.copy()))
    query = draw_values(rng, (len(reqs), num_q_heads, d), dtype)
    need = _ceil_div(system_len, block_size) + sum(_ceil_div(len(r.tokens), block_size) + 1 for r in reqs)
    sc = PrefixScenario(
        name=name, seed=seed, dtype=dtype, num_blocks=math.ceil(1.25 * need), block_size=block_size,
        num_kv_heads=hkv, num_q_heads=num_q_heads, head_dim=d, scale=1.0 / math.sqrt(d),
        system_tokens=sys_tok, system_keys=sys_k, system_values=sys_v, requests=reqs, query=query,
    )
    if kv_fp8:
        sc.kv_dtype = "fp8_e4m3"
        sc.k_scale, sc.v_scale = fp8_scales(hkv)
    return sc


def config_prefix_unaligned(kv_fp8: bool = False) -> PrefixScenario:
    """70B attention heads (Hq 64, Hkv 8, D 128, bf16, 16-token blocks); a
    600-token system prompt (37 full blocks and a tail of 8); 12 requests:
    six extend the whole prompt, two leave it 3 ids before its end (inside
    the tail), one after 200 ids (inside a full block), one shares nothing,
    one is the prompt alone, one repeats the first request."""
    shares = [600] * 6 + [597, 597, 200, 0, 600]
    own = [1, 8, 9, 57, 250, 431, 3, 120, 77, 300, 0]
    return prefix_scenario("prefix_unaligned" + ("_fp8" if kv_fp8 else ""), SEED_BASE + 20, "bf16", 600,
                           shares, own, 64, 8, 128, 16, duplicate_of=4, kv_fp8=kv_fp8)


def config_prefix_unaligned_small() -> PrefixScenario:
    """fp32, Hq 4, Hkv 2, D 64, 64-token blocks, a 150-token system prompt
    (two full blocks and a tail of 22)."""
    shares = [150, 150, 149, 128, 10, 0, 150]
    own = [5, 42, 1, 64, 100, 7, 0]
    return prefix_scenario("prefix_unaligned_small", SEED_BASE + 21, "f32", 150, shares, own,
                           4, 2, 64, 64, duplicate_of=1)


PREFIX_CONFIGS = {
    "prefix_unaligned": config_prefix_unaligned,
    "prefix_unaligned_fp8": lambda: config_prefix_unaligned(kv_fp8=True),
    "prefix_unaligned_small": config_prefix_unaligned_small,
}


# ---------------------------------------------------------------------------
# Continuous batching: a stream of requests and the K/V rows they write
# ---------------------------------------------------------------------------

def batching_requests(seed: int, count: int, block_size: int, max_blocks: int, prompt_lo: int = 50,
                      prompt_hi: int = 500, gen_lo: int = 16, gen_hi: int = 256):
    """``count`` requests (id, prompt_len, max_tokens, arrival iteration):
    prompts U[prompt_lo, prompt_hi], generations U[gen_lo, gen_hi] (clipped to
    the table's room), arrivals spread over the first iterations."""
    rng = np.random.Generator(np.random.PCG64([seed, 40]))
    reqs = []
    room = max_blocks * block_size
    for i in range(count):
        p = int(rng.integers(prompt_lo, prompt_hi, endpoint=True))
        g = int(min(rng.integers(gen_lo, gen_hi, endpoint=True), room - p))
        reqs.append((i, p, max(1, g), int(rng.integers(0, max(1, count // 4)))))
    return reqs


def request_rows(seed: int, rid: int, positions, num_kv_heads: int, head_dim: int, dtype: str):
    """K and V rows of request ``rid`` at ``positions`` (each row drawn from
    its own (seed, request, position) stream, so any row can be redrawn)."""
    pos = list(positions)
    k = np.empty((len(pos), num_kv_heads, head_dim), dtype=RAW_DTYPES[dtype])
    v = np.empty_like(k)
    for j, p in enumerate(pos):
        r = np.random.default_rng([seed, rid, int(p)])
        k[j] = draw_values(r, (num_kv_heads, head_dim), dtype)
        v[j] = draw_values(r, (num_kv_heads, head_dim), dtype)
    return k, v


def request_query(seed: int, rid: int, iteration: int, num_q_heads: int, head_dim: int, dtype: str):
    r = np.random.default_rng([seed, rid, 1 << 30, iteration])
    return draw_values(r, (num_q_heads, head_dim), dtype)

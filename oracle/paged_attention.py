"""Oracle: gather through block tables, naive softmax attention, ring + RoPE.

TEST INFRASTRUCTURE ONLY (see the package docstring).  float64 throughout.

Sources (web pages; cited by title and section):

* "端侧 SLM 显存保活术：在 4GB 内存板卡上实现轻量 PagedAttention 与 KV 缓存分块"
  (sheratonhq.com/news/141880), section "注意力寻址：非连续物理块的间接寻址":
  a logical token index T splits into logical block T // block_size and
  offset T % block_size; the block table maps the logical block to a
  physical block, and the row sits at (physical block, offset).
* "大模型推理内存优化：从 KV Cache 分页到连续批处理的工程实践"
  (pwwt.cn/news/3010209), section "KV Cache 的内存开销与分页机制": decode
  reads every cached K/V vector of the request through its block table;
  each request has its own table; blocks may be shared.
* Page "wzjinhao.cn/news/69573" (deferred speculative decoding with a
  circular context), section "环形上下文与注意力沉淀机制", the Slot(pos)
  equation: slot = pos for pos < S, else S + ((pos - S) mod W); section
  "C++ 环形 KV 缓存管理内核实现": the resident keys are taken in cache order
  (sinks first, then the window oldest first), which here follows from the
  last position written to each slot; keys must be rotated so that RoPE
  keeps the right relative distance as the ring slides.

The pages do not define the softmax itself; decode here is the textbook
single-query attention: scores s_t = scale * <q, k_t>, weights
p = exp(s - max s) / sum exp(s - max s), output sum_t p_t v_t.
"""
from __future__ import annotations

import numpy as np

from . import fp8

# ---------------------------------------------------------------------------
# dtype handling (exact widening of stored values)
# ---------------------------------------------------------------------------


def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values to float64 exactly.  bf16 arrives as uint16 bits."""
    if dtype in ("f32", "f16"):
        return np.asarray(raw).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(raw).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# addressing
# ---------------------------------------------------------------------------


def slot_of(block_table_row: np.ndarray, logical_index: int, block_size: int) -> int:
    """Flat pool slot of a logical index: physical block * block_size + offset."""
    logical_block = logical_index // block_size
    offset = logical_index % block_size
    phys = int(block_table_row[logical_block])
    return phys * block_size + offset


def gather_rows(pool: np.ndarray, block_table_row: np.ndarray, indices, block_size: int) -> np.ndarray:
    """Rows [Hkv, D] of ``pool`` ([num_blocks, block_size, Hkv, D]) for the given
    logical (or ring-slot) indices, looked up through one block-table row."""
    indices = np.asarray(indices, dtype=np.int64)
    out = np.empty((indices.size,) + pool.shape[2:], dtype=pool.dtype)
    for i, t in enumerate(indices):
        logical_block = int(t) // block_size
        offset = int(t) % block_size
        phys = int(block_table_row[logical_block])
        if not 0 <= phys < pool.shape[0]:
            raise IndexError(f"block id {phys} outside the pool")
        out[i] = pool[phys, offset]
    return out


# ---------------------------------------------------------------------------
# ring (attention sink + rolling window)
# ---------------------------------------------------------------------------


def ring_slot(pos: int, sink: int, window: int) -> int:
    """Slot(pos) = pos if pos < S, else S + ((pos - S) mod W)."""
    if pos < 0:
        raise ValueError("negative position")
    if pos < sink:
        return int(pos)
    return int(sink + (pos - sink) % window)


def ring_writer(slot: int, n: int, sink: int, window: int) -> int:
    """Logical position whose key a ring slot holds after positions 0..n-1
    were written in order, or -1 if no position has reached the slot.

    By the Slot(pos) equation a sink slot r < S is written only by position
    r, and a window slot r >= S by the positions r, r + W, r + 2W, ...; the
    slot keeps the last of them below n.
    """
    if slot < 0 or slot >= sink + window or slot > n - 1:
        return -1
    if slot < sink:
        return int(slot)
    return int(slot + window * ((n - 1 - slot) // window))


def ring_cache_order(n: int, sink: int, window: int) -> list:
    """Ring slots of the resident keys in cache order after n appends.

    Cache order is the order of the logical positions the resident keys
    hold (so the sink keys, positions 0..S-1, come first, then the window
    from its oldest surviving position to the newest): every slot that a
    position has reached is resident, sorted by the position of its last
    writer.
    """
    resident = [r for r in range(min(n, sink + window))]
    return sorted(resident, key=lambda r: ring_writer(r, n, sink, window))


def ring_cache_index(slot: int, n: int, sink: int, window: int) -> int:
    """Inverse of ``ring_cache_order``: position in cache order of a ring slot."""
    order = ring_cache_order(n, sink, window)
    return order.index(slot)


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """theta_i = base ** (-2 i / D), i < D / 2 (float64)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def rope_rotate_half(x: np.ndarray, position, base: float) -> np.ndarray:
    """Rotate the pairs (x_i, x_{i + D/2}) by the angle position * theta_i.

    ``x`` is [..., D]; ``position`` broadcasts against x's leading axes.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    theta = rope_inv_freq(d, base)
    ang = np.asarray(position, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, lo * s + hi * c], axis=-1)


# ---------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------


def attention_one_group(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of the query rows q [G, D] over keys/values [n, D]."""
    n = keys.shape[0]
    if n == 0:
        return np.zeros((q.shape[0], values.shape[1]), dtype=np.float64)
    scores = scale * (q @ keys.T)  # [G, n]
    scores = scores - scores.max(axis=1, keepdims=True)
    weights = np.exp(scores)
    weights = weights / weights.sum(axis=1, keepdims=True)
    return weights @ values  # [G, D]


def decode(query, k_pool, v_pool, block_tables, context_lens, scale, dtype, block_size,
           ring=None, kv_dtype=None, k_scale=None, v_scale=None) -> np.ndarray:
    """Single-token decode attention over a paged KV cache (float64 output).

    query [B, Hq, D]; pools [num_blocks, block_size, Hkv, D]; block_tables
    [B, max_blocks] int; context_lens [B].  q head h reads KV head h // G with
    G = Hq / Hkv.  ``ring`` (object with sink, window, rope_base) switches to
    the sink + ring cache: the resident keys in cache order j = 0..L-1 are
    rotated by j, the query by L - 1.  ``kv_dtype`` "fp8_e4m3" / "fp8_e5m2":
    the pools hold E4M3 / E5M2 codes whose values are scaled per KV head by
    k_scale / v_scale.
    """
    q_all = to_f64(query, dtype)
    b_count, hq, d = q_all.shape
    hkv = k_pool.shape[2]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    out = np.zeros((b_count, hq, d), dtype=np.float64)
    for b in range(b_count):
        n = int(context_lens[b])
        if n == 0:
            continue
        if ring is None:
            idx = np.arange(n)
        else:
            idx = np.asarray(ring_cache_order(n, ring.sink, ring.window), dtype=np.int64)
        if kv_dtype in fp8.KV_FORMATS:
            fmt = fp8.KV_FORMATS[kv_dtype]
            keys = fp8.dequantize_rows(gather_rows(k_pool, block_tables[b], idx, block_size), k_scale, fmt)
            vals = fp8.dequantize_rows(gather_rows(v_pool, block_tables[b], idx, block_size), v_scale, fmt)
        else:
            keys = to_f64(gather_rows(k_pool, block_tables[b], idx, block_size), dtype)  # [L, Hkv, D]
            vals = to_f64(gather_rows(v_pool, block_tables[b], idx, block_size), dtype)
        q_b = q_all[b]
        if ring is not None:
            length = idx.size
            keys = rope_rotate_half(keys, np.arange(length)[:, None], ring.rope_base)
            q_b = rope_rotate_half(q_b, length - 1, ring.rope_base)
        for g in range(hkv):
            heads = slice(g * group, (g + 1) * group)
            out[b, heads] = attention_one_group(q_b[heads], keys[:, g, :], vals[:, g, :], scale)
    return out


def decode_multi(query, k_pool, v_pool, block_tables, context_lens, scale, dtype, block_size,
                 q_len, kv_dtype=None, k_scale=None, v_scale=None) -> np.ndarray:
    """Attention of ``q_len`` new tokens per sequence over the paged cache
    (float64 output [B, q_len, Hq, D]).

    Speculative verification ("推迟投机解码" of wzjinhao.cn/news/69573,
    section "嵌入式流式推理的访存墙与投机瓶颈": the target model scores a
    batch of draft tokens at once) and chunked prefill ("大模型推理内存优化…",
    pwwt.cn/news/3010209, section "工程边界与架构取舍": a long prompt is
    processed in pieces between decode steps) both attend with several new
    tokens whose K/V are already in the cache.
    Reading: ``context_lens[b]`` counts them; new token i of sequence b sits
    at position p = context_lens[b] - q_len + i and attends causally to the
    cached positions 0..p; a token with p < 0 attends to nothing and gives
    zeros.  query [B, q_len, Hq, D]; the GQA map is that of ``decode``.
    """
    q_all = to_f64(query, dtype)
    b_count, ql, hq, d = q_all.shape
    if ql != q_len:
        raise ValueError("query must be [B, q_len, Hq, D]")
    hkv = k_pool.shape[2]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    out = np.zeros((b_count, q_len, hq, d), dtype=np.float64)
    for b in range(b_count):
        n_ctx = int(context_lens[b])
        if n_ctx <= 0:
            continue
        # the sequence's keys in logical order, gathered once; token i sees a prefix
        idx = np.arange(n_ctx)
        if kv_dtype in fp8.KV_FORMATS:
            fmt = fp8.KV_FORMATS[kv_dtype]
            keys_all = fp8.dequantize_rows(gather_rows(k_pool, block_tables[b], idx, block_size), k_scale, fmt)
            vals_all = fp8.dequantize_rows(gather_rows(v_pool, block_tables[b], idx, block_size), v_scale, fmt)
        else:
            keys_all = to_f64(gather_rows(k_pool, block_tables[b], idx, block_size), dtype)
            vals_all = to_f64(gather_rows(v_pool, block_tables[b], idx, block_size), dtype)
        for i in range(q_len):
            n = n_ctx - q_len + i + 1  # keys visible to new token i
            if n <= 0:
                continue
            keys, vals = keys_all[:n], vals_all[:n]
            for g in range(hkv):
                heads = slice(g * group, (g + 1) * group)
                out[b, i, heads] = attention_one_group(q_all[b, i, heads], keys[:, g, :], vals[:, g, :], scale)
    return out


def decode_verify_ring(query, draft_keys, draft_values, k_pool, v_pool, block_tables, context_lens, scale,
                       dtype, block_size, ring, kv_dtype=None, k_scale=None, v_scale=None) -> np.ndarray:
    """Speculative verification over the sink + ring cache (float64 output
    [B, q_len, Hq, D]).

    Page "wzjinhao.cn/news/69573": the target model scores a step of draft
    tokens in one pass (section "嵌入式流式推理的访存墙与投机瓶颈") over the
    sink + ring cache of section "环形上下文与注意力沉淀机制", and the
    drafts it rejects are rolled back.  Reading: stream b has committed
    positions 0..n-1 (n = context_lens[b]) in the ring; draft i, at position
    n + i, has its query row query[b, i] and its K/V rows draft_keys[b, i],
    draft_values[b, i] (query dtype), which are not in the cache.  Row i is
    the single-token ring decode that sequential decoding would give for
    draft i: over the ring as it would be after writing drafts 0..i at their
    slots (an 8-bit pool holds their codes), with cache-order RoPE.  The
    pools themselves are not changed, so rejected drafts leave nothing to
    undo.
    """
    q_all = to_f64(query, dtype)
    b_count, q_len, hq, d = q_all.shape
    hkv = k_pool.shape[2]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    kv8 = kv_dtype in fp8.KV_FORMATS
    out = np.zeros((b_count, q_len, hq, d), dtype=np.float64)
    for b in range(b_count):
        n = int(context_lens[b])
        if kv8:  # a written draft holds its codes
            fmt = fp8.KV_FORMATS[kv_dtype]
            dk = fp8.dequantize_rows(quantize_for_cache(draft_keys[b], dtype, k_scale, kv_dtype), k_scale, fmt)
            dv = fp8.dequantize_rows(quantize_for_cache(draft_values[b], dtype, v_scale, kv_dtype), v_scale, fmt)
        else:
            dk, dv = to_f64(draft_keys[b], dtype), to_f64(draft_values[b], dtype)
        for i in range(q_len):
            total = n + i + 1  # positions written once draft i is
            order = ring_cache_order(total, ring.sink, ring.window)
            keys = np.empty((len(order), hkv, d))
            vals = np.empty((len(order), hkv, d))
            for j, r in enumerate(order):
                pos = ring_writer(r, total, ring.sink, ring.window)
                if pos >= n:  # a draft of this step
                    keys[j], vals[j] = dk[pos - n], dv[pos - n]
                    continue
                kr = gather_rows(k_pool, block_tables[b], [r], block_size)
                vr = gather_rows(v_pool, block_tables[b], [r], block_size)
                if kv8:
                    keys[j] = fp8.dequantize_rows(kr, k_scale, fp8.KV_FORMATS[kv_dtype])[0]
                    vals[j] = fp8.dequantize_rows(vr, v_scale, fp8.KV_FORMATS[kv_dtype])[0]
                else:
                    keys[j], vals[j] = to_f64(kr, dtype)[0], to_f64(vr, dtype)[0]
            length = len(order)
            keys = rope_rotate_half(keys, np.arange(length)[:, None], ring.rope_base)
            q_i = rope_rotate_half(q_all[b, i], length - 1, ring.rope_base)
            for g in range(hkv):
                heads = slice(g * group, (g + 1) * group)
                out[b, i, heads] = attention_one_group(q_i[heads], keys[:, g, :], vals[:, g, :], scale)
    return out


# ---------------------------------------------------------------------------
# write side
# ---------------------------------------------------------------------------


def reshape_and_cache_(k_pool, v_pool, keys, values, slot_mapping, block_size):
    """In place: copy token i's K/V rows [Hkv, D] to flat slot ``slot_mapping[i]``.

    Negative slots are padding and skipped; every other row keeps its bytes.
    Duplicate slots within one call are rejected (the result would depend on
    write order).
    """
    seen = set()
    capacity = k_pool.shape[0] * block_size
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        slot = int(slot)
        if slot < 0:
            continue
        if slot >= capacity:
            raise IndexError(f"slot {slot} outside the pool")
        if slot in seen:
            raise ValueError(f"duplicate slot {slot}")
        seen.add(slot)
        k_pool[slot // block_size, slot % block_size] = keys[i]
        v_pool[slot // block_size, slot % block_size] = values[i]


def reshape_and_cache(k_pool, v_pool, keys, values, slot_mapping, block_size):
    """Copying form of ``reshape_and_cache_``: returns the new pools."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    reshape_and_cache_(k_out, v_out, keys, values, slot_mapping, block_size)
    return k_out, v_out


def quantize_for_cache(rows_raw, act_dtype, scale, kv_dtype: str = "fp8_e4m3") -> np.ndarray:
    """8-bit codes (E4M3 or E5M2, by ``kv_dtype``) of raw activation rows
    [m, Hkv, D] (f16/bf16/f32 storage)."""
    return fp8.quantize_rows(to_f64(rows_raw, act_dtype).astype(np.float32), scale, fp8.KV_FORMATS[kv_dtype])


def build_pools(case):
    """Fill a NaN pool with every write of a ``workloads.DecodeCase``.

    Slots come from this module's own addressing (and ring mapping).
    Returns (k_pool, v_pool, slot_mappings) where slot_mappings lists the
    int64 slots used for each write chunk.
    """
    k_pool = case.empty_pool()
    v_pool = case.empty_pool()
    slot_lists = []
    for ch in case.writes:
        row = case.block_tables[ch.seq]
        slots = []
        for p in ch.positions:
            p = int(p)
            r = p if case.ring is None else ring_slot(p, case.ring.sink, case.ring.window)
            slots.append(slot_of(row, r, case.block_size))
        slots = np.asarray(slots, dtype=np.int64)
        keys, values = ch.keys, ch.values
        if getattr(case, "kv_dtype", None) in fp8.KV_FORMATS:
            keys = quantize_for_cache(keys, case.dtype, case.k_scale, case.kv_dtype)
            values = quantize_for_cache(values, case.dtype, case.v_scale, case.kv_dtype)
        reshape_and_cache_(k_pool, v_pool, keys, values, slots, case.block_size)
        slot_lists.append(slots)
    return k_pool, v_pool, slot_lists

"""Paged decode attention for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libpa_mi355x.so`` (declared in
``include/pa.h``).  Functions here only marshal arguments: torch tensors are
passed as raw device pointers with torch's current HIP stream; every step of
the path runs in the library's HIP kernels or its host C++ allocator.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import _lib
from ._lib import PaRing

__all__ = [
    "PaError", "Pool", "Ring", "ring_slot", "compute_slot_mapping", "reshape_and_cache",
    "decode_workspace_bytes", "rope_table_bytes", "rope_table_init", "decode", "decode_append",
    "decode_append_noalloc", "decode_noalloc_scratch_bytes",
    "check_decode_inputs", "DTYPES",
    "block_hashes", "copy_blocks", "set_option", "read_probe", "decode_multi_workspace_bytes", "decode_multi", "Batcher",
    "decode_verify_ring", "decode_verify_ring_workspace_bytes",
]

DTYPES = {"f32": _lib.PA_F32, "f16": _lib.PA_F16, "bf16": _lib.PA_BF16}
KV8_FORMATS = {"e4m3": _lib.PA_FP8_E4M3, "e5m2": _lib.PA_FP8_E5M2}


class PaError(RuntimeError):
    def __init__(self, status: int, what: str):
        lib = _lib.load()
        name = lib.pa_status_str(status).decode()
        detail = lib.pa_last_hip_error().decode() if status == _lib.PA_ERR_HIP else ""
        super().__init__(f"{what}: {name}" + (f" ({detail})" if detail else ""))
        self.status = status


def _check(status: int, what: str) -> None:
    if status != _lib.PA_OK:
        raise PaError(status, what)


def _torch_dtype_name(t) -> str:
    import torch

    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


def _stream_ptr(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name: str) -> ctypes.c_void_p:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _index_tensor(t, name: str, shape=None, min_rows=None) -> None:
    """Device-resident index data is read by the kernels as int32: refuse
    any other dtype or a shape the call does not expect."""
    import torch

    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32 (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if min_rows is not None and (t.dim() != 2 or t.shape[0] < min_rows or t.shape[1] < 1):
        raise ValueError(f"{name} must be [>= {min_rows}, max_blocks] (got {tuple(t.shape)})")


class Ring:
    """Sink + ring configuration with its device RoPE table (float32, filled
    by ``rope_table_init`` for ``capacity`` >= sink + window positions and
    head size ``head_dim``)."""

    def __init__(self, sink: int, window: int, rope_base: float, rope_table, head_dim: Optional[int] = None,
                 capacity: Optional[int] = None):
        import torch

        self.sink, self.window, self.rope_base, self.rope_table = sink, window, rope_base, rope_table
        self.capacity = int(sink + window if capacity is None else capacity)
        if rope_table is None:
            self.head_dim = int(head_dim or 0)
            return
        if not rope_table.is_cuda or not rope_table.is_contiguous() or rope_table.dtype != torch.float32:
            raise ValueError("rope_table must be a contiguous float32 device tensor")
        if head_dim is None:  # the table holds capacity rows of head_dim floats
            if self.capacity <= 0 or rope_table.numel() % self.capacity:
                raise ValueError("cannot infer head_dim from the rope table; pass head_dim")
            head_dim = rope_table.numel() // self.capacity
        self.head_dim = int(head_dim)
        need = rope_table_bytes(self.capacity, self.head_dim)
        if need == 0 or rope_table.numel() * 4 < need:
            raise ValueError(f"rope_table holds {rope_table.numel() * 4} bytes; "
                             f"{self.capacity} positions at head_dim {self.head_dim} need {need}")
        if self.capacity < sink + window:
            raise ValueError("rope table capacity is below sink + window")

    def as_struct(self) -> PaRing:
        ptr = self.rope_table.data_ptr() if self.rope_table is not None else None
        return PaRing(self.sink, self.window, self.rope_base, 0, ptr, self.capacity, self.head_dim)


def _ring_ptr(ring: Optional[Ring]):
    if ring is None:
        return None
    return ctypes.byref(ring.as_struct())


class Pool:
    """One layer's paged K/V pools (caller-owned device tensors) + allocator."""

    def __init__(self, k_cache, v_cache, block_size: int, act_dtype=None, k_scale=None, v_scale=None,
                 kv_format: str = "e4m3"):
        """``k_cache``/``v_cache`` of dtype uint8 make an 8-bit pool of codes
        in ``kv_format`` ("e4m3" or "e5m2"): ``act_dtype`` (torch.float16 /
        torch.bfloat16) is then the dtype of queries, outputs and written
        rows, and ``k_scale``/``v_scale`` hold one float per KV head."""
        import torch

        lib = _lib.load()
        if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype or k_cache.dim() != 4:
            raise ValueError("k_cache and v_cache must both be [num_blocks, block_size, Hkv, D]")
        num_blocks, bs, hkv, d = k_cache.shape
        if bs != block_size:
            raise ValueError("block_size does not match the pool shape")
        self.k_cache, self.v_cache = k_cache, v_cache
        self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim = num_blocks, bs, hkv, d
        handle = ctypes.c_void_p()
        self.kv_fp8 = k_cache.dtype == torch.uint8
        if self.kv_fp8:
            if act_dtype not in (torch.float16, torch.bfloat16) or k_scale is None or v_scale is None:
                raise ValueError("an 8-bit pool needs act_dtype (f16/bf16) and per-head k_scale, v_scale")
            self.act_dtype = act_dtype
            self.dtype = {torch.float16: "f16", torch.bfloat16: "bf16"}[act_dtype]
            ks = np.ascontiguousarray(k_scale, dtype=np.float32)
            vs = np.ascontiguousarray(v_scale, dtype=np.float32)
            if ks.shape != (hkv,) or vs.shape != (hkv,):
                raise ValueError("k_scale and v_scale need one value per KV head")
            if kv_format not in KV8_FORMATS:
                raise ValueError(f"kv_format must be one of {sorted(KV8_FORMATS)}")
            self.kv_format = kv_format
            fp = ctypes.POINTER(ctypes.c_float)
            _check(lib.pa_create_pool_kv8(ctypes.byref(handle), num_blocks, bs, hkv, d, KV8_FORMATS[kv_format],
                                          DTYPES[self.dtype], ks.ctypes.data_as(fp), vs.ctypes.data_as(fp),
                                          _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache")),
                   "pa_create_pool_kv8")
        else:
            self.kv_format = None
            self.act_dtype = k_cache.dtype
            self.dtype = _torch_dtype_name(k_cache)
            _check(lib.pa_create_pool(ctypes.byref(handle), num_blocks, bs, hkv, d, DTYPES[self.dtype],
                                      _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache")),
                   "pa_create_pool")
        self._h = handle
        self._lib = lib

    @property
    def handle(self):
        return self._h

    def close(self) -> None:
        if self._h:
            self._lib.pa_destroy_pool(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc_block(self) -> int:
        return self._lib.pa_alloc_block(self._h)

    def incref(self, block_id: int) -> None:
        _check(self._lib.pa_incref_block(self._h, block_id), "pa_incref_block")

    def decref(self, block_id: int) -> None:
        _check(self._lib.pa_decref_block(self._h, block_id), "pa_decref_block")

    def refcount(self, block_id: int) -> int:
        return self._lib.pa_get_refcount(self._h, block_id)

    def stats(self) -> dict:
        s = _lib.PaPoolStats()
        _check(self._lib.pa_get_stats(self._h, ctypes.byref(s)), "pa_get_stats")
        return {"total": s.total, "used": s.used, "shared": s.shared, "free": s.free}

    # -- prefix reuse and copy-on-write (host state only) --------------------
    def prefix_match(self, tokens, max_blocks: Optional[int] = None):
        """Longest cached prefix of ``tokens``: (block ids, tokens covered);
        each block gains a reference for the caller."""
        t = _tokens(tokens)
        cap = (t.shape[0] // self.block_size + 1) if max_blocks is None else int(max_blocks)
        out = np.empty(max(cap, 1), dtype=np.int32)
        nb, nt = ctypes.c_int32(), ctypes.c_int64()
        _check(self._lib.pa_prefix_match(self._h, t.ctypes.data_as(ctypes.c_void_p), t.shape[0],
                                         out.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(nb),
                                         ctypes.byref(nt)), "pa_prefix_match")
        return [int(x) for x in out[: nb.value]], int(nt.value)

    def prefix_insert(self, tokens, blocks, tail: bool = False, resident: bool = False) -> int:
        """List ``blocks`` (block i holds tokens [i*bs, (i+1)*bs)); returns new entries."""
        t = _tokens(tokens)
        b = np.ascontiguousarray(blocks, dtype=np.int32)
        flags = (_lib.PA_PREFIX_TAIL if tail else 0) | (_lib.PA_PREFIX_RESIDENT if resident else 0)
        made = ctypes.c_int32()
        _check(self._lib.pa_prefix_insert(self._h, t.ctypes.data_as(ctypes.c_void_p), t.shape[0],
                                          b.ctypes.data_as(ctypes.c_void_p), b.shape[0], flags,
                                          ctypes.byref(made)), "pa_prefix_insert")
        return int(made.value)

    def prefix_evict(self, max_blocks: int):
        """Free up to ``max_blocks`` index-only blocks; returns their ids in order."""
        out = np.empty(max(int(max_blocks), 1), dtype=np.int32)
        n = ctypes.c_int32()
        _check(self._lib.pa_prefix_evict(self._h, int(max_blocks), out.ctypes.data_as(ctypes.c_void_p),
                                         ctypes.byref(n)), "pa_prefix_evict")
        return [int(x) for x in out[: n.value]]

    def prefix_clear(self) -> None:
        _check(self._lib.pa_prefix_clear(self._h), "pa_prefix_clear")

    def prefix_stats(self) -> dict:
        s = _lib.PaPrefixStats()
        _check(self._lib.pa_prefix_get_stats(self._h, ctypes.byref(s)), "pa_prefix_get_stats")
        return {"entries": s.entries, "tail_entries": s.tail_entries, "resident": s.resident,
                "index_only": s.index_only}

    def cow_block(self, block_id: int):
        """(block to write, whether its old contents must be copied over)."""
        out = ctypes.c_int32()
        _check(self._lib.pa_cow_block(self._h, int(block_id), ctypes.byref(out)), "pa_cow_block")
        return int(out.value), int(out.value) != int(block_id)


def _tokens(tokens) -> np.ndarray:
    t = np.asarray(tokens)
    if t.size and (t.min() < 0 or t.max() > 0xFFFFFFFF):
        raise ValueError("token ids must fit in uint32")
    return np.ascontiguousarray(t, dtype=np.uint32).reshape(-1)


def block_hashes(tokens, block_size: int) -> list:
    """Chained 64-bit keys of the full blocks of ``tokens``."""
    t = _tokens(tokens)
    out = np.zeros(max(t.shape[0] // max(int(block_size), 1), 1), dtype=np.uint64)
    _check(_lib.load().pa_block_hashes(t.ctypes.data_as(ctypes.c_void_p), t.shape[0], int(block_size),
                                       out.ctypes.data_as(ctypes.c_void_p)), "pa_block_hashes")
    return [int(x) for x in out[: t.shape[0] // int(block_size)]]


def copy_blocks(pool: Pool, src_blocks, dst_blocks, stream=None) -> None:
    """Device: block dst[i] of both pools takes block src[i]'s contents
    (device int32 tensors of equal length; negative ids are padding)."""
    n = int(src_blocks.shape[0])
    if tuple(dst_blocks.shape) != (n,):
        raise ValueError("src_blocks and dst_blocks must have the same length")
    if n == 0:
        return
    import torch

    if src_blocks.dtype != torch.int32 or dst_blocks.dtype != torch.int32:
        raise ValueError("block ids must be int32")
    _check(_lib.load().pa_copy_blocks(pool.handle, _dev_ptr(src_blocks, "src_blocks"),
                                      _dev_ptr(dst_blocks, "dst_blocks"), n, _stream_ptr(stream)),
           "pa_copy_blocks")


def set_option(name: str, value: int) -> int:
    """Set a kernel-configuration override (``PA_FORCE_VALU``, ...; 0 = the
    library's choice); returns the previous value.  For tests and
    measurements."""
    lib = _lib.load()
    opt = _lib.PA_OPTIONS[name]
    old = int(lib.pa_get_option(opt))
    _check(lib.pa_set_option(opt, int(value)), "pa_set_option")
    return old


READ_PROBE_CHECKSUMS = 4096


def read_probe(src, checksums, stream=None) -> None:
    """Streaming-read probe over the bytes of device tensor ``src``
    (measurement aid); ``checksums`` is a device int32/uint32 tensor of
    4096 entries receiving per-work-group XOR checksums."""
    nbytes = src.numel() * src.element_size()
    if checksums.numel() * checksums.element_size() < 4 * READ_PROBE_CHECKSUMS:
        raise ValueError("checksums must hold 4096 32-bit words")
    _check(_lib.load().pa_read_probe(_dev_ptr(src, "src"), nbytes, _dev_ptr(checksums, "checksums"),
                                     _stream_ptr(stream)), "pa_read_probe")


def ring_slot(pos: int, sink: int, window: int) -> int:
    return _lib.load().pa_ring_slot(pos, sink, window)


def compute_slot_mapping(pool: Pool, block_tables: np.ndarray, seq_ids, positions,
                         ring: Optional[Ring] = None) -> np.ndarray:
    """Host slot computation (int32 [n]) through the host copy of the tables."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sid = np.ascontiguousarray(seq_ids, dtype=np.int32)
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    out = np.empty(sid.shape[0], dtype=np.int32)
    _check(_lib.load().pa_compute_slot_mapping(
        pool.handle, bt.ctypes.data_as(ctypes.c_void_p), bt.shape[0], bt.shape[1],
        sid.ctypes.data_as(ctypes.c_void_p), pos.ctypes.data_as(ctypes.c_void_p), sid.shape[0],
        _ring_ptr(ring), out.ctypes.data_as(ctypes.c_void_p)), "pa_compute_slot_mapping")
    return out


def reshape_and_cache(pool: Pool, key, value, slot_mapping, stream=None) -> None:
    """Device scatter of key/value [N, Hkv, D] into the pool at slot_mapping [N] (int32)."""
    n = int(slot_mapping.shape[0])
    if n == 0:
        return
    if key.dtype != pool.act_dtype or value.dtype != pool.act_dtype:
        raise ValueError("key/value dtype must match the pool")
    if tuple(key.shape) != (n, pool.num_kv_heads, pool.head_dim) or key.shape != value.shape:
        raise ValueError("key/value must be [N, Hkv, D]")
    _index_tensor(slot_mapping, "slot_mapping", shape=(n,))
    _check(_lib.load().pa_reshape_and_cache(
        pool.handle, _dev_ptr(key, "key"), _dev_ptr(value, "value"),
        _dev_ptr(slot_mapping, "slot_mapping"), n, _stream_ptr(stream)), "pa_reshape_and_cache")


def decode_workspace_bytes(pool: Pool, num_seqs: int, num_q_heads: int, max_context_len: int,
                           ring: Optional[Ring] = None) -> int:
    return int(_lib.load().pa_decode_workspace_bytes(pool.handle, num_seqs, num_q_heads,
                                                     max_context_len, _ring_ptr(ring)))


def rope_table_bytes(capacity: int, head_dim: int) -> int:
    return int(_lib.load().pa_rope_table_bytes(capacity, head_dim))


def rope_table_init(table, capacity: int, head_dim: int, rope_base: float, stream=None) -> None:
    if table.numel() * table.element_size() < rope_table_bytes(capacity, head_dim):
        raise ValueError("rope table buffer too small")
    _check(_lib.load().pa_rope_table_init(_dev_ptr(table, "rope_table"), capacity, head_dim,
                                          rope_base, _stream_ptr(stream)), "pa_rope_table_init")


def _check_tables(pool: Pool, block_tables, context_lens, num_seqs: int, ring: Optional[Ring]) -> None:
    _index_tensor(context_lens, "context_lens", shape=(num_seqs,))
    _index_tensor(block_tables, "block_tables", min_rows=num_seqs)
    if ring is not None and ring.rope_table is not None and ring.head_dim != pool.head_dim:
        raise ValueError(f"the ring's rope table is for head_dim {ring.head_dim}, the pool's is {pool.head_dim}")


def decode(pool: Pool, out, query, block_tables, context_lens, max_context_len: int,
           scale: float, ring: Optional[Ring] = None, workspace=None, stream=None) -> None:
    """Paged decode attention into ``out`` [B, Hq, D] (device tensors, async)."""
    b, hq, d = query.shape
    if tuple(out.shape) != (b, hq, d) or d != pool.head_dim:
        raise ValueError("out/query must be [B, Hq, D] with D = the pool's head size")
    if query.dtype != pool.act_dtype or out.dtype != pool.act_dtype:
        raise ValueError("query/out dtype must match the pool")
    _check_tables(pool, block_tables, context_lens, b, ring)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev_ptr(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().pa_decode(
        pool.handle, _dev_ptr(out, "out"), _dev_ptr(query, "query"),
        _dev_ptr(block_tables, "block_tables"), int(block_tables.shape[1]),
        _dev_ptr(context_lens, "context_lens"), b, hq, int(max_context_len), float(scale),
        _ring_ptr(ring), ws_ptr, ws_bytes, _stream_ptr(stream)), "pa_decode")


def _check_append(pool: Pool, out, query, key, value, slot_mapping, block_tables, context_lens,
                  ring: Optional[Ring]) -> int:
    b, hq, d = query.shape
    if tuple(out.shape) != (b, hq, d) or d != pool.head_dim:
        raise ValueError("out/query must be [B, Hq, D] with D = the pool's head size")
    if query.dtype != pool.act_dtype or out.dtype != pool.act_dtype:
        raise ValueError("query/out dtype must match the pool")
    if key.dtype != pool.act_dtype or value.dtype != pool.act_dtype:
        raise ValueError("key/value dtype must match the pool")
    if tuple(key.shape) != (b, pool.num_kv_heads, d) or key.shape != value.shape:
        raise ValueError("key/value must be [B, Hkv, D]")
    _index_tensor(slot_mapping, "slot_mapping", shape=(b,))
    _check_tables(pool, block_tables, context_lens, b, ring)
    return b


def decode_append(pool: Pool, out, query, key, value, slot_mapping, block_tables, context_lens,
                  max_context_len: int, scale: float, ring: Optional[Ring] = None, workspace=None,
                  stream=None) -> None:
    """One decode step that also stores each sequence's new token: key/value
    [B, Hkv, D] go to slot_mapping [B] (the slot of position
    context_lens[b] - 1) and ``out`` [B, Hq, D] is the decode attention over
    the cache including them."""
    b = _check_append(pool, out, query, key, value, slot_mapping, block_tables, context_lens, ring)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev_ptr(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().pa_decode_append(
        pool.handle, _dev_ptr(out, "out"), _dev_ptr(query, "query"), _dev_ptr(key, "key"),
        _dev_ptr(value, "value"), _dev_ptr(slot_mapping, "slot_mapping"),
        _dev_ptr(block_tables, "block_tables"), int(block_tables.shape[1]),
        _dev_ptr(context_lens, "context_lens"), b, query.shape[1], int(max_context_len), float(scale),
        _ring_ptr(ring), ws_ptr, ws_bytes, _stream_ptr(stream)), "pa_decode_append")


def decode_append_noalloc(pool: Pool, out, query, key, value, slot_mapping, block_tables, context_lens,
                          max_context_len: int, scale: float, ring: Optional[Ring] = None, stream=None) -> None:
    """``decode_append`` without a workspace: the library's per-GPU scratch
    array holds the split-K partials (see pa_decode_append_noalloc)."""
    b = _check_append(pool, out, query, key, value, slot_mapping, block_tables, context_lens, ring)
    _check(_lib.load().pa_decode_append_noalloc(
        pool.handle, _dev_ptr(out, "out"), _dev_ptr(query, "query"), _dev_ptr(key, "key"),
        _dev_ptr(value, "value"), _dev_ptr(slot_mapping, "slot_mapping"),
        _dev_ptr(block_tables, "block_tables"), int(block_tables.shape[1]),
        _dev_ptr(context_lens, "context_lens"), b, query.shape[1], int(max_context_len), float(scale),
        _ring_ptr(ring), _stream_ptr(stream)), "pa_decode_append_noalloc")


def decode_noalloc_scratch_bytes() -> int:
    return int(_lib.load().pa_decode_noalloc_scratch_bytes())


def check_decode_inputs(pool: Pool, block_tables, context_lens, max_context_len: int,
                        ring: Optional[Ring] = None, slot_mapping=None, counts=None, stream=None):
    """Debug counts (device int32 [4]) of out-of-range lengths, block ids a
    decode reads, and slots; see pa_check_decode_inputs.  Asynchronous."""
    import torch

    if counts is None:
        counts = torch.empty(4, dtype=torch.int32, device=block_tables.device)
    n_slots = 0 if slot_mapping is None else int(slot_mapping.shape[0])
    _check(_lib.load().pa_check_decode_inputs(
        pool.handle, _dev_ptr(block_tables, "block_tables"), int(block_tables.shape[1]),
        _dev_ptr(context_lens, "context_lens"), int(context_lens.shape[0]), int(max_context_len),
        _ring_ptr(ring), None if slot_mapping is None else _dev_ptr(slot_mapping, "slot_mapping"), n_slots,
        _dev_ptr(counts, "counts"), _stream_ptr(stream)), "pa_check_decode_inputs")
    return counts


def decode_multi_workspace_bytes(pool: Pool, num_seqs: int, q_len: int, num_q_heads: int,
                                 max_context_len: int) -> int:
    return int(_lib.load().pa_decode_multi_workspace_bytes(pool.handle, num_seqs, q_len, num_q_heads,
                                                           max_context_len))


def decode_multi(pool: Pool, out, query, block_tables, context_lens, max_context_len: int,
                 scale: float, workspace=None, stream=None) -> None:
    """Causal attention of q_len new tokens per sequence: ``query``/``out``
    [B, q_len, Hq, D] (device tensors, async)."""
    b, ql, hq, d = query.shape
    if tuple(out.shape) != (b, ql, hq, d) or d != pool.head_dim:
        raise ValueError("out/query must be [B, q_len, Hq, D] with D = the pool's head size")
    if query.dtype != pool.act_dtype or out.dtype != pool.act_dtype:
        raise ValueError("query/out dtype must match the pool")
    _check_tables(pool, block_tables, context_lens, b, None)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev_ptr(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().pa_decode_multi(
        pool.handle, _dev_ptr(out, "out"), _dev_ptr(query, "query"),
        _dev_ptr(block_tables, "block_tables"), int(block_tables.shape[1]),
        _dev_ptr(context_lens, "context_lens"), b, ql, hq, int(max_context_len), float(scale),
        ws_ptr, ws_bytes, _stream_ptr(stream)), "pa_decode_multi")


def decode_verify_ring_workspace_bytes(pool: Pool, num_seqs: int, q_len: int, num_q_heads: int) -> int:
    return int(_lib.load().pa_decode_verify_ring_workspace_bytes(pool.handle, num_seqs, q_len, num_q_heads))


def decode_verify_ring(pool: Pool, out, query, draft_key, draft_value, block_tables, context_lens,
                       max_context_len: int, scale: float, ring: Ring, workspace=None, stream=None) -> None:
    """Speculative verification over the sink + ring cache: ``query``/``out``
    [B, q_len, Hq, D], the drafts' K/V rows ``draft_key``/``draft_value``
    [B, q_len, Hkv, D]; context_lens [B] counts committed positions only.
    The cache is only read (device tensors, async)."""
    b, ql, hq, d = query.shape
    if tuple(out.shape) != (b, ql, hq, d) or d != pool.head_dim:
        raise ValueError("out/query must be [B, q_len, Hq, D] with D = the pool's head size")
    if query.dtype != pool.act_dtype or out.dtype != pool.act_dtype:
        raise ValueError("query/out dtype must match the pool")
    if tuple(draft_key.shape) != (b, ql, pool.num_kv_heads, d) or draft_key.shape != draft_value.shape:
        raise ValueError("draft_key/draft_value must be [B, q_len, Hkv, D]")
    if draft_key.dtype != pool.act_dtype or draft_value.dtype != pool.act_dtype:
        raise ValueError("draft_key/draft_value dtype must match the pool")
    if ring is None:
        raise ValueError("ring verification needs the ring")
    _check_tables(pool, block_tables, context_lens, b, ring)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev_ptr(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.load().pa_decode_verify_ring(
        pool.handle, _dev_ptr(out, "out"), _dev_ptr(query, "query"), _dev_ptr(draft_key, "draft_key"),
        _dev_ptr(draft_value, "draft_value"), _dev_ptr(block_tables, "block_tables"), int(block_tables.shape[1]),
        _dev_ptr(context_lens, "context_lens"), b, ql, hq, int(max_context_len), float(scale), _ring_ptr(ring),
        ws_ptr, ws_bytes, _stream_ptr(stream)), "pa_decode_verify_ring")


class Batcher:
    """Continuous-batching driver over a pool (host state in the library)."""

    def __init__(self, pool: Pool, max_batch: int, max_blocks_per_seq: int):
        self._lib = _lib.load()
        self.pool = pool  # keeps the pool alive while the driver holds its blocks
        self.max_batch, self.max_blocks_per_seq = int(max_batch), int(max_blocks_per_seq)
        h = ctypes.c_void_p()
        _check(self._lib.pa_batcher_create(pool.handle, self.max_batch, self.max_blocks_per_seq,
                                           ctypes.byref(h)), "pa_batcher_create")
        self._h = h
        n, mb = self.max_batch, self.max_blocks_per_seq
        self._ids = np.empty(n, dtype=np.uint64)
        self._tables = np.empty((n, mb), dtype=np.int32)
        self._ctx = np.empty(n, dtype=np.int32)
        self._ws = np.empty(n, dtype=np.int32)
        self._wc = np.empty(n, dtype=np.int32)
        self._pre = np.empty(n, dtype=np.int32)

    def close(self) -> None:
        if self._h:
            self._lib.pa_batcher_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, request_id: int, prompt_len: int, max_tokens: int) -> None:
        _check(self._lib.pa_batcher_add(self._h, int(request_id), int(prompt_len), int(max_tokens)),
               "pa_batcher_add")

    def schedule(self):
        """One iteration's batch: dict of arrays (ids, tables, context_lens,
        write_start, write_count, prefill) and the info counters."""
        info = _lib.PaBatchInfo()
        p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
        _check(self._lib.pa_batcher_schedule(self._h, p(self._ids), p(self._tables), p(self._ctx), p(self._ws),
                                             p(self._wc), p(self._pre), ctypes.byref(info)), "pa_batcher_schedule")
        n = info.scheduled
        batch = {"ids": self._ids[:n].copy(), "tables": self._tables[:n].copy(),
                 "context_lens": self._ctx[:n].copy(), "write_start": self._ws[:n].copy(),
                 "write_count": self._wc[:n].copy(), "prefill": self._pre[:n].astype(bool)}
        return batch, {f: getattr(info, f) for f, _ in _lib.PaBatchInfo._fields_}

    def step(self, request_id: int) -> None:
        _check(self._lib.pa_batcher_step(self._h, int(request_id)), "pa_batcher_step")

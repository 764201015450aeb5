"""Admission of a prefix-sharing workload through a prefix-cache API.

The same caller logic drives the oracle's ``PrefixCacheModel`` and the
library's C ABI: warm up the system prompt (write it once, list every block
of it as resident, tail included, and drop the warm-up's own references),
then admit each request: match its prompt, copy-on-write a partially
covered last block, allocate the rest, and list its full blocks.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

from oracle.allocator import BlockAllocatorModel
from oracle.prefix import PrefixCacheModel


@dataclass
class Admission:
    system_blocks: List[int]
    tables: List[List[int]]  # per request, logical order
    covered: List[int]  # ids each request found cached
    copies: List[Tuple[int, int]]  # (source, destination) block copies, in order


class ModelApi:
    def __init__(self, num_blocks, block_size):
        self.m = PrefixCacheModel(BlockAllocatorModel(num_blocks), block_size)

    def alloc(self):
        return self.m.alloc.alloc()

    def release(self, b):
        self.m.release(b)

    def match(self, tokens):
        return self.m.match([int(t) for t in tokens], 1 << 20)

    def cow(self, b):
        return self.m.cow(b)

    def insert(self, tokens, blocks, tail=False, resident=False):
        return self.m.insert([int(t) for t in tokens], blocks, tail=tail, resident=resident)

    def refcount(self, b):
        return self.m.alloc.refcount[b]


class LibApi:
    """The C ABI on an existing pool handle (host calls only)."""

    def __init__(self, lib, handle, block_size):
        self.lib, self.h, self.bs = lib, handle, block_size

    def _ok(self, st, what):
        if st != 0:
            raise RuntimeError(f"{what} returned {st}")

    def alloc(self):
        return self.lib.pa_alloc_block(self.h)

    def release(self, b):
        self._ok(self.lib.pa_decref_block(self.h, b), "pa_decref_block")

    def match(self, tokens):
        t = np.ascontiguousarray(tokens, dtype=np.uint32)
        cap = t.shape[0] // self.bs + 1
        out = np.empty(cap, dtype=np.int32)
        nb, nt = ctypes.c_int32(), ctypes.c_int64()
        self._ok(self.lib.pa_prefix_match(self.h, t.ctypes.data_as(ctypes.c_void_p), t.shape[0],
                                          out.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(nb),
                                          ctypes.byref(nt)), "pa_prefix_match")
        return [int(x) for x in out[: nb.value]], int(nt.value)

    def cow(self, b):
        out = ctypes.c_int32()
        st = self.lib.pa_cow_block(self.h, b, ctypes.byref(out))
        if st == -2:
            return -1, False
        self._ok(st, "pa_cow_block")
        return int(out.value), int(out.value) != b

    def insert(self, tokens, blocks, tail=False, resident=False):
        t = np.ascontiguousarray(tokens, dtype=np.uint32)
        b = np.ascontiguousarray(blocks, dtype=np.int32)
        made = ctypes.c_int32()
        self._ok(self.lib.pa_prefix_insert(self.h, t.ctypes.data_as(ctypes.c_void_p), t.shape[0],
                                           b.ctypes.data_as(ctypes.c_void_p), b.shape[0],
                                           (1 if tail else 0) | (2 if resident else 0),
                                           ctypes.byref(made)), "pa_prefix_insert")
        return int(made.value)

    def refcount(self, b):
        return self.lib.pa_get_refcount(self.h, b)


def admit(api, sc) -> Admission:
    bs = sc.block_size
    p = len(sc.system_tokens)
    sys_blocks = [api.alloc() for _ in range(math.ceil(p / bs))]
    assert min(sys_blocks, default=0) >= 0
    api.insert(sc.system_tokens, sys_blocks, tail=True, resident=True)
    for b in sys_blocks:
        api.release(b)
    tables, covered, copies = [], [], []
    for r in sc.requests:
        n = len(r.tokens)
        blocks, cov = api.match(r.tokens)
        if cov % bs and cov < n:  # the request writes into a shared partial block
            new, copied = api.cow(blocks[-1])
            assert new >= 0, "pool too small"
            if copied:
                copies.append((blocks[-1], new))
            blocks[-1] = new
        while len(blocks) * bs < n:
            b = api.alloc()
            assert b >= 0, "pool too small"
            blocks.append(b)
        api.insert(r.tokens, blocks)
        tables.append(blocks)
        covered.append(cov)
    return Admission(sys_blocks, tables, covered, copies)


def padded_tables(adm: Admission, pad: int) -> np.ndarray:
    width = max(1, max(len(t) for t in adm.tables))
    out = np.full((len(adm.tables), width), pad, dtype=np.int32)
    for i, t in enumerate(adm.tables):
        out[i, : len(t)] = t
    return out

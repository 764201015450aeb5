"""Reference model of prefix-aware block reuse with copy-on-write.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Ollama的内存管理策略：从KV Cache Block分配到Prefix-aware内存复用的演进"
(xdnf.cn/news/5086), sections "三、KV Cache内存管理的工程实现" and
"四、内存管理策略的边界", and the shared resident prefix of
"端侧 SLM 显存保活术…" (sheratonhq.com/news/141880), section "共享前缀块".
What the pages fix:

* blocks are found by a 64-bit FNV-1a style hash of the token ids a block
  covers (token ids, not K/V values), one token id folded per step:
  h ^= id; h *= 0x100000001b3 (mod 2^64), starting from 0xcbf29ce484222325;
* a hash hit must be confirmed on the token ids themselves (collisions);
* a reused block gains a reference; the last release frees it;
* a block with more than one reference is read-only: a writer copies it to a
  private block first (copy-on-write);
* eviction reclaims blocks nobody else uses, least recently used first;
  a warmed-up prefix (a system prompt) stays resident.

Readings where the pages' code leaves a step open or gets it wrong:

* chaining: block i is keyed by the fold continued from block i-1's hash
  (the first block starts from the offset basis), so its key covers every
  token up to its end; the pages' hash restarts at each block;
* verification compares the block's token ids and requires the entry to hang
  off the entry matched for the previous block, so a collision can never
  join two different prefixes;
* the index holds one reference on each block it lists, so a block stays
  allocated after every sequence using it is released, and a block held by
  the index alone is what eviction may free; resident entries are never
  evicted; only leaf entries (no entry hangs off them) are evicted, least
  recent use first, ties broken by creation order; every match and insert
  call is one tick of the use clock and stamps the entries it walks;
* full blocks are keyed by hash; a partial last block ("tail", fewer tokens
  than a block) is listed under its parent entry and matches when its token
  ids are a prefix of the remaining request tokens, longest first;
* copy-on-write of a block with one reference returns the block itself; with
  more, a fresh block (lowest free id) replaces it, the old block loses the
  writer's reference, and the writer copies the old contents over.

Parity status: ``fnv1a_fold``/``chained_block_hashes`` pinned by published
FNV-1a test vectors (token ids = byte values), by the chaining identity
(chained key of block i = one-shot fold of the whole prefix) and by the
multiplier's 2^40 + 0x1b3 split; ``PrefixCacheModel`` pinned by scenarios
worked by hand from the rules above and by invariants (reference counts
equal holders, no block freed while listed); ``copy_blocks`` pinned by
write-then-copy round trips.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .allocator import AllocatorError, BlockAllocatorModel

FNV_OFFSET_BASIS = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
_MASK64 = (1 << 64) - 1
ROOT = -1  # parent of the first block of every prefix


def fnv1a_fold(h: int, tokens: Sequence[int]) -> int:
    """Continue a 64-bit FNV-1a fold from ``h`` over 32-bit token ids."""
    for t in tokens:
        h ^= int(t) & 0xFFFFFFFF
        h = (h * FNV_PRIME) & _MASK64
    return h


def chained_block_hashes(tokens: Sequence[int], block_size: int) -> List[int]:
    """Key of every full block: the fold continued from the previous key."""
    h = FNV_OFFSET_BASIS
    out = []
    for i in range(len(tokens) // block_size):
        h = fnv1a_fold(h, tokens[i * block_size:(i + 1) * block_size])
        out.append(h)
    return out


@dataclass
class _Entry:
    serial: int
    block: int
    parent: int  # serial of the parent entry, ROOT for the first block
    tokens: Tuple[int, ...]
    key: Optional[int]  # chained hash (full blocks); None for a tail
    resident: bool = False
    last_use: int = 0
    children: int = 0


@dataclass
class PrefixCacheModel:
    """Prefix index over a ``BlockAllocatorModel`` (the same block ids)."""

    alloc: BlockAllocatorModel
    block_size: int
    entries: Dict[int, _Entry] = field(default_factory=dict)
    clock: int = 0
    next_serial: int = 0

    # -- lookups -----------------------------------------------------------
    def _full_child(self, parent: int, key: int, toks: Tuple[int, ...]) -> Optional[_Entry]:
        for e in self.entries.values():
            if e.key is not None and e.parent == parent and e.key == key and e.tokens == toks:
                return e
        return None

    def _tail_child(self, parent: int, toks: Tuple[int, ...]) -> Optional[_Entry]:
        for e in self.entries.values():
            if e.key is None and e.parent == parent and e.tokens == toks:
                return e
        return None

    def indexed_blocks(self) -> set:
        return {e.block for e in self.entries.values()}

    # -- match ---------------------------------------------------------------
    def match(self, tokens: Sequence[int], max_blocks: int) -> Tuple[List[int], int]:
        """Longest verified cached prefix of ``tokens``: its blocks (each
        gains a reference for the caller) and the number of tokens covered."""
        self.clock += 1
        toks = [int(t) & 0xFFFFFFFF for t in tokens]
        bs, n = self.block_size, len(toks)
        parent, h, p, blocks = ROOT, FNV_OFFSET_BASIS, 0, []
        while len(blocks) < max_blocks and n - p >= bs:
            piece = tuple(toks[p:p + bs])
            key = fnv1a_fold(h, piece)
            e = self._full_child(parent, key, piece)
            if e is None:
                break
            blocks.append(e.block)
            e.last_use = self.clock
            parent, h, p = e.serial, key, p + bs
        if len(blocks) < max_blocks:
            best = None
            for e in self.entries.values():
                if e.key is None and e.parent == parent:
                    m = len(e.tokens)
                    if m <= n - p and tuple(toks[p:p + m]) == e.tokens:
                        if best is None or m > len(best.tokens):
                            best = e
            if best is not None:
                blocks.append(best.block)
                best.last_use = self.clock
                p += len(best.tokens)
        for b in blocks:
            self.alloc.incref(b)
        return blocks, p

    # -- insert ----------------------------------------------------------------
    def insert(self, tokens: Sequence[int], blocks: Sequence[int], tail: bool = False,
               resident: bool = False) -> int:
        """List a sequence's blocks (block i holds tokens [i*bs, (i+1)*bs)).

        Full blocks always; the partial last block too when ``tail``.  Blocks
        whose (parent, tokens) are listed already are skipped.  Returns the
        number of new entries; raises ``AllocatorError`` and changes nothing
        when a new entry's block is free, listed already or used twice."""
        toks = [int(t) & 0xFFFFFFFF for t in tokens]
        bs, n = self.block_size, len(toks)
        nfull = n // bs
        has_tail = bool(tail) and n % bs != 0
        if len(blocks) < nfull + (1 if has_tail else 0):
            raise AllocatorError("inval", "fewer blocks than the tokens need")
        plan = []  # (existing entry) or (block, key, tokens) for a new one
        parent, h, new_from = ROOT, FNV_OFFSET_BASIS, None
        listed = self.indexed_blocks()
        for i in range(nfull):
            piece = tuple(toks[i * bs:(i + 1) * bs])
            h = fnv1a_fold(h, piece)
            e = self._full_child(parent, h, piece) if new_from is None else None
            if e is not None:
                plan.append(e)
                parent = e.serial
            else:
                if new_from is None:
                    new_from = len(plan)
                plan.append((int(blocks[i]), h, piece))
        if has_tail:
            piece = tuple(toks[nfull * bs:])
            e = self._tail_child(parent, piece) if new_from is None else None
            if e is not None:
                plan.append(e)
            else:
                if new_from is None:
                    new_from = len(plan)
                plan.append((int(blocks[nfull]), None, piece))
        new_blocks = [x[0] for x in plan if not isinstance(x, _Entry)]
        for b in new_blocks:
            if not 0 <= b < self.alloc.num_blocks:
                raise AllocatorError("inval", f"block id {b} outside the pool")
            if self.alloc.refcount[b] == 0:
                raise AllocatorError("state", f"block {b} is free")
            if b in listed:
                raise AllocatorError("state", f"block {b} is listed already")
        if len(set(new_blocks)) != len(new_blocks):
            raise AllocatorError("state", "a block is used twice")
        self.clock += 1
        parent = ROOT
        created = 0
        for x in plan:
            if isinstance(x, _Entry):
                e = x
            else:
                b, key, piece = x
                e = _Entry(self.next_serial, b, parent, piece, key)
                self.next_serial += 1
                self.entries[e.serial] = e
                if parent != ROOT:
                    self.entries[parent].children += 1
                self.alloc.incref(b)
                created += 1
            e.last_use = self.clock
            if resident:
                e.resident = True
            parent = e.serial
        return created

    # -- copy-on-write -------------------------------------------------------------
    def cow(self, block: int) -> Tuple[int, bool]:
        """A block the caller may write: the block itself when the caller
        holds its only reference, else a fresh block that replaces it (the
        caller copies the old contents).  Returns (-1, False) and changes
        nothing when no block is free.  The caller must hold a reference, so
        a block held by the index alone is refused."""
        if not 0 <= block < self.alloc.num_blocks:
            raise AllocatorError("inval", f"block id {block} outside the pool")
        rc = self.alloc.refcount[block]
        if rc == 0:
            raise AllocatorError("state", f"block {block} is free")
        if rc == 1 and block in self.indexed_blocks():
            raise AllocatorError("state", f"block {block} is held only by the prefix index")
        if rc == 1:
            return block, False
        fresh = self.alloc.alloc()
        if fresh < 0:
            return -1, False
        self.alloc.decref(block)
        return fresh, True

    # -- release -------------------------------------------------------------------
    def release(self, block: int) -> None:
        """Drop a caller's reference; the index's own reference cannot be
        dropped this way."""
        if 0 <= block < self.alloc.num_blocks and self.alloc.refcount[block] == 1 \
                and block in self.indexed_blocks():
            raise AllocatorError("state", f"block {block} is held only by the prefix index")
        self.alloc.decref(block)

    # -- eviction ------------------------------------------------------------------
    def evict(self, want: int) -> List[int]:
        """Free up to ``want`` blocks held by the index alone: leaf entries,
        not resident, least recently used first (ties: oldest entry)."""
        freed = []
        while len(freed) < want:
            cands = [e for e in self.entries.values()
                     if not e.resident and e.children == 0 and self.alloc.refcount[e.block] == 1]
            if not cands:
                break
            e = min(cands, key=lambda x: (x.last_use, x.serial))
            self._drop(e)
            freed.append(e.block)
        return freed

    def clear(self) -> None:
        """Drop every entry and the index's references (resident ones too)."""
        for e in sorted(self.entries.values(), key=lambda x: -x.serial):
            self.alloc.decref(e.block)
        self.entries.clear()

    def _drop(self, e: _Entry) -> None:
        del self.entries[e.serial]
        if e.parent != ROOT:
            self.entries[e.parent].children -= 1
        self.alloc.decref(e.block)

    def stats(self) -> dict:
        es = list(self.entries.values())
        return {
            "entries": len(es),
            "tail_entries": sum(1 for e in es if e.key is None),
            "resident": sum(1 for e in es if e.resident),
            "index_only": sum(1 for e in es if self.alloc.refcount[e.block] == 1),
        }


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, src: Sequence[int], dst: Sequence[int]) -> None:
    """In place: block dst[i] of both pools takes the contents of block
    src[i].  Pairs with an id outside the pool are skipped (negative ids are
    padding).  Destinations are distinct and no destination is a source."""
    nb = k_pool.shape[0]
    for s, d in zip(src, dst):
        s, d = int(s), int(d)
        if 0 <= s < nb and 0 <= d < nb:
            k_pool[d] = k_pool[s]
            v_pool[d] = v_pool[s]

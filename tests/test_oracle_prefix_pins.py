"""Pins for the oracle's prefix index, copy-on-write and block copy.

* the per-token fold against published FNV-1a 64 test vectors (token ids
  below 256 fold exactly like bytes);
* chaining: "foobar" in blocks of three is keyed FNV("foo"), FNV("foobar");
  every block key equals a one-shot fold of the whole prefix;
* the multiply by the FNV prime against its 2^40 + 0x1b3 split;
* a genuine key collision (birthday-built) is refused by token verification;
* match / insert / copy-on-write / eviction on scenarios worked by hand;
* random operation sequences keep every reference count equal to its
  holders (caller references + index entries), and never free a listed block;
* block copy: write-then-copy round trips.
"""
import os

import numpy as np
import pytest

from fnv_collision import colliding_pair
from oracle.allocator import AllocatorError, BlockAllocatorModel
from oracle.prefix import (FNV_OFFSET_BASIS, PrefixCacheModel, chained_block_hashes, copy_blocks,
                           fnv1a_fold)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fnv_vectors():
    rows = []
    for line in open(os.path.join(GOLDEN, "fnv1a64_vectors.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        q1 = line.index('"')
        q2 = line.index('"', q1 + 1)
        rows.append((line[q1 + 1:q2], int(line[q2 + 1:].split()[0], 16)))
    return rows


def test_fold_matches_published_vectors():
    rows = _fnv_vectors()
    assert len(rows) == 12
    for s, want in rows:
        assert fnv1a_fold(FNV_OFFSET_BASIS, [ord(c) for c in s]) == want, s


def test_chained_keys_of_foobar_in_blocks_of_three():
    keys = chained_block_hashes([ord(c) for c in "foobar"], 3)
    assert keys == [0xDCB27518FED9D577, 0x85944171F73967E8]  # FNV-1a("foo"), FNV-1a("foobar")
    assert chained_block_hashes([ord(c) for c in "foobar!"], 3) == keys  # partial block: no key
    assert chained_block_hashes([ord(c) for c in "fo"], 3) == []


def test_chained_key_is_fold_of_whole_prefix():
    rng = np.random.default_rng(1)
    toks = [int(x) for x in rng.integers(0, 1 << 32, size=16 * 7 + 5, dtype=np.uint64)]
    keys = chained_block_hashes(toks, 16)
    assert len(keys) == 7
    for i, k in enumerate(keys):
        h = FNV_OFFSET_BASIS
        for t in toks[: 16 * (i + 1)]:  # one token at a time, from the basis
            h = fnv1a_fold(h, [t])
        assert k == h
    # restarting each block at the basis (no chaining) gives other keys
    assert keys[1] != fnv1a_fold(FNV_OFFSET_BASIS, toks[16:32])


def test_fold_step_against_prime_split():
    rng = np.random.default_rng(2)
    for _ in range(2000):
        h = int(rng.integers(0, 1 << 63)) * 2 + int(rng.integers(0, 2))
        t = int(rng.integers(0, 1 << 32))
        x = h ^ t
        want = ((x << 40) + x * 0x1B3) % (1 << 64)
        assert fnv1a_fold(h, [t]) == want
    # ids wider than 32 bits keep their low 32 bits
    assert fnv1a_fold(FNV_OFFSET_BASIS, [(1 << 32) + 97]) == fnv1a_fold(FNV_OFFSET_BASIS, [97])


def test_collision_is_refused_by_token_verification():
    a, b = colliding_pair(4, seed=3)
    assert a != b
    assert chained_block_hashes(a, 4) == chained_block_hashes(b, 4)
    m = PrefixCacheModel(BlockAllocatorModel(8), 4)
    blk = m.alloc.alloc()
    assert m.insert(a, [blk]) == 1
    assert m.match(b + [1, 2, 3], 8) == ([], 0)
    assert m.match(a + [1, 2, 3], 8) == ([blk], 4)
    # the colliding block is a different prefix: listed on its own
    blk2 = m.alloc.alloc()
    assert m.insert(b, [blk2]) == 1
    assert m.match(b, 8) == ([blk2], 4)


def test_hand_worked_scenario():
    """Block size 4, pool of 8 blocks; every number below follows from the
    rules in the oracle's docstring, worked by hand."""
    m = PrefixCacheModel(BlockAllocatorModel(8), 4)
    a = list(range(1, 11))  # 10 tokens: two full blocks and a tail of 2
    blocks = [m.alloc.alloc() for _ in range(3)]
    assert blocks == [0, 1, 2]
    assert m.insert(a, blocks, tail=True, resident=True) == 3
    assert m.alloc.refcount[:4] == [2, 2, 2, 0]
    for b in blocks:  # the warm-up drops its own references
        m.release(b)
    assert m.alloc.refcount[:4] == [1, 1, 1, 0]
    assert m.stats() == {"entries": 3, "tail_entries": 1, "resident": 3, "index_only": 3}
    with pytest.raises(AllocatorError):  # the index's reference is not the caller's
        m.release(0)
    with pytest.raises(AllocatorError):  # nor may a caller write through it
        m.cow(0)

    # B extends the prompt: both full blocks and the tail are reused
    blocks_b, covered = m.match(a + [50, 51], 16)
    assert (blocks_b, covered) == ([0, 1, 2], 10)
    assert m.alloc.refcount[:4] == [2, 2, 2, 0]
    # B writes token 10 into the shared tail: copy-on-write takes block 3
    assert m.cow(2) == (3, True)
    assert m.alloc.refcount[:4] == [2, 2, 1, 1]
    assert m.cow(3) == (3, False)  # B owns block 3 alone now

    # C shares the first block only; D stops before the tail's second token;
    # E covers both full blocks exactly; F shares nothing
    assert m.match([1, 2, 3, 4, 9, 9, 9, 9], 16) == ([0], 4)
    assert m.match(list(range(1, 10)), 16) == ([0, 1], 8)
    assert m.match(list(range(1, 9)), 16) == ([0, 1], 8)
    assert m.match([2, 3, 4, 5, 6], 16) == ([], 0)
    assert m.alloc.refcount[:4] == [5, 4, 1, 1]
    # the caller's capacity bounds the match
    assert m.match(a + [50, 51], 1) == ([0], 4)
    for b in [0, 0, 1, 0, 1, 0]:  # C, D, E, the capped match release
        m.release(b)
    assert m.alloc.refcount[:4] == [2, 2, 1, 1]

    # B lists its three full blocks: blocks 0 and 1 are known, block 3 is new
    assert m.insert(a + [50, 51], [0, 1, 3]) == 1
    assert m.alloc.refcount[:4] == [2, 2, 1, 2]
    for b in [0, 1, 3]:  # B finishes
        m.release(b)
    assert m.alloc.refcount[:4] == [1, 1, 1, 1]
    # every resident entry stays; B's block is the only one eviction may free
    assert m.evict(5) == [3]
    assert m.alloc.refcount[:4] == [1, 1, 1, 0]
    assert m.evict(5) == []
    m.clear()
    assert m.alloc.refcount[:4] == [0, 0, 0, 0]


def test_eviction_order_is_least_recent_leaf_first():
    m = PrefixCacheModel(BlockAllocatorModel(16), 2)
    # three chains of two full blocks each: P = [1,2 | 3,4], Q = [5,6 | 7,8], R = [1,2 | 9,9]
    p = [m.alloc.alloc() for _ in range(2)]
    m.insert([1, 2, 3, 4], p)  # clock 1
    q = [m.alloc.alloc() for _ in range(2)]
    m.insert([5, 6, 7, 8], q)  # clock 2
    r = [m.alloc.alloc()]
    m.insert([1, 2, 9, 9], [p[0], r[0]])  # clock 3: reuses P's first entry
    for b in p + q + r:
        m.release(b)
    assert p == [0, 1] and q == [2, 3] and r == [4]
    got, cov = m.match([5, 6, 7, 8], 4)  # clock 4: Q is the most recent now
    for b in got:
        m.release(b)
    # leaves: P's second block (used at clock 1), R's (clock 3), Q's (clock 4);
    # the shared first entry of P and R becomes a leaf once both are gone
    assert m.evict(1) == [1]
    assert m.evict(1) == [4]
    assert m.evict(1) == [0]  # P/R's first entry (clock 3) before Q's (clock 4)
    assert m.evict(9) == [3, 2]


def test_insert_refuses_bad_blocks_and_changes_nothing():
    m = PrefixCacheModel(BlockAllocatorModel(8), 4)
    b0 = m.alloc.alloc()
    with pytest.raises(AllocatorError) as e:
        m.insert(list(range(8)), [b0, 5])  # block 5 is free
    assert e.value.kind == "state"
    assert m.entries == {} and m.alloc.refcount[b0] == 1
    b1 = m.alloc.alloc()
    with pytest.raises(AllocatorError):
        m.insert(list(range(8)), [b0, b0])  # used twice
    with pytest.raises(AllocatorError) as e:
        m.insert(list(range(8)), [b0])  # too few blocks
    assert e.value.kind == "inval"
    assert m.insert(list(range(8)), [b0, b1]) == 2
    b2 = m.alloc.alloc()
    with pytest.raises(AllocatorError):
        m.insert([7, 7, 7, 7], [b1])  # block 1 is listed already
    assert m.insert(list(range(8)), [b2, b2]) == 0  # both known: nothing new
    assert m.alloc.refcount[:3] == [2, 2, 1]


def test_cow_when_pool_is_full_changes_nothing():
    m = PrefixCacheModel(BlockAllocatorModel(2), 4)
    b0, b1 = m.alloc.alloc(), m.alloc.alloc()
    m.alloc.incref(b0)
    assert m.cow(b0) == (-1, False)
    assert m.alloc.refcount == [2, 1]
    with pytest.raises(AllocatorError):
        m.cow(7)


def test_random_operations_keep_counts_equal_to_holders():
    rng = np.random.default_rng(11)
    bs, nb = 4, 48
    m = PrefixCacheModel(BlockAllocatorModel(nb), bs)
    vocab = [1, 2, 3]  # a tiny vocabulary makes prefixes collide often
    seqs = []  # (tokens, blocks) held by callers
    for step in range(1500):
        op = rng.integers(0, 5)
        if op <= 1:  # admit a sequence: match, copy-on-write the tail, allocate, list
            n = int(rng.integers(1, 20))
            toks = [vocab[int(i)] for i in rng.integers(0, 3, size=n)]
            blocks, cov = m.match(toks, 64)
            ok = True
            if cov % bs and cov < n:  # a partial tail that we write into
                new, copied = m.cow(blocks[-1])
                if new < 0:
                    ok = False
                else:
                    blocks[-1] = new
            while ok and len(blocks) * bs < n:
                b = m.alloc.alloc()
                if b < 0:
                    m.evict(1)
                    b = m.alloc.alloc()
                if b < 0:
                    ok = False
                    break
                blocks.append(b)
            if not ok:
                for b in blocks:
                    m.release(b)
                continue
            if rng.integers(0, 2):
                m.insert(toks, blocks, tail=bool(rng.integers(0, 2)), resident=rng.integers(0, 8) == 0)
            seqs.append((toks, blocks))
        elif op == 2 and seqs:
            toks, blocks = seqs.pop(int(rng.integers(0, len(seqs))))
            for b in blocks:
                m.release(b)
        elif op == 3:
            m.evict(int(rng.integers(0, 4)))
        holders = [0] * nb
        for _, blocks in seqs:
            for b in blocks:
                holders[b] += 1
        for e in m.entries.values():
            holders[e.block] += 1
        assert holders == m.alloc.refcount, step
        assert len(m.indexed_blocks()) == len(m.entries)
    assert m.stats()["entries"] > 0


def test_copy_blocks_round_trip():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((6, 4, 2, 8))
    v = rng.standard_normal((6, 4, 2, 8))
    k0, v0 = k.copy(), v.copy()
    copy_blocks(k, v, [1, 4, -1, 2, 9], [3, 0, 5, 5, 1])
    assert np.array_equal(k[3], k0[1]) and np.array_equal(v[3], v0[1])
    assert np.array_equal(k[0], k0[4]) and np.array_equal(v[0], v0[4])
    assert np.array_equal(k[5], k0[2]) and np.array_equal(v[5], v0[2])  # (-1, 5) is padding
    for i in (1, 2, 4):  # sources and untouched blocks keep their contents
        assert np.array_equal(k[i], k0[i]) and np.array_equal(v[i], v0[i])

"""Pins for the oracle's continuous-batching scheduler: iterations worked by
hand from the page's three steps (decoding requests first, then
first-come-first-served admission that stops at the first request that does
not fit, then the release of finished requests), preemption when no block
is free, and invariants under random traffic.
"""
import numpy as np
import pytest

from oracle.allocator import AllocatorError, BlockAllocatorModel
from oracle.batching import ContinuousBatchingModel


def _model(num_blocks, bs=4, max_batch=3, max_blocks=8):
    return ContinuousBatchingModel(BlockAllocatorModel(num_blocks), bs, max_batch, max_blocks)


def _view(batch):
    return [(s.rid, s.prefill, s.table, s.context_len, s.write_start, s.write_count) for s in batch]


def test_hand_worked_iterations():
    """Block size 4, six blocks, batch of at most 3."""
    m = _model(6)
    m.add(1, 5, 3)
    m.add(2, 8, 2)
    m.add(3, 9, 1)
    m.add(4, 2, 2)
    # 1: requests 1 and 2 fit (2 + 2 blocks); 3 needs 3 of the 2 left: it
    # goes back to the head of the queue and admission stops (4 waits too)
    batch, info = m.schedule()
    assert _view(batch) == [(1, True, [0, 1], 5, 0, 5), (2, True, [2, 3], 8, 0, 8)]
    assert (info.scheduled, info.prefill, info.waiting, info.active) == (2, 2, 2, 2)
    m.step(1)
    m.step(2)
    # 2: request 1 holds 6 tokens in 2 blocks; request 2 holds 9 and takes
    # block 4; one block is left, still short of request 3's three
    batch, info = m.schedule()
    assert _view(batch) == [(1, False, [0, 1], 6, 5, 1), (2, False, [2, 3, 4], 9, 8, 1)]
    assert info.prefill == 0 and info.waiting == 2
    m.step(1)
    m.step(2)  # request 2 reaches its 2 tokens
    # 3: request 2 is finished: not scheduled, freed at the end of the call
    batch, info = m.schedule()
    assert _view(batch) == [(1, False, [0, 1], 7, 6, 1)]
    assert (info.freed_requests, info.freed_blocks, info.active, info.waiting) == (1, 3, 1, 2)
    assert m.alloc.refcount == [1, 1, 0, 0, 0, 0]
    m.step(1)  # request 1 reaches its 3 tokens
    # 4: request 3 takes blocks 2, 3, 4 and request 4 block 5; request 1 leaves
    batch, info = m.schedule()
    assert _view(batch) == [(3, True, [2, 3, 4], 9, 0, 9), (4, True, [5], 2, 0, 2)]
    assert (info.prefill, info.freed_requests, info.freed_blocks) == (2, 1, 2)
    assert m.alloc.refcount == [0, 0, 1, 1, 1, 1]
    m.step(3)  # finished after one token
    m.step(4)
    batch, info = m.schedule()
    assert _view(batch) == [(4, False, [5], 3, 2, 1)]
    assert (info.freed_requests, info.freed_blocks) == (1, 3)


def test_preemption_without_free_blocks():
    """Three blocks of 4 tokens, two requests of 4-token prompts: the second
    cannot grow while the first holds the last block, sits out until the
    first is freed, then resumes where it stopped."""
    m = _model(3, max_batch=2)
    m.add(1, 4, 5)
    m.add(2, 4, 5)
    batch, _ = m.schedule()
    assert [s.rid for s in batch] == [1, 2]
    m.step(1)
    m.step(2)
    preempted = 0
    for it in range(20):
        batch, info = m.schedule()
        preempted += info.preempted
        ids = [s.rid for s in batch]
        if it < 4:
            assert ids == [1] and info.preempted == 1
        for s in batch:
            m.step(s.rid)
        if not m.active and not m.waiting:
            break
    assert preempted == 5  # iterations 2..5 and the one where request 1 is freed
    assert m.alloc.refcount == [0, 0, 0]


def test_refusals():
    m = _model(4, max_blocks=2)
    with pytest.raises(AllocatorError):
        m.add(1, 0, 3)
    with pytest.raises(AllocatorError):
        m.add(1, 5, 4)  # 9 tokens need 3 blocks of 4
    m.add(1, 5, 3)
    with pytest.raises(AllocatorError):
        m.add(1, 2, 2)  # known id
    with pytest.raises(AllocatorError):
        m.step(1)  # not admitted yet


def test_invariants_under_random_traffic():
    rng = np.random.default_rng(12)
    bs, nb, mb = 16, 40, 12
    m = ContinuousBatchingModel(BlockAllocatorModel(nb), bs, 6, mb)
    next_id = 0
    total_prefill = total_preempted = 0
    for it in range(600):
        for _ in range(int(rng.integers(0, 3))):
            p = int(rng.integers(1, 100))
            mt = int(rng.integers(1, mb * bs - p + 1))
            m.add(next_id, p, mt)
            next_id += 1
        batch, info = m.schedule()
        total_prefill += info.prefill
        total_preempted += info.preempted
        assert len(batch) <= m.max_batch
        held = [b for r in m.active for b in r.table]
        assert len(held) == len(set(held))
        assert sorted(held) == [i for i, c in enumerate(m.alloc.refcount) if c > 0]
        for s in batch:
            assert len(s.table) == -(-s.context_len // bs)
            assert s.write_start + s.write_count == s.context_len
            m.step(s.rid)
    assert total_prefill > 20 and total_preempted > 0

"""Two different token-id blocks with the same 64-bit FNV-1a key.

With whole 32-bit token ids folded per step, a collision after two tokens
takes a birthday search over the first id only: the state after id t0 is
((s0 ^ t0) * prime) mod 2^64, and once two choices of t0 agree in the upper
32 bits of that state, the second id can cancel the lower 32 bits.  Every
later id being equal, the two blocks then share their key.  The search is
written here from that argument (numpy uint64 arithmetic wraps mod 2^64),
independently of the oracle and of the library.
"""
from __future__ import annotations

import numpy as np

OFFSET_BASIS = 0xCBF29CE484222325
PRIME = 0x100000001B3


def colliding_pair(block_size: int, seed: int = 0, s0: int = OFFSET_BASIS):
    """Two token lists of ``block_size`` ids (uint32) that differ in their first
    two ids and fold from state ``s0`` to the same key."""
    rng = np.random.default_rng(seed)
    hi0 = np.uint64(s0 & 0xFFFFFFFF00000000)
    lo0 = np.uint64(s0 & 0xFFFFFFFF)
    u = np.unique(rng.integers(0, 1 << 32, size=1 << 19, dtype=np.uint64))
    with np.errstate(over="ignore"):
        s1 = (hi0 | u) * np.uint64(PRIME)
    hi = s1 >> np.uint64(32)
    order = np.argsort(hi, kind="stable")
    hs = hi[order]
    dup = np.flatnonzero(hs[1:] == hs[:-1])
    if dup.size == 0:
        raise RuntimeError("no collision found; try another seed")
    i, j = order[dup[0]], order[dup[0] + 1]
    t0a, t0b = int(u[i] ^ lo0), int(u[j] ^ lo0)
    lo_a, lo_b = int(s1[i]) & 0xFFFFFFFF, int(s1[j]) & 0xFFFFFFFF
    t1a = int(rng.integers(0, 1 << 32))
    t1b = t1a ^ lo_a ^ lo_b
    rest = [int(x) for x in rng.integers(0, 1 << 32, size=block_size - 2)]
    return [t0a, t1a] + rest, [t0b, t1b] + rest

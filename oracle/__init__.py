"""Plain fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything
in this package.  The HIP library never links, imports or calls it, and it
imports nothing from the HIP library: the two share no code.  The only module
both consume is ``workloads`` (seeded input draws, no method arithmetic).

Everything here is deliberately slow and obvious: numpy in float64, one
sequence and one head at a time, no blocking, fusion or reordering beyond
what the definitions state.  Stored f32/f16/bf16 inputs widen exactly to
float64.

Parity status of each function (what pins it is listed in the tests):

* ``gather_rows``, ``decode``: pinned (dense-attention special case against
  a library routine, pure-Python brute force, n = 1, constant keys,
  permutation and shared-prefix invariance, write-then-read round trip).
* ``decode_multi`` (several new tokens per sequence, causal): pinned
  (q_len = 1 equals ``decode``; each new token equals ``decode`` over its
  own prefix; dense causal attention against torch's
  scaled_dot_product_attention with an explicit mask; keys after a token's
  position never change its row; tokens before position 0 give zeros).
* ``ring_slot``, ``ring_cache_order``, ``ring_cache_index``: pinned (values
  worked by hand from the sink + ring slot equation, brute-force last-writer
  simulation).
* ``rope_rotate_half``: pinned (complex-multiplication form, norm
  preservation, relative-position invariance, identity at position 0).  The
  pairing convention itself is a reading, not fixed by the pages.
* ``reshape_and_cache``: pinned (write-then-gather round trip, untouched
  rows keep their bytes).
* ``BlockAllocatorModel``: pinned (lowest-free-id order, exhaustion, release
  at the last reference, stats).
* ``batching`` (continuous-batching scheduler over the pool): pinned
  (iterations worked by hand from the page's three steps, preemption and
  resumption, refusals, invariants under random traffic).  Visiting order,
  allocation order and token positions are readings.
* closed forms in ``sizes``: pinned against the numbers the pages print.
* ``fp8`` (E4M3 and E5M2 values, nearest-even encoding with saturation,
  per-head scaling) and ``quantize_for_cache``: pinned (codes worked by hand
  from the format definitions, every code round-trips, rounding is monotone
  and nearest, ties go to the even code, E5M2 values equal IEEE binary16
  numbers with the code as top byte); the formats and scaling rule are
  readings, the page names FP8 storage without fixing either.
* ``prefix`` (chained FNV-1a block keys, the prefix index with token
  verification, copy-on-write, least-recent leaf eviction, block copy):
  pinned (published FNV-1a test vectors, chaining identity, the prime's
  2^40 + 0x1b3 split, a birthday-built key collision refused by
  verification, scenarios worked by hand, reference counts equal to holders
  under random operations, copy round trips).  Chaining, verification
  against the parent entry, the index's own reference and tail entries are
  readings: the page's listing leaves them open or gets them wrong.
"""
from . import fp8  # noqa: F401
from . import prefix  # noqa: F401
from . import batching  # noqa: F401
from .paged_attention import (  # noqa: F401
    quantize_for_cache,
    to_f64,
    gather_rows,
    slot_of,
    attention_one_group,
    decode,
    decode_multi,
    decode_verify_ring,
    reshape_and_cache,
    reshape_and_cache_,
    build_pools,
    ring_slot,
    ring_cache_order,
    ring_cache_index,
    rope_inv_freq,
    rope_rotate_half,
    ring_writer,
)
from .allocator import BlockAllocatorModel  # noqa: F401
from . import sizes  # noqa: F401

"""Reference model of the continuous-batching scheduler that drives the
paged cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "大模型推理内存优化：从 KV Cache 分页到连续批处理的工程实践"
(pwwt.cn/news/3010209): its scheduler decides, every iteration, which
requests run, and manages their blocks.  One scheduling call takes three
steps in this order:

1. every request in the decoding state stays in the batch; when the tokens
   it holds (prompt + generated) need more blocks than its table has, it
   gets one more block, and when none is free it sits this iteration out
   (preempted) and keeps what it has;
2. waiting requests are admitted first-come first-served while the batch
   is below its maximum size and the free blocks cover the prompt
   (ceil(prompt / block_size) blocks, allocated at once); the first that
   does not fit goes back to the head of the queue and admission stops;
3. requests that have generated their maximum number of tokens leave, and
   their blocks return to the pool.

After an iteration each scheduled request advances by one generated token
(the step call); reaching the maximum marks it finished, so step 3 of the
next scheduling call frees it.

Readings where the page leaves a step open:

* order: decoding requests are visited in admission order (the page keeps
  them in a hash map, whose order is unspecified); the batch lists them in
  that order, then the requests admitted in this call;
* blocks come from the pool's allocator (lowest free id first, the
  embedded page's allocator) rather than the page's own FIFO free list;
  blocks are returned by dropping the request's reference;
* tokens: the admission iteration is the prefill, which writes the prompt's
  K/V at positions 0 .. prompt - 1 and produces the first generated token;
  every later iteration writes the K/V of the token generated last, at
  position prompt + generated - 1, and attends over prompt + generated
  positions (which is what the page's block count covers);
* a request must have a prompt of at least one token and a table wide
  enough for prompt + max_tokens tokens; other requests are refused.

Parity status: pinned by iterations worked by hand from the three steps
(admission order, head-of-queue blocking, preemption, freeing at the next
call), and by invariants (every held block belongs to exactly one request,
each decoding request holds ceil(tokens / block_size) blocks, the batch
never exceeds its maximum).
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Deque, List

from .allocator import AllocatorError, BlockAllocatorModel

WAITING, DECODING, FINISHED = "waiting", "decoding", "finished"


@dataclass
class Request:
    rid: int
    prompt_len: int
    max_tokens: int
    generated: int = 0
    table: List[int] = field(default_factory=list)
    state: str = WAITING


@dataclass
class Scheduled:
    rid: int
    prefill: bool
    table: List[int]
    context_len: int  # positions attended after this iteration's writes
    write_start: int  # first position written this iteration
    write_count: int


@dataclass
class IterationInfo:
    scheduled: int = 0
    prefill: int = 0
    preempted: int = 0
    freed_requests: int = 0
    freed_blocks: int = 0
    waiting: int = 0
    active: int = 0


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class ContinuousBatchingModel:
    alloc: BlockAllocatorModel
    block_size: int
    max_batch: int
    max_blocks_per_seq: int
    waiting: Deque[Request] = field(default_factory=deque)
    active: List[Request] = field(default_factory=list)  # admission order

    def add(self, rid: int, prompt_len: int, max_tokens: int) -> None:
        if prompt_len < 1 or max_tokens < 1:
            raise AllocatorError("inval", "a request needs a prompt and at least one token to generate")
        if _ceil_div(prompt_len + max_tokens, self.block_size) > self.max_blocks_per_seq:
            raise AllocatorError("inval", "the request does not fit a block table")
        if any(r.rid == rid for r in self.active) or any(r.rid == rid for r in self.waiting):
            raise AllocatorError("state", f"request {rid} is known already")
        self.waiting.append(Request(rid, prompt_len, max_tokens))

    def schedule(self):
        info = IterationInfo()
        batch: List[Scheduled] = []
        # step 1: decoding requests stay, growing by a block when needed
        for r in self.active:
            if r.state != DECODING:
                continue
            tokens = r.prompt_len + r.generated
            if _ceil_div(tokens, self.block_size) > len(r.table):
                b = self.alloc.alloc()
                if b < 0:
                    info.preempted += 1
                    continue
                r.table.append(b)
            pos = tokens - 1
            batch.append(Scheduled(r.rid, False, list(r.table), tokens, pos, 1))
        # step 2: admit waiting requests while the batch has room and blocks fit
        while len(batch) < self.max_batch and self.waiting:
            r = self.waiting.popleft()
            need = _ceil_div(r.prompt_len, self.block_size)
            if self.alloc.num_blocks - sum(1 for c in self.alloc.refcount if c > 0) >= need:
                r.table = [self.alloc.alloc() for _ in range(need)]
                r.state = DECODING
                self.active.append(r)
                batch.append(Scheduled(r.rid, True, list(r.table), r.prompt_len, 0, r.prompt_len))
                info.prefill += 1
            else:
                self.waiting.appendleft(r)
                break
        # step 3: finished requests leave and free their blocks
        keep = []
        for r in self.active:
            if r.generated >= r.max_tokens:
                for b in r.table:
                    self.alloc.decref(b)
                info.freed_requests += 1
                info.freed_blocks += len(r.table)
            else:
                keep.append(r)
        self.active = keep
        info.scheduled = len(batch)
        info.waiting = len(self.waiting)
        info.active = len(self.active)
        return batch, info

    def step(self, rid: int) -> None:
        for r in self.active:
            if r.rid == rid:
                if r.state != DECODING:
                    raise AllocatorError("state", f"request {rid} is not decoding")
                r.generated += 1
                if r.generated >= r.max_tokens:
                    r.state = FINISHED
                return
        raise AllocatorError("inval", f"request {rid} is not active")

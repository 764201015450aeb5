"""Reference model of the block allocator with reference counts.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* "端侧 SLM 显存保活术…" (sheratonhq.com/news/141880), section
  "嵌入式轻量 Block 分配器设计": a free bitmap scanned word by word with a
  count-trailing-zeros step, so allocation hands out the lowest free id
  first and reports -1 once the pool is exhausted.
* "Ollama的内存管理策略：从KV Cache Block分配到Prefix-aware内存复用的演进"
  (xdnf.cn/news/5086), section "三、KV Cache内存管理的工程实现": blocks
  carry a reference count; a shared prefix block is referenced by every
  sequence using it; releasing decrements the count and the last release
  returns the block to the free pool; pool statistics report total, used,
  shared (count above one) and free blocks.

Error model (a reading: the pages' code ignores misuse): an id outside the
pool is "inval"; referencing or releasing a free block is "state".
"""
from __future__ import annotations


class AllocatorError(Exception):
    def __init__(self, kind: str, msg: str):
        super().__init__(msg)
        self.kind = kind  # "inval" | "state"


class BlockAllocatorModel:
    def __init__(self, num_blocks: int):
        if num_blocks <= 0:
            raise AllocatorError("inval", "num_blocks must be positive")
        self.refcount = [0] * num_blocks

    @property
    def num_blocks(self) -> int:
        return len(self.refcount)

    def alloc(self) -> int:
        for block_id, rc in enumerate(self.refcount):
            if rc == 0:
                self.refcount[block_id] = 1
                return block_id
        return -1

    def _check(self, block_id: int) -> None:
        if not 0 <= block_id < self.num_blocks:
            raise AllocatorError("inval", f"block id {block_id} outside the pool")
        if self.refcount[block_id] == 0:
            raise AllocatorError("state", f"block {block_id} is free")

    def incref(self, block_id: int) -> None:
        self._check(block_id)
        self.refcount[block_id] += 1

    def decref(self, block_id: int) -> None:
        self._check(block_id)
        self.refcount[block_id] -= 1

    def stats(self) -> dict:
        used = sum(1 for rc in self.refcount if rc > 0)
        shared = sum(1 for rc in self.refcount if rc > 1)
        return {"total": self.num_blocks, "used": used, "shared": shared,
                "free": self.num_blocks - used}

"""CPU oracle for the block bookkeeping around the paged KV pool: a reference-counted
allocator of physical blocks with copy-on-write appends, and the block copy itself.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
this module: only the tests and the benchmark use it.  It shares no code with the
library's allocator or its HIP copy kernel.

What it computes, and where that is defined (pages cited by title and section):

* Serving-engine KV page (ttlab, "LLM KV cache 02"), section 2 "PagedAttention",
  subsection "blocks and block table": blocks of 16 tokens may sit anywhere in free
  memory; a request takes one new block at the moment its current block is full.  So
  appending the token at position pos needs a fresh block exactly when pos % 16 == 0.
* Same page, subsection "block sharing": requests that share a prompt (parallel
  sampling, beam search) point their tables at the same blocks, each block carries a
  reference count, and a block is copied only when one of its holders has to append
  into it (copy-on-write).  So: forking a table adds one reference to each of its
  blocks; releasing a table removes one, and a block with no references is free
  again; appending into a block with more than one reference first moves the
  appending table onto a private copy (one copy per block), leaving the others on the
  original.

Readings where the pages are silent (also listed in the design notes):
* Which free block is taken: the lowest-numbered one (deterministic, so the library
  and this oracle can be compared id for id).
* An append that would need more blocks than are free fails as a whole and changes
  nothing.
* A copy replaces every row of the block (all kv heads, all 16 offsets) in both
  pools, bit for bit; the stale rows of a partly used block travel too, which is
  harmless (only offsets below the context length are ever read).
"""
from __future__ import annotations

import heapq

import numpy as np

BLOCK_SIZE = 16


class OutOfBlocks(Exception):
    """An append needed more free blocks than the pool has; nothing was changed."""


class RefcountAllocator:
    """Physical blocks 0..num_blocks-1, each with a reference count (0 = free)."""

    def __init__(self, num_blocks: int):
        self.num_blocks = num_blocks
        self.ref = [0] * num_blocks
        self._free = list(range(num_blocks))      # a min-heap of free ids
        heapq.heapify(self._free)

    def num_free(self) -> int:
        return len(self._free)

    def _take(self) -> int:
        b = heapq.heappop(self._free)
        self.ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            heapq.heappush(self._free, b)

    def fork(self, table: list[int]) -> list[int]:
        """Another request shares every block of `table` (block sharing)."""
        for b in table:
            self.ref[b] += 1
        return list(table)

    def release(self, table: list[int]) -> None:
        """A request finishes: one reference fewer on each of its blocks."""
        for b in table:
            self._drop(b)

    def append(self, table: list[int], context_len: int, num_new: int):
        """Append num_new tokens after context_len cached ones to the request whose
        blocks are `table` (modified in place).  Returns (slots, copies): the flat slot
        of each new token and the (source, destination) block pairs to copy before the
        new tokens are written."""
        # What the append needs, before anything changes.
        need = 0
        shared_seen = set()
        for i in range(num_new):
            pos = context_len + i
            lb = pos // BLOCK_SIZE
            # (blocks this append creates are private: only existing ones can be shared)
            if pos % BLOCK_SIZE == 0:
                need += 1
            elif lb < len(table) and lb not in shared_seen and self.ref[table[lb]] > 1:
                shared_seen.add(lb)
                need += 1
        if need > self.num_free():
            raise OutOfBlocks(f"append needs {need} blocks, {self.num_free()} free")
        slots, copies = [], []
        for i in range(num_new):
            pos = context_len + i
            lb, off = divmod(pos, BLOCK_SIZE)
            if off == 0:
                assert lb == len(table), "table must end at the last used block"
                table.append(self._take())
            elif self.ref[table[lb]] > 1:
                src = table[lb]
                dst = self._take()
                self.ref[src] -= 1          # still held by the others, never freed here
                table[lb] = dst
                copies.append((src, dst))
            slots.append(table[lb] * BLOCK_SIZE + off)
        return slots, copies


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, copies) -> tuple[np.ndarray, np.ndarray]:
    """Bit copy of whole blocks (all kv heads and offsets) in both pools, in order."""
    kp, vp = k_pool.copy(), v_pool.copy()
    for src, dst in copies:
        kp[dst] = kp[src]
        vp[dst] = vp[src]
    return kp, vp

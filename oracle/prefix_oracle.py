"""CPU oracle for prefix caching: per-block content keys and a block pool that keeps the
contents of freed blocks for reuse, evicting the least recently used first.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
this module: only the tests and the benchmark use it.  It shares no code with the
library's prefix cache (the hash here is Python's hashlib).

What it computes, and where that is defined (pages cited by title and section):

* Serving-engine KV page (ttlab, "LLM KV cache 02"), section 4 "prefix cache":
  - every block gets a key = hash(key of the previous block, this block's token ids,
    extra inputs), the extras being a LoRA adapter, hashes of multimodal inputs and a
    cache salt that separates users;
  - since the previous key is hashed in, one key stands for the whole prefix up to
    and including its block: the same 16 tokens behind different prefixes get
    different keys;
  - only full blocks are cached;
  - a finished request's blocks are not dropped but go to a queue of free blocks
    whose contents are kept; when space is needed the least recently used is evicted
    first, and a finished request's blocks enter that queue tail first, so its last
    blocks (least likely to be reused) are evicted before its first ones;
  - the default hash is SHA-256.
* "How inference engines actually work" page (xiaohu-jiedu), prefix caching in the
  agent-traffic section: the engine hashes each computed block; a new request whose
  prefix matches points its table at the blocks already in memory, transparently, and
  only the new tail is prefilled (10 turns adding one unit each: 10 units of prefill
  instead of 1 + 2 + ... + 10 = 55).

Readings where the pages are silent (also listed in the design notes):
* Hash input layout: the previous key (32 bytes; 32 zero bytes before the first
  block), then the block's 16 token ids as little-endian int32, then the length of
  the extras as little-endian uint32 and the extras bytes.
* A free block that holds no cached content is used before a cached one is evicted
  (eviction happens only when space is needed); among content-free blocks the lowest
  id goes first, as in the plain allocator.
* A hit on a cached block that sits in the eviction queue takes it out of the queue.
* Registering a key that already names another block keeps the existing mapping.
"""
from __future__ import annotations

import collections
import hashlib
import heapq
import struct

BLOCK_SIZE = 16
KEY_BYTES = 32
ROOT_KEY = bytes(KEY_BYTES)


class OutOfBlocks(Exception):
    """More blocks were needed than are free or evictable; nothing was changed."""


def block_key(parent: bytes, block_tokens, extras: bytes = b"") -> bytes:
    """Key of one full block: SHA-256 over (parent key, token ids, extras)."""
    assert len(parent) == KEY_BYTES and len(block_tokens) == BLOCK_SIZE
    msg = bytes(parent) + struct.pack("<16i", *[int(t) for t in block_tokens])
    msg += struct.pack("<I", len(extras)) + bytes(extras)
    return hashlib.sha256(msg).digest()


def block_keys(tokens, extras: bytes = b"", parent: bytes = ROOT_KEY) -> list[bytes]:
    """Keys of every full block of `tokens` (a partial last block gets none)."""
    keys, prev = [], parent
    for b in range(len(tokens) // BLOCK_SIZE):
        prev = block_key(prev, tokens[b * BLOCK_SIZE:(b + 1) * BLOCK_SIZE], extras)
        keys.append(prev)
    return keys


class PrefixCachingAllocator:
    """Blocks 0..num_blocks-1 with reference counts; blocks with no references are
    either free (no content kept, lowest id first) or evictable (their cached content
    kept, in least-recently-used order)."""

    def __init__(self, num_blocks: int):
        self.num_blocks = num_blocks
        self.ref = [0] * num_blocks
        self._free = list(range(num_blocks))          # min-heap of content-free blocks
        heapq.heapify(self._free)
        self.evictable = collections.OrderedDict()    # block -> None, front = evict next
        self.key_of: dict[int, bytes] = {}            # cached block -> key
        self.block_of: dict[bytes, int] = {}          # key -> cached block

    def num_free(self) -> int:
        """Blocks that can be handed out: free plus evictable."""
        return len(self._free) + len(self.evictable)

    def _take(self) -> int:
        if self._free:
            b = heapq.heappop(self._free)
        else:                                         # evict the least recently used
            b, _ = self.evictable.popitem(last=False)
            del self.block_of[self.key_of.pop(b)]
        self.ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.evictable[b] = None              # most recently used end
            else:
                heapq.heappush(self._free, b)

    def match(self, keys) -> list[int]:
        """Blocks of the longest run of leading keys that are cached; each gains a
        reference (and leaves the eviction queue)."""
        hit = []
        for k in keys:
            b = self.block_of.get(k)
            if b is None:
                break
            hit.append(b)
        for b in hit:
            if self.ref[b] == 0:
                del self.evictable[b]
            self.ref[b] += 1
        return hit

    def register(self, table, keys) -> None:
        """Cache the full blocks table[i] under keys[i] (an existing key keeps its
        block)."""
        for b, k in zip(table, keys):
            if k in self.block_of or b in self.key_of:
                continue
            self.block_of[k] = b
            self.key_of[b] = k

    def fork(self, table) -> list[int]:
        for b in table:
            self.ref[b] += 1
        return list(table)

    def release(self, table) -> None:
        """A request ends: its blocks lose one reference each, tail first, so that the
        tail enters the eviction queue first."""
        for b in reversed(table):
            self._drop(b)

    def append(self, table: list[int], context_len: int, num_new: int):
        """As the plain allocator's append (a new block at each 16-token boundary, a
        private copy of a shared partly filled last block first); returns (slots,
        copies).  Fails as a whole with OutOfBlocks."""
        need = 0
        for i in range(num_new):
            pos = context_len + i
            lb = pos // BLOCK_SIZE
            if pos % BLOCK_SIZE == 0:
                need += 1
            elif i == 0 and lb < len(table) and self.ref[table[lb]] > 1:
                need += 1
        if need > self.num_free():
            raise OutOfBlocks(f"append needs {need} blocks, {self.num_free()} available")
        slots, copies = [], []
        for i in range(num_new):
            pos = context_len + i
            lb, off = divmod(pos, BLOCK_SIZE)
            if off == 0:
                assert lb == len(table), "table must end at the last used block"
                table.append(self._take())
            elif i == 0 and self.ref[table[lb]] > 1:
                src = table[lb]
                dst = self._take()
                self.ref[src] -= 1
                table[lb] = dst
                copies.append((src, dst))
            slots.append(table[lb] * BLOCK_SIZE + off)
        return slots, copies

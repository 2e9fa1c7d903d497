"""The prefix-caching oracle against its pins, and the pins against planted mistakes."""
import collections
import hashlib
import heapq
import struct

import pytest

import oracle.prefix_oracle as P
from tests import prefix_pins as PP


@pytest.mark.parametrize("pin", PP.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _fails(monkeypatch, attr, replacement, pins):
    """With oracle attribute `attr` replaced, at least one of `pins` must fail."""
    with monkeypatch.context() as m:
        m.setattr(P, attr, replacement) if not isinstance(attr, tuple) else \
            m.setattr(attr[0], attr[1], replacement)
        failed = 0
        for pin in pins:
            try:
                pin()
            except (AssertionError, P.OutOfBlocks, KeyError, IndexError):
                failed += 1
        assert failed > 0, f"no pin caught the planted mistake in {attr}"


def test_mutant_keys_without_parent(monkeypatch):
    def key(parent, block_tokens, extras=b""):
        msg = struct.pack("<16i", *[int(t) for t in block_tokens])
        msg += struct.pack("<I", len(extras)) + bytes(extras)
        return hashlib.sha256(msg).digest()
    _fails(monkeypatch, "block_key", key, [PP.pin_a_key_stands_for_the_whole_prefix])


def test_mutant_extras_ignored(monkeypatch):
    orig = P.block_key
    _fails(monkeypatch, "block_key", lambda parent, toks, extras=b"": orig(parent, toks),
           [PP.pin_extras_separate_users])


def test_mutant_partial_block_gets_a_key(monkeypatch):
    def keys(tokens, extras=b"", parent=P.ROOT_KEY):
        out, prev = [], parent
        for b in range((len(tokens) + 15) // 16):
            blk = list(tokens[b * 16:(b + 1) * 16]) + [0] * 16
            prev = P.block_key(prev, blk[:16], extras)
            out.append(prev)
        return out
    _fails(monkeypatch, "block_keys", keys,
           [PP.pin_a_key_stands_for_the_whole_prefix, PP.pin_shared_prefix_3000_tokens])


def test_mutant_release_head_first(monkeypatch):
    def release(self, table):
        for b in table:
            self._drop(b)
    _fails(monkeypatch, (P.PrefixCachingAllocator, "release"), release,
           [PP.pin_eviction_is_lru_and_tail_first])


def test_mutant_evict_before_free(monkeypatch):
    def take(self):
        if self.evictable:
            b, _ = self.evictable.popitem(last=False)
            del self.block_of[self.key_of.pop(b)]
        else:
            b = heapq.heappop(self._free)
        self.ref[b] = 1
        return b
    _fails(monkeypatch, (P.PrefixCachingAllocator, "_take"), take,
           [PP.pin_free_blocks_before_eviction])


def test_mutant_hit_left_in_queue(monkeypatch):
    def match(self, keys):
        hit = []
        for k in keys:
            b = self.block_of.get(k)
            if b is None:
                break
            hit.append(b)
        for b in hit:
            self.ref[b] += 1
        return hit
    _fails(monkeypatch, (P.PrefixCachingAllocator, "match"), match,
           [PP.pin_eviction_is_lru_and_tail_first, PP.pin_random_operations_keep_states])


def test_mutant_free_drops_content(monkeypatch):
    def drop(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                del self.block_of[self.key_of.pop(b)]
            heapq.heappush(self._free, b)
    _fails(monkeypatch, (P.PrefixCachingAllocator, "_drop"), drop,
           [PP.pin_agent_turns_ten_units_not_fifty_five])


def test_mutant_mru_eviction(monkeypatch):
    def take(self):
        if self._free:
            b = heapq.heappop(self._free)
        else:
            b, _ = self.evictable.popitem(last=True)
            del self.block_of[self.key_of.pop(b)]
        self.ref[b] = 1
        return b
    _fails(monkeypatch, (P.PrefixCachingAllocator, "_take"), take,
           [PP.pin_eviction_is_lru_and_tail_first, PP.pin_free_blocks_before_eviction])

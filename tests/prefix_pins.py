"""Pins of the prefix-caching oracle (oracle/prefix_oracle.py) to facts that do not come
from the oracle itself: the serving-engine page's account of block keys and of the
eviction queue (section 4, "prefix cache"), its shared-prefix measurement (a
3,000-token common prefix), the inference-engine page's agent example (10 turns of
prefill: 10 units instead of 55), and brute-force invariants of the block states."""
from __future__ import annotations

import numpy as np

import oracle.prefix_oracle as P


def _tokens(seed: int, n: int) -> list[int]:
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(x) for x in rng.integers(0, 151_936, n)]


def check_states(a: "P.PrefixCachingAllocator", tables: list[list[int]]) -> None:
    """Brute force: each block is held, free or evictable, never two of these; cached
    blocks and keys map one to one; free blocks carry no key, evictable ones do; the
    counts equal the number of live tables naming each block."""
    counts = [0] * a.num_blocks
    for t in tables:
        for b in t:
            counts[b] += 1
    assert counts == a.ref
    free = set(a._free)
    ev = set(a.evictable)
    assert len(free) == len(a._free) and not (free & ev)
    for b in range(a.num_blocks):
        assert (a.ref[b] > 0) + (b in free) + (b in ev) == 1, b
        if b in free:
            assert b not in a.key_of
        if b in ev:
            assert b in a.key_of
    assert {k: b for b, k in a.key_of.items()} == a.block_of
    assert a.num_free() == len(free) + len(ev)


def pin_a_key_stands_for_the_whole_prefix():
    """The same 16 tokens behind different prefixes get different keys; equal
    prefixes give equal keys up to the first differing block and different keys from
    there on; only full blocks get keys."""
    base = _tokens(1, 16 * 6)
    other = list(base)
    other[16 * 2 + 5] += 1                         # change one token of block 2
    ka, kb = P.block_keys(base), P.block_keys(other)
    assert len(ka) == 6
    assert ka[:2] == kb[:2]
    assert all(x != y for x, y in zip(ka[2:], kb[2:]))
    shifted = _tokens(2, 16) + base[16:32]         # block 1 of base behind another block 0
    assert P.block_keys(shifted)[1] != ka[1]
    assert len(P.block_keys(base[:40])) == 2       # 40 tokens: two full blocks
    assert len(P.block_keys(base[:15])) == 0
    assert P.block_keys(base) == P.block_keys(list(base))


def pin_extras_separate_users():
    """A different cache salt (or adapter, or multimodal hash) changes every key."""
    t = _tokens(3, 64)
    k0 = P.block_keys(t, b"salt-A")
    assert k0 == P.block_keys(t, b"salt-A")
    assert all(x != y for x, y in zip(k0, P.block_keys(t, b"salt-B")))
    assert all(x != y for x, y in zip(k0, P.block_keys(t)))


def pin_agent_turns_ten_units_not_fifty_five():
    """The inference-engine page's agent example: 10 turns, each resending the history
    plus one new unit.  With prefix caching only the new unit is prefilled: 10 units in
    all, against 1 + 2 + ... + 10 = 55 without.  (A unit here is 32 tokens.)"""
    unit = 32
    history = _tokens(4, 10 * unit)
    a = P.PrefixCachingAllocator(64)
    with_cache = without = 0
    for turn in range(1, 11):
        prompt = history[:turn * unit]
        keys = P.block_keys(prompt)
        table = a.match(keys)
        cached = len(table) * P.BLOCK_SIZE
        with_cache += len(prompt) - cached
        without += len(prompt)
        a.append(table, cached, len(prompt) - cached)
        a.register(table, keys)
        check_states(a, [table])
        a.release(table)                            # the turn ends; contents are kept
    assert with_cache == 10 * unit
    assert without == 55 * unit


def pin_shared_prefix_3000_tokens():
    """The serving-engine page's measurement: a 3,000-token common prefix with a
    different 32-token tail per request.  The second request finds 187 full blocks,
    2,992 tokens, in the cache (the block straddling the prefix end differs), so only
    40 tokens are prefilled; the shared-prefix decode workload uses the same 187
    blocks."""
    prefix = _tokens(5, 3000)
    a = P.PrefixCachingAllocator(512)
    tables = []
    for r in range(3):
        prompt = prefix + _tokens(100 + r, 32)
        keys = P.block_keys(prompt)
        assert len(keys) == 189
        t = a.match(keys)
        assert len(t) == (0 if r == 0 else 187)
        a.append(t, len(t) * 16, len(prompt) - len(t) * 16)
        a.register(t, keys)
        tables.append(t)
    assert tables[1][:187] == tables[0][:187] == tables[2][:187]
    assert all(a.ref[b] == 3 for b in tables[0][:187])
    check_states(a, tables)


def pin_eviction_is_lru_and_tail_first():
    """A finished request's blocks enter the eviction queue tail first, so when space
    is needed its last block goes first; a hit takes a block out of the queue."""
    a = P.PrefixCachingAllocator(4)
    t = []
    toks = _tokens(6, 64)
    a.append(t, 0, 64)                              # all four blocks
    a.register(t, P.block_keys(toks))
    a.release(t)
    assert list(a.evictable) == [t[3], t[2], t[1], t[0]] and a.num_free() == 4
    hit = a.match(P.block_keys(toks)[:2])           # re-use the first two blocks
    assert hit == t[:2] and list(a.evictable) == [t[3], t[2]]
    u = []
    a.append(u, 0, 17)                              # needs two blocks: evicts t3, t2
    assert u == [t[3], t[2]]
    assert P.block_keys(toks)[3] not in a.block_of and P.block_keys(toks)[2] not in a.block_of
    check_states(a, [hit, u])


def pin_free_blocks_before_eviction():
    """Blocks without cached content are handed out before any cached one is evicted."""
    a = P.PrefixCachingAllocator(6)
    t = []
    toks = _tokens(7, 32)
    a.append(t, 0, 32)                              # blocks 0, 1
    a.register(t, P.block_keys(toks))
    a.release(t)                                    # evictable: 1, 0; free: 2..5
    u = []
    a.append(u, 0, 64)
    assert u == [2, 3, 4, 5] and len(a.evictable) == 2
    w = []
    a.append(w, 0, 1)                               # now evicts the LRU one: block 1
    assert w == [1]
    check_states(a, [u, w])


def pin_match_stops_at_first_miss():
    toks = _tokens(8, 64)
    keys = P.block_keys(toks)
    a = P.PrefixCachingAllocator(8)
    t = []
    a.append(t, 0, 64)
    a.register([t[0], t[2]], [keys[0], keys[2]])    # block 1 not cached
    hit = a.match(keys)
    assert hit == [t[0]]
    check_states(a, [t, hit])


def pin_random_operations_keep_states():
    """Random requests (some sharing prefixes), releases and evictions; the brute-force
    state invariants hold after every operation, and a matched prefix always names
    blocks whose keys are exactly the request's leading keys."""
    rng = np.random.Generator(np.random.PCG64(9))
    prefixes = [_tokens(200 + i, int(rng.integers(16, 200))) for i in range(4)]
    a = P.PrefixCachingAllocator(48)
    live, live_keys = [], []
    for _ in range(300):
        if live and rng.random() < 0.4:
            k = int(rng.integers(0, len(live)))
            a.release(live.pop(k))
            live_keys.pop(k)
        else:
            pre = prefixes[int(rng.integers(0, len(prefixes)))]
            prompt = pre + _tokens(int(rng.integers(0, 10**6)), int(rng.integers(0, 40)))
            keys = P.block_keys(prompt)
            t = a.match(keys)
            assert [a.key_of[b] for b in t] == keys[:len(t)]
            try:
                a.append(t, len(t) * 16, len(prompt) - len(t) * 16)
            except P.OutOfBlocks:
                a.release(t)
                check_states(a, live)
                continue
            a.register(t, keys)
            live.append(t)
            live_keys.append(keys)
        check_states(a, live)


ALL_PINS = [
    pin_a_key_stands_for_the_whole_prefix,
    pin_extras_separate_users,
    pin_agent_turns_ten_units_not_fifty_five,
    pin_shared_prefix_3000_tokens,
    pin_eviction_is_lru_and_tail_first,
    pin_free_blocks_before_eviction,
    pin_match_stops_at_first_miss,
    pin_random_operations_keep_states,
]

"""Pins of the block-bookkeeping oracle (oracle/blocks_oracle.py) to facts that do not
come from the oracle itself: the serving-engine page's account of block sharing
(section 2, "block sharing": reference counts, a copy only when a holder appends),
its block rule (section 2, "blocks and block table": a new block when the current one
is full), counting invariants checked by brute force, and the slot formula of the
input generator, which is written independently of the oracle."""
from __future__ import annotations

import numpy as np

import oracle.blocks_oracle as B


def check_invariants(alloc: "B.RefcountAllocator", tables: list[list[int]],
                     ctx: list[int]) -> None:
    """Brute force: every block's count equals the number of live tables naming it; the
    free blocks are exactly those with count 0; every table holds ceil(ctx/16) blocks
    with no block twice."""
    counts = [0] * alloc.num_blocks
    for t, c in zip(tables, ctx):
        assert len(t) == -(-c // 16), (len(t), c)
        assert len(set(t)) == len(t)
        for b in t:
            counts[b] += 1
    assert counts == alloc.ref, "reference counts differ from table references"
    assert alloc.num_free() == sum(1 for c in counts if c == 0)


def pin_parallel_sampling_shares_then_copies_once_per_holder():
    """Three samples of one 40-token prompt: one table forked twice.  Each sample then
    appends one token into the shared, partly filled third block: the first two
    appenders get private copies (the page: a copy only when a holder appends), the
    last one finds itself the only holder and writes in place.  The two full prompt
    blocks stay shared by all three; 5 blocks hold what 9 would without sharing."""
    a = B.RefcountAllocator(16)
    t0 = []
    slots0, cp = a.append(t0, 0, 40)
    assert cp == [] and t0 == [0, 1, 2]
    assert slots0 == list(range(40))
    t1, t2 = a.fork(t0), a.fork(t0)
    assert a.ref[:3] == [3, 3, 3]
    s1, c1 = a.append(t1, 40, 1)
    s2, c2 = a.append(t2, 40, 1)
    s0, c0 = a.append(t0, 40, 1)
    assert c1 == [(2, 3)] and c2 == [(2, 4)] and c0 == []
    assert s1 == [3 * 16 + 8] and s2 == [4 * 16 + 8] and s0 == [2 * 16 + 8]
    assert t1 == [0, 1, 3] and t2 == [0, 1, 4] and t0 == [0, 1, 2]
    assert a.ref[:5] == [3, 3, 1, 1, 1]
    assert 16 - a.num_free() == 5
    check_invariants(a, [t0, t1, t2], [41, 41, 41])


def pin_new_block_exactly_at_block_boundaries():
    """A fresh block at positions 0, 16, 32, ... and never in between, shared or not;
    a shared table appending at a boundary needs no copy."""
    a = B.RefcountAllocator(8)
    t = []
    for c in range(0, 33):
        before = len(t)
        slots, copies = a.append(t, c, 1)
        assert copies == []
        assert len(t) == before + (1 if c % 16 == 0 else 0)
        assert slots == [t[c // 16] * 16 + c % 16]
    u = a.fork(t)                     # 33 tokens: blocks 0, 1 full, block 2 holds 1
    _, copies = a.append(u, 33, 15)   # fills block 2 of u: one copy, then in place
    assert copies == [(2, 3)] and u == [0, 1, 3]
    _, copies = a.append(u, 48, 1)    # position 48 starts a new block: no copy
    assert copies == [] and u == [0, 1, 3, 4]
    check_invariants(a, [t, u], [33, 49])


def pin_lowest_free_block_first():
    a = B.RefcountAllocator(6)
    t = []
    a.append(t, 0, 16 * 4)
    assert t == [0, 1, 2, 3]
    a.release([t[1], t[3]])
    u = []
    a.append(u, 0, 17)
    assert u == [1, 3]
    w = []
    a.append(w, 0, 1)
    assert w == [4]


def pin_out_of_blocks_changes_nothing():
    a = B.RefcountAllocator(4)
    t = []
    a.append(t, 0, 50)                # 4 blocks: the pool is full
    u = a.fork(t)
    ref_before, t_before, u_before = list(a.ref), list(t), list(u)
    for ctx_new in (1, 14):           # a copy of the last block is needed: no room
        try:
            a.append(u, 50, ctx_new)
        except B.OutOfBlocks:
            pass
        else:
            raise AssertionError("append past the pool did not fail")
        assert a.ref == ref_before and t == t_before and u == u_before


def pin_release_returns_everything():
    rng = np.random.Generator(np.random.PCG64(11))
    a = B.RefcountAllocator(64)
    tables, ctx = [], []
    for _ in range(6):
        t = []
        n = int(rng.integers(1, 60))
        a.append(t, 0, n)
        tables.append(t)
        ctx.append(n)
    for k in range(3):
        tables.append(a.fork(tables[k]))
        ctx.append(ctx[k])
    for k in range(len(tables)):
        add = int(rng.integers(0, 20))
        a.append(tables[k], ctx[k], add)
        ctx[k] += add
    check_invariants(a, tables, ctx)
    for t in tables:
        a.release(t)
    assert a.num_free() == 64 and a.ref == [0] * 64


def pin_random_operations_keep_invariants():
    """Random forks, appends and releases; the brute-force counts hold after each."""
    rng = np.random.Generator(np.random.PCG64(5))
    a = B.RefcountAllocator(96)
    tables, ctx = [], []
    for _ in range(400):
        op = rng.integers(0, 4)
        if op == 0 or not tables:
            t = []
            n = int(rng.integers(1, 40))
            try:
                a.append(t, 0, n)
            except B.OutOfBlocks:
                continue
            tables.append(t)
            ctx.append(n)
        elif op == 1:
            k = int(rng.integers(0, len(tables)))
            tables.append(a.fork(tables[k]))
            ctx.append(ctx[k])
        elif op == 2:
            k = int(rng.integers(0, len(tables)))
            add = int(rng.integers(1, 24))
            try:
                a.append(tables[k], ctx[k], add)
                ctx[k] += add
            except B.OutOfBlocks:
                pass
        else:
            k = int(rng.integers(0, len(tables)))
            a.release(tables.pop(k))
            ctx.pop(k)
        check_invariants(a, tables, ctx)


def pin_slots_match_the_generators_formula():
    """The slots an append hands out equal the slot mapping the input generator builds
    from its own table (written independently of this oracle): a request holding the
    generator's first five blocks appends positions 70..78."""
    import heapq

    from workloads import make_batch
    rng = np.random.Generator(np.random.PCG64(0))
    b = make_batch(rng, name="s", dtype="f32", num_q_heads=2, num_kv_heads=1, head_dim=64,
                   num_blocks=40, context_lens=[79], query_lens=[9])
    t = [int(x) for x in b.block_tables[0, :5]]
    a = B.RefcountAllocator(40)
    for blk in t:
        a.ref[blk] = 1
        a._free.remove(blk)
    heapq.heapify(a._free)
    slots, copies = a.append(t, 70, 9)
    assert copies == []
    assert slots == [int(x) for x in b.slot_mapping]


def pin_copy_makes_private_equal_to_shared():
    """After a copy, gathering the copied request's keys through its new table gives
    exactly what the shared table gave; no other block changes."""
    rng = np.random.Generator(np.random.PCG64(3))
    nb, hkv, d = 12, 2, 8
    kp = rng.standard_normal((nb, hkv, 16, d)).astype(np.float32)
    vp = rng.standard_normal((nb, hkv, 16, d)).astype(np.float32)
    a = B.RefcountAllocator(nb)
    t = []
    a.append(t, 0, 37)
    u = a.fork(t)
    _, copies = a.append(u, 37, 1)
    kp2, vp2 = B.copy_blocks(kp, vp, copies)
    for pos in range(37):
        lb, off = divmod(pos, 16)
        assert np.array_equal(kp2[u[lb], :, off], kp[t[lb], :, off])
        assert np.array_equal(vp2[u[lb], :, off], vp[t[lb], :, off])
    touched = {dst for _, dst in copies}
    for blk in range(nb):
        if blk not in touched:
            assert np.array_equal(kp2[blk], kp[blk]) and np.array_equal(vp2[blk], vp[blk])
        else:
            assert np.array_equal(kp2[blk], kp[copies[0][0]])


ALL_PINS = [
    pin_parallel_sampling_shares_then_copies_once_per_holder,
    pin_new_block_exactly_at_block_boundaries,
    pin_lowest_free_block_first,
    pin_out_of_blocks_changes_nothing,
    pin_release_returns_everything,
    pin_random_operations_keep_invariants,
    pin_slots_match_the_generators_formula,
    pin_copy_makes_private_equal_to_shared,
]

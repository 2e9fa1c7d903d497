"""Pins that tie the CPU oracle to something other than itself.

Each `pin_*` function raises AssertionError when the oracle disagrees with:
  * a brute-force pure-Python evaluation on tiny inputs (own slot arithmetic, own
    bf16 decoding, math.exp / math.fsum),
  * a library routine for a textbook special case (torch fp64 scaled-dot-product
    attention with an explicit mask and repeated KV heads),
  * closed forms (one key, constant V rows, zero query, two keys, a one-hot probe),
  * invariants stated on the pages (permuting physical blocks, shared == private
    blocks, paged == contiguous, chunking, stale slots),
  * values printed on the pages (tests/golden/pages_facts.json).
The functions are plain (not pytest tests) so that the mutation tests can run all of
them against deliberately broken copies of the oracle.
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np

import oracle.pagedkv_oracle as O
from workloads import make_batch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def _facts():
    with open(GOLDEN) as f:
        return json.load(f)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------------------
# brute force (independent arithmetic)
# ---------------------------------------------------------------------------

def _bf16_scalar(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _scalar(raw, dtype) -> float:
    return _bf16_scalar(raw) if dtype == "bf16" else float(raw)


def brute_force(batch, k_pool, v_pool):
    """Pure-Python attention reading the pool through flat slots."""
    hq, hkv, d = batch.num_q_heads, batch.num_kv_heads, batch.head_dim
    nb = k_pool.shape[0]
    kflat = k_pool.transpose(0, 2, 1, 3).reshape(nb * 16, hkv, d)
    vflat = v_pool.transpose(0, 2, 1, 3).reshape(nb * 16, hkv, d)
    out = np.zeros((batch.total_q, hq, d))
    for s in range(batch.num_seqs):
        a, b = int(batch.query_start_loc[s]), int(batch.query_start_loc[s + 1])
        c = int(batch.context_lens[s])
        for i in range(b - a):
            last = c - (b - a) + i          # newest key this row may see
            for h in range(hq):
                g = h * hkv // hq           # KV head: heads are grouped in order
                logits = []
                for j in range(last + 1):
                    slot = int(batch.block_tables[s][j // 16]) * 16 + (j % 16)
                    dot = math.fsum(_scalar(batch.q[a + i, h, e], batch.dtype)
                                    * _scalar(kflat[slot, g, e], batch.dtype)
                                    for e in range(d))
                    logits.append(batch.scale * dot)
                top = max(logits)
                lse = top + math.log(math.fsum(math.exp(x - top) for x in logits))
                for e in range(d):
                    acc = []
                    for j in range(last + 1):
                        slot = int(batch.block_tables[s][j // 16]) * 16 + (j % 16)
                        acc.append(math.exp(logits[j] - lse)
                                   * _scalar(vflat[slot, g, e], batch.dtype))
                    out[a + i, h, e] = math.fsum(acc)
    return out


def _tiny_batch(seed, dtype):
    rng = _rng(seed)
    return make_batch(rng, name="tiny", dtype=dtype, num_q_heads=4, num_kv_heads=2,
                      head_dim=8, num_blocks=24, context_lens=[1, 16, 17, 40, 33],
                      query_lens=[1, 3, 1, 17, 33], stale="nan")


def pin_brute_force():
    for seed, dtype in ((0, "f32"), (1, "bf16"), (2, "f32")):
        b = _tiny_batch(seed, dtype)
        kp, vp, out = O.step(b)
        ref = brute_force(b, kp, vp)
        err = np.abs(out - ref).max()
        assert err <= 1e-12, f"brute force mismatch {err} ({dtype}, seed {seed})"


# ---------------------------------------------------------------------------
# library special case: torch fp64 SDPA on contiguous K/V
# ---------------------------------------------------------------------------

def pin_library_sdpa():
    import torch

    rng = _rng(7)
    hq, hkv, d = 8, 2, 32
    for ctx, qn in ((300, 1), (300, 45), (129, 129)):
        q = rng.standard_normal((qn, hq, d))
        K = rng.standard_normal((ctx, hkv, d))
        V = rng.standard_normal((ctx, hkv, d))
        scale = 0.3
        got = O.attention_contiguous(q, K, V, scale, np.arange(ctx - qn, ctx))
        rep = hq // hkv
        tq = torch.from_numpy(q).permute(1, 0, 2)[None]
        tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(rep, 0)[None]
        tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(rep, 0)[None]
        # bottom-right causal: row i may see key j iff j <= ctx - qn + i
        allow = torch.ones(qn, ctx, dtype=torch.bool).tril(diagonal=ctx - qn)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.contiguous(), tv.contiguous(), attn_mask=allow, scale=scale)
        ref = ref[0].permute(1, 0, 2).numpy()
        err = np.abs(got - ref).max()
        assert err <= 1e-12, f"sdpa mismatch {err} at ctx={ctx} q={qn}"


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def pin_single_key():
    rng = _rng(3)
    q = rng.standard_normal((1, 4, 16))
    K = rng.standard_normal((1, 2, 16))
    V = rng.standard_normal((1, 2, 16))
    out = O.attention_contiguous(q, K, V, 0.25, [0])
    for h in range(4):
        assert np.array_equal(out[0, h], V[0, h // 2]), "one key must return its V row"


def pin_constant_values():
    rng = _rng(4)
    ctx, qn = 37, 5
    q = rng.standard_normal((qn, 4, 16))
    K = rng.standard_normal((ctx, 2, 16))
    u = rng.standard_normal((2, 16))
    V = np.broadcast_to(u, (ctx, 2, 16)).copy()
    out = O.attention_contiguous(q, K, V, 0.7, np.arange(ctx - qn, ctx))
    for h in range(4):
        assert np.abs(out[:, h] - u[h // 2]).max() <= 1e-13, "constant V rows"


def pin_zero_query_mean():
    rng = _rng(5)
    ctx, qn = 23, 4
    q = np.zeros((qn, 2, 8))
    K = rng.standard_normal((ctx, 1, 8))
    V = rng.standard_normal((ctx, 1, 8))
    pos = np.arange(ctx - qn, ctx)
    out = O.attention_contiguous(q, K, V, 1.0, pos)
    for i in range(qn):
        mean = V[: pos[i] + 1, 0].mean(axis=0)
        assert np.abs(out[i, 0] - mean).max() <= 1e-13, "zero query -> mean of seen V"


def pin_two_keys_logistic():
    rng = _rng(6)
    q = rng.standard_normal((1, 1, 8))
    K = rng.standard_normal((2, 1, 8))
    V = rng.standard_normal((2, 1, 8))
    scale = 0.9
    out = O.attention_contiguous(q, K, V, scale, [1])
    delta = scale * float(np.dot(q[0, 0], K[0, 0] - K[1, 0]))
    w0 = 1.0 / (1.0 + math.exp(-delta))        # logistic of the score gap
    want = w0 * V[0, 0] + (1.0 - w0) * V[1, 0]
    assert np.abs(out[0, 0] - want).max() <= 1e-14, "two-key logistic form"


def pin_one_hot_probe():
    """Huge scale + a unique best key: the output is that key's V row, bit for bit."""
    rng = _rng(8)
    for target in (0, 15, 16, 31, 47, 52):
        b = make_batch(rng, name="probe", dtype="bf16", num_q_heads=2, num_kv_heads=1,
                       head_dim=8, num_blocks=12, context_lens=[53], query_lens=[1])
        # q = e0; key j's first coordinate is -|j - target| (exact in bf16)
        qf = np.zeros((1, 2, 8), np.float32)
        qf[0, :, 0] = 1.0
        from workloads import bf16_round_bits
        b.q = bf16_round_bits(qf)
        kp, vp = O.kv_write(b.k_pool, b.v_pool, b.k_new, b.v_new, b.slot_mapping)
        for j in range(53):
            blk = int(b.block_tables[0][j // 16])
            kp[blk, 0, j % 16, :] = bf16_round_bits(np.array([-abs(j - target)] + [0.0] * 7,
                                                             np.float32))
        b.scale = 1.0e4
        out = O.paged_attention(b.q, kp, vp, b.block_tables, b.context_lens,
                                b.query_start_loc, b.scale, b.dtype)
        blk = int(b.block_tables[0][target // 16])
        want = O.to_f64(vp[blk, 0, target % 16], "bf16")
        for h in range(2):
            assert np.array_equal(out[0, h], want), f"one-hot probe at key {target}"


# ---------------------------------------------------------------------------
# invariants from the pages
# ---------------------------------------------------------------------------

def _mixed(seed, dtype="bf16", stale="random", **kw):
    args = dict(name="mixed", dtype=dtype, num_q_heads=8, num_kv_heads=2, head_dim=16,
                num_blocks=96, context_lens=[70, 1, 129, 33, 16],
                query_lens=[1, 1, 40, 33, 0], stale=stale)
    args.update(kw)
    return make_batch(_rng(seed), **args)


def pin_block_permutation():
    b = _mixed(11)
    kp, vp, out = O.step(b)
    perm = _rng(99).permutation(b.num_blocks)
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    tables2 = np.where(b.block_tables >= 0, perm[np.maximum(b.block_tables, 0)], -1)
    out2 = O.paged_attention(b.q, kp2, vp2, tables2.astype(np.int32), b.context_lens,
                             b.query_start_loc, b.scale, b.dtype)
    assert np.array_equal(out, out2), "relabelling physical blocks changed the output"


def pin_shared_equals_private():
    rng = _rng(12)
    b = make_batch(rng, name="share", dtype="bf16", num_q_heads=4, num_kv_heads=2,
                   head_dim=16, num_blocks=64, context_lens=[70, 75, 90],
                   query_lens=[1, 1, 1], shared_prefix_blocks=4)
    kp, vp, out = O.step(b)
    # private copies of the 4 shared blocks for sequences 1 and 2
    tables = b.block_tables.copy()
    used = set(int(x) for x in tables.ravel() if x >= 0)
    free = [x for x in range(b.num_blocks) if x not in used]
    kp2, vp2 = kp.copy(), vp.copy()
    for s in (1, 2):
        for lb in range(4):
            dst = free.pop()
            kp2[dst] = kp[tables[s, lb]]
            vp2[dst] = vp[tables[s, lb]]
            tables[s, lb] = dst
    out2 = O.paged_attention(b.q, kp2, vp2, tables, b.context_lens, b.query_start_loc,
                             b.scale, b.dtype)
    assert np.array_equal(out, out2), "shared blocks differ from private copies"


def pin_paged_equals_contiguous():
    rng = _rng(13)
    hq, hkv, d, ctx, qn = 4, 2, 16, 45, 6
    K = rng.standard_normal((ctx, hkv, d))
    V = rng.standard_normal((ctx, hkv, d))
    q = rng.standard_normal((qn, hq, d))
    want = O.attention_contiguous(q, K, V, 0.5, np.arange(ctx - qn, ctx))
    nb = 10
    kp = rng.standard_normal((nb, hkv, 16, d))
    vp = rng.standard_normal((nb, hkv, 16, d))
    table = rng.permutation(nb)[:3].astype(np.int32)
    for j in range(ctx):      # scatter the contiguous cache into pool slots
        kp[table[j // 16], :, j % 16] = K[j]
        vp[table[j // 16], :, j % 16] = V[j]
    got = O.paged_attention(q.astype(np.float32).astype(np.float64), kp, vp,
                            table[None], np.array([ctx]), np.array([0, qn]), 0.5, "f32")
    # pools were built in float64; compare through the float32 storage path
    want32 = O.attention_contiguous(
        q.astype(np.float32).astype(np.float64), K.astype(np.float32).astype(np.float64),
        V.astype(np.float32).astype(np.float64), 0.5, np.arange(ctx - qn, ctx))
    assert np.array_equal(got, want32), "paged result differs from contiguous"
    assert np.abs(want - want32).max() < 1e-5


def pin_chunking():
    """Chunk [a, b) over context b == rows a..b-1 of one-shot prefill over [0, b)."""
    rng = _rng(14)
    hq, hkv, d, n = 4, 2, 16, 90
    K = rng.standard_normal((n, hkv, d))
    V = rng.standard_normal((n, hkv, d))
    q = rng.standard_normal((n, hq, d))
    full = O.attention_contiguous(q, K, V, 0.4, O.query_positions(n, n))
    for a, b in ((0, 32), (32, 64), (64, 90), (50, 51), (89, 90)):
        part = O.attention_contiguous(q[a:b], K[:b], V[:b], 0.4, O.query_positions(b, b - a))
        assert np.abs(part - full[a:b]).max() <= 1e-13, f"chunk [{a},{b}) differs"
    dec = O.attention_contiguous(q[n - 1:n], K, V, 0.4, O.query_positions(n, 1))
    assert np.abs(dec[0] - full[n - 1]).max() <= 1e-13, "decode != last prefill row"


def pin_gqa_equals_repeated_heads():
    b = _mixed(15)
    kp, vp, out = O.step(b)
    rep = b.num_q_heads // b.num_kv_heads
    kp2 = np.repeat(kp, rep, axis=1)
    vp2 = np.repeat(vp, rep, axis=1)
    out2 = O.paged_attention(b.q, kp2, vp2, b.block_tables, b.context_lens,
                             b.query_start_loc, b.scale, b.dtype)
    assert np.array_equal(out, out2), "GQA differs from repeated KV heads"


def pin_stale_slots_ignored():
    b1 = _mixed(16, stale="random")
    b2 = _mixed(16, stale="nan")
    o1 = O.step(b1)[2]
    o2 = O.step(b2)[2]
    assert not np.isnan(o2).any(), "NaN from a stale slot reached the output"
    assert np.array_equal(o1, o2), "stale slot contents changed the output"


def pin_write_gather_roundtrip():
    for dtype in ("f32", "bf16"):
        b = _mixed(17, dtype=dtype)
        kp, vp = O.kv_write(b.k_pool, b.v_pool, b.k_new, b.v_new, b.slot_mapping)
        for s in range(b.num_seqs):
            a, e = int(b.query_start_loc[s]), int(b.query_start_loc[s + 1])
            c = int(b.context_lens[s])
            kg = O.gather(kp, b.block_tables[s], c)
            vg = O.gather(vp, b.block_tables[s], c)
            # the new tokens are the last q_len positions of the sequence
            assert kg[c - (e - a):].tobytes() == b.k_new[a:e].tobytes(), "K round trip"
            assert vg[c - (e - a):].tobytes() == b.v_new[a:e].tobytes(), "V round trip"
        # slot 0 is written, a negative slot is skipped, nothing else changes
        kp2, vp2 = O.kv_write(b.k_pool, b.v_pool, b.k_new[:2], b.v_new[:2],
                              np.array([0, -1], np.int32))
        assert kp2[0, :, 0].tobytes() == b.k_new[0].tobytes(), "slot 0 not written"
        assert vp2[0, :, 0].tobytes() == b.v_new[0].tobytes(), "slot 0 not written"
        changed = (kp2.view(np.uint8) != b.k_pool.view(np.uint8)).sum()
        assert changed <= b.k_new[0].nbytes, "write touched more than one slot"


# ---------------------------------------------------------------------------
# values printed on the pages
# ---------------------------------------------------------------------------

def pin_pages_chunk_boundaries():
    """The pages' 8K prompt / 2K budget example: each chunk's rows sit at its slice."""
    f = _facts()
    assert O.BLOCK_SIZE == f["block_size"]["value"]
    ex = f["chunked_prefill_8k_prompt_2k_budget"]
    for lo, hi in ex["chunks_inclusive"]:
        pos = O.query_positions(hi + 1, hi - lo + 1)    # context so far = hi + 1 keys
        assert pos[0] == lo and pos[-1] == hi and len(pos) == ex["budget"]


def pin_pages_block_waste():
    """Waste is below one block: a context of c keys occupies ceil(c/16) table rows."""
    f = _facts()
    maxw = f["last_block_waste_below_block_size"]["max_wasted_slots"]
    rng = _rng(18)
    lens = [1, 15, 16, 17, 31, 32, 33, 100]
    b = make_batch(rng, name="waste", dtype="f32", num_q_heads=1, num_kv_heads=1,
                   head_dim=4, num_blocks=40, context_lens=lens, query_lens=[1] * len(lens))
    for s, c in enumerate(lens):
        nrows = int((b.block_tables[s] >= 0).sum())
        assert 0 <= nrows * 16 - c <= maxw
        O.gather(b.k_pool, b.block_tables[s], c)    # reads only the used rows


ALL_PINS = [
    pin_brute_force, pin_library_sdpa, pin_single_key, pin_constant_values,
    pin_zero_query_mean, pin_two_keys_logistic, pin_one_hot_probe,
    pin_block_permutation, pin_shared_equals_private, pin_paged_equals_contiguous,
    pin_chunking, pin_gqa_equals_repeated_heads, pin_stale_slots_ignored,
    pin_write_gather_roundtrip, pin_pages_chunk_boundaries, pin_pages_block_waste,
]

"""CPU oracle for attention over a paged KV cache (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
this module: only the tests, the smoke check and the benchmark's CPU-baseline leg use
it.  It shares no code with the HIP library.

What it computes, and where that is defined (pages cited by title and section):

* Serving-engine KV page (ttlab, "LLM KV cache 02"), section 2 "PagedAttention: split
  KV into blocks", subsection "blocks and block table": K/V are cut into fixed
  16-token blocks; every request keeps a logical-block -> physical-block table; blocks
  may sit anywhere in the pool; a fresh block is taken when the current one fills; and
  the attention kernel, walking the table over scattered blocks, must give the same
  result as a contiguous array.  So the oracle is that plain definition: gather each
  sequence's K/V through its table into a contiguous array (`gather`), then run
  ordinary softmax attention on it (`attention_contiguous`).
* Same page, subsection "block sharing": several tables may name the same physical
  block.  `gather` reads through the table, so sharing needs no special case.
* "How inference engines actually work" page (xiaohu-jiedu), section on the KV cache:
  each step computes only the new token's K/V column and reads the past ones from the
  cache.  So a step first writes the new K/V into the pool (`kv_write`), then attends
  over all keys including the new ones.
* Same page, "Chunked Prefill" subsection: a long prompt is processed as consecutive
  slices over several passes, each slice following the already-processed positions.
  So a query chunk of length q over a context of c keys holds positions c-q .. c-1,
  and row i sees keys 0 .. c-q+i (bottom-right causal alignment, `query_positions`).

Readings where the pages are silent (each also listed in the design notes):
* Pool layout [num_blocks][num_kv_heads][16][head_dim]; flat slot = block*16 + offset.
* A negative slot in the write means "skip this token".
* Grouped-query attention: query head h reads KV head h // (Hq / Hkv).
* Softmax is the plain max-subtracted one with a caller-given scale; no masks other
  than the causal one.
* bf16 values are exact in fp64; the oracle computes in fp64 throughout.
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


# ---------------------------------------------------------------------------
# element decoding (bf16 values are carried as uint16 bit patterns)
# ---------------------------------------------------------------------------

def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage -> float64.  bf16: the 16 bits are the top half of a float32."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# O1: the slot write (bit copy)
# ---------------------------------------------------------------------------

def locate(slot: int) -> tuple[int, int]:
    """Flat pool slot -> (physical block, offset inside the block)."""
    return slot // BLOCK_SIZE, slot % BLOCK_SIZE


def kv_write(k_pool, v_pool, k_new, v_new, slot_mapping):
    """Copy each new token's K/V rows into its pool slot; returns new pools.

    Tokens are applied in order; a negative slot is skipped.  The copy is of raw
    storage, so it is bit-exact by construction.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = locate(int(slot))
        k_out[blk, :, off, :] = k_new[t]
        v_out[blk, :, off, :] = v_new[t]
    return k_out, v_out


# ---------------------------------------------------------------------------
# O2: the block-table gather
# ---------------------------------------------------------------------------

def table_lookup(table_row, pos: int) -> tuple[int, int]:
    """Logical token position -> (physical block, offset) through one table row."""
    return int(table_row[pos // BLOCK_SIZE]), pos % BLOCK_SIZE


def gather(pool, table_row, ctx: int) -> np.ndarray:
    """Contiguous [ctx, num_kv_heads, head_dim] copy (raw storage) of one sequence."""
    out = np.empty((ctx, pool.shape[1], pool.shape[3]), dtype=pool.dtype)
    for j in range(ctx):
        blk, off = table_lookup(table_row, j)
        out[j] = pool[blk, :, off, :]
    return out


# ---------------------------------------------------------------------------
# O3: attention over a contiguous cache
# ---------------------------------------------------------------------------

def kv_head_of(h: int, group: int) -> int:
    """Grouped-query mapping: consecutive query heads share one KV head."""
    return h // group


def query_positions(ctx: int, q_len: int) -> np.ndarray:
    """Positions of a query chunk's rows: the last q_len positions of the context."""
    return np.arange(ctx - q_len, ctx, dtype=np.int64)


def softmax_rows(scores: np.ndarray) -> np.ndarray:
    """Row-wise softmax; -inf entries get weight 0."""
    m = scores.max(axis=1, keepdims=True)
    w = np.exp(scores - m)
    return w / w.sum(axis=1, keepdims=True)


def attention_contiguous(q, K, V, scale: float, positions) -> np.ndarray:
    """Causal softmax attention on contiguous float64 K/V.

    q [rows, Hq, d], K/V [ctx, Hkv, d], positions [rows]: row r sees keys
    0 .. positions[r].  Returns float64 [rows, Hq, d].
    """
    rows, hq, d = q.shape
    ctx, hkv, _ = K.shape
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    positions = np.asarray(positions, dtype=np.int64)
    if rows and (positions.min() < 0 or positions.max() >= ctx):
        raise ValueError("query position outside the context")
    group = hq // hkv
    hidden = np.arange(ctx)[None, :] > positions[:, None]
    out = np.zeros((rows, hq, d), dtype=np.float64)
    for h in range(hq):
        kvh = kv_head_of(h, group)
        s = (q[:, h, :] @ K[:, kvh, :].T) * scale
        s[hidden] = -np.inf
        out[:, h, :] = softmax_rows(s) @ V[:, kvh, :]
    return out


def paged_attention(q, k_pool, v_pool, block_tables, context_lens, query_start_loc,
                    scale: float, dtype: str) -> np.ndarray:
    """Varlen paged attention: per sequence, gather through the table, then attend.

    q [total_q, Hq, d] raw; pools [num_blocks, Hkv, 16, d] raw; block_tables int32
    [num_seqs, max_blocks]; context_lens [num_seqs]; query_start_loc [num_seqs+1].
    Returns float64 [total_q, Hq, d].
    """
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    ctxs = np.asarray(context_lens, dtype=np.int64)
    total_q = int(qsl[-1])
    out = np.zeros((total_q,) + tuple(q.shape[1:]), dtype=np.float64)
    for s in range(ctxs.shape[0]):
        a, b = int(qsl[s]), int(qsl[s + 1])
        q_len, ctx = b - a, int(ctxs[s])
        if q_len == 0:
            continue
        if q_len > ctx:
            raise ValueError(f"sequence {s}: {q_len} queries but {ctx} keys")
        K = to_f64(gather(k_pool, block_tables[s], ctx), dtype)
        V = to_f64(gather(v_pool, block_tables[s], ctx), dtype)
        out[a:b] = attention_contiguous(to_f64(q[a:b], dtype), K, V, scale,
                                        query_positions(ctx, q_len))
    return out


def step(batch):
    """One engine step on a `PagedBatch`: slot write, then varlen paged attention.

    Returns (k_pool_after, v_pool_after, out_f64).
    """
    k_pool, v_pool = kv_write(batch.k_pool, batch.v_pool, batch.k_new, batch.v_new,
                              batch.slot_mapping)
    out = paged_attention(batch.q, k_pool, v_pool, batch.block_tables,
                          batch.context_lens, batch.query_start_loc, batch.scale,
                          batch.dtype)
    return k_pool, v_pool, out

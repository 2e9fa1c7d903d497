"""Seeded synthetic batches shaped like the paged-KV attention workloads.

Every batch is one engine step over a paged KV pool: each sequence already owns a run
of 16-token physical blocks reached through its row of the block table, and this step
brings `q_len` new tokens per sequence (1 for decode, more for a prefill chunk).  The
new tokens' K/V (`k_new`, `v_new`) are written into the pool at `slot_mapping`, after
which attention runs over `context_lens` keys (the counts include the new tokens).

Only random draws and bookkeeping live here (lengths, a shuffled block order, N(0, 1)
values, the flat slot index of each new token).  No attention arithmetic is done.

Layouts (all C-contiguous):
  k_pool, v_pool   [num_blocks, num_kv_heads, 16, head_dim]
  block_tables     int32 [num_seqs, max_blocks_per_seq]; unused entries are -1
  context_lens     int32 [num_seqs]
  query_start_loc  int32 [num_seqs + 1], query_start_loc[0] == 0
  q                [total_q, num_q_heads, head_dim]
  k_new, v_new     [total_q, num_kv_heads, head_dim]
  slot_mapping     int32 [total_q]
Element storage: "f32" arrays are float32; "bf16" arrays are uint16 bit patterns of
bfloat16 values obtained from float32 N(0, 1) draws by round-to-nearest-even.

Draw order for one batch (fixed, so a seed names one batch): the config's lengths,
then the block permutation, then q, the K pool, the V pool, k_new, v_new.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK_SIZE = 16

CONFIG_NAMES = (
    "tiny_f32_decode",
    "llama32_1b_decode",
    "qwen3_1p7b_decode_640",
    "shared_prefix_decode",
    "chunked_prefill_mixed",
)


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even.

    Uses torch's CPU float32->bfloat16 cast (IEEE RNE) as a data-preparation step.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@dataclasses.dataclass
class PagedBatch:
    name: str
    dtype: str  # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    query_start_loc: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    slot_mapping: np.ndarray
    scale: float
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int32)

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_round_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def _nan_value(dtype: str):
    return np.float32("nan") if dtype == "f32" else np.uint16(0x7FC0)


def make_batch(
    rng: np.random.Generator,
    *,
    name: str,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    num_blocks: int,
    context_lens,
    query_lens,
    shared_prefix_blocks: int = 0,
    max_blocks_per_seq: int | None = None,
    stale: str = "random",
    scale: float | None = None,
) -> PagedBatch:
    """Build one paged batch.

    Physical blocks come from one seeded permutation of the pool, taken in order, so no
    two sequences share a block unless `shared_prefix_blocks` > 0, in which case the
    first that many permutation entries are the leading table entries of every row.
    `stale="nan"` fills every pool slot that holds no token of this batch with NaN.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(query_lens, dtype=np.int64)
    n = int(ctx.shape[0])
    if ql.shape != ctx.shape:
        raise ValueError("context_lens and query_lens differ in length")
    if np.any(ql > ctx) or np.any(ql < 0):
        raise ValueError("need 0 <= q_len <= context_len")
    nblk = [(int(c) + BLOCK_SIZE - 1) // BLOCK_SIZE for c in ctx]
    if shared_prefix_blocks and any(b < shared_prefix_blocks for b in nblk):
        raise ValueError("a sequence is shorter than the shared prefix")
    width = max(nblk) if n else 1
    if max_blocks_per_seq is not None:
        if max_blocks_per_seq < width:
            raise ValueError("max_blocks_per_seq too small")
        width = max_blocks_per_seq
    width = max(width, 1)
    need = shared_prefix_blocks + sum(b - shared_prefix_blocks for b in nblk)
    if need > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {need}")

    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((n, width), -1, dtype=np.int32)
    cursor = shared_prefix_blocks
    for s in range(n):
        tables[s, :shared_prefix_blocks] = perm[:shared_prefix_blocks]
        own = nblk[s] - shared_prefix_blocks
        tables[s, shared_prefix_blocks:nblk[s]] = perm[cursor:cursor + own]
        cursor += own

    qsl = np.zeros(n + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(ql)
    total_q = int(qsl[-1])

    q = _draw_values(rng, (total_q, num_q_heads, head_dim), dtype)
    pool_shape = (num_blocks, num_kv_heads, BLOCK_SIZE, head_dim)
    k_pool = _draw_values(rng, pool_shape, dtype)
    v_pool = _draw_values(rng, pool_shape, dtype)
    k_new = _draw_values(rng, (total_q, num_kv_heads, head_dim), dtype)
    v_new = _draw_values(rng, (total_q, num_kv_heads, head_dim), dtype)

    # Flat pool slot of each new token: the scheduler's bookkeeping, an input to the
    # write.  New tokens are the last q_len positions of each sequence.
    slots = np.empty(total_q, dtype=np.int32)
    for s in range(n):
        for i in range(int(ql[s])):
            pos = int(ctx[s]) - int(ql[s]) + i
            slots[qsl[s] + i] = tables[s, pos // BLOCK_SIZE] * BLOCK_SIZE + pos % BLOCK_SIZE

    if stale == "nan":
        used = np.zeros((num_blocks, BLOCK_SIZE), dtype=bool)
        for s in range(n):
            for j in range(int(ctx[s])):
                used[tables[s, j // BLOCK_SIZE], j % BLOCK_SIZE] = True
        nanv = _nan_value(dtype)
        k_pool.transpose(0, 2, 1, 3)[~used] = nanv
        v_pool.transpose(0, 2, 1, 3)[~used] = nanv
    elif stale != "random":
        raise ValueError(f"unknown stale mode {stale!r}")

    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return PagedBatch(
        name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, num_blocks=num_blocks, k_pool=k_pool, v_pool=v_pool,
        block_tables=tables, context_lens=ctx.astype(np.int32), query_start_loc=qsl,
        q=q, k_new=k_new, v_new=v_new, slot_mapping=slots, scale=float(scale),
        meta={"shared_prefix_blocks": shared_prefix_blocks},
    )


def make_config(name: str, seed: int = 0, *, stale: str = "random") -> PagedBatch:
    """The five named workloads, each drawn from `numpy.random.Generator(PCG64(seed))`.

    Uniform integer ranges are inclusive of both ends.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "tiny_f32_decode":
        ctx = [5, 17, 33, 64]
        return make_batch(rng, name=name, dtype="f32", num_q_heads=4, num_kv_heads=2,
                          head_dim=64, num_blocks=64, context_lens=ctx,
                          query_lens=[1] * 4, stale=stale)
    if name == "llama32_1b_decode":
        ctx = rng.integers(128, 2048, size=32, endpoint=True)
        return make_batch(rng, name=name, dtype="bf16", num_q_heads=32, num_kv_heads=8,
                          head_dim=64, num_blocks=8192, context_lens=ctx,
                          query_lens=[1] * 32, stale=stale)
    if name == "qwen3_1p7b_decode_640":
        ctx = rng.integers(512, 640, size=34, endpoint=True)
        return make_batch(rng, name=name, dtype="bf16", num_q_heads=16, num_kv_heads=8,
                          head_dim=128, num_blocks=1378, context_lens=ctx,
                          query_lens=[1] * 34, stale=stale)
    if name == "shared_prefix_decode":
        gen = rng.integers(0, 128, size=32, endpoint=True)
        ctx = 187 * BLOCK_SIZE + 40 + gen
        return make_batch(rng, name=name, dtype="bf16", num_q_heads=16, num_kv_heads=8,
                          head_dim=128, num_blocks=1378, context_lens=ctx,
                          query_lens=[1] * 32, shared_prefix_blocks=187, stale=stale)
    if name == "chunked_prefill_mixed":
        dec = rng.integers(300, 4096, size=31, endpoint=True)
        ctx = np.concatenate([[3500], dec])
        ql = np.concatenate([[2017], np.ones(31, dtype=np.int64)])
        return make_batch(rng, name=name, dtype="bf16", num_q_heads=16, num_kv_heads=8,
                          head_dim=128, num_blocks=8192, context_lens=ctx,
                          query_lens=ql, stale=stale)
    raise KeyError(f"unknown config {name!r}; known: {CONFIG_NAMES}")

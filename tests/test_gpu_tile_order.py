"""GPU parity for batches of many prefill chunks.

The chunk kernel numbers the row tiles of all chunk sequences densely (a sequence of
q >= 2 query rows has ceil(q / BM) of them, BM = 64 rows with two query heads per kv
head and 32 with four) and finds each tile's sequence with a scan over the query
offsets, every thread of the workgroup counting a run of sequences.  The cases: many
equal 64-row chunks over shared blocks (each chunk exactly one row tile); chunks of
every length class around the tile size between decode rows and empty sequences
(q = 0); more than 512 sequences, so each thread of the lookup counts several; and a
launch whose few tiles over long contexts are split into key ranges and merged.  The
pool slots no row owns hold NaN; whole outputs are compared with the oracle.
"""
import numpy as np
import pytest

import oracle.pagedkv_oracle as O
from tests.gpu_util import DeviceBatch, out_f64, tolerance
from workloads import make_batch

pytestmark = pytest.mark.gpu


def _check(b, what):
    print(f"[case] {what}", flush=True)
    _, _, ref = O.step(b)
    got = out_f64(DeviceBatch(b).step())
    tol = tolerance(b, ref)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{what}: {len(bad)} elements off, first {bad[0]}, max {err.max():.3g}"


def test_equal_chunks_over_shared_blocks():
    rng = np.random.Generator(np.random.PCG64(71))
    ctx, n = 640, 32
    b = make_batch(rng, name="chunks64", dtype="bf16", num_q_heads=16, num_kv_heads=8,
                   head_dim=128, num_blocks=ctx // 16 + 4 * n + 8, context_lens=[ctx] * n,
                   query_lens=[64] * n, shared_prefix_blocks=ctx // 16 - 4, stale="nan")
    _check(b, "32 chunks of 64 rows, shared blocks")


@pytest.mark.parametrize("hq,hkv,d", [(16, 8, 128), (32, 8, 64)])
def test_chunk_lengths_between_decode_rows_and_empty_sequences(hq, hkv, d):
    rng = np.random.Generator(np.random.PCG64(72 + d))
    ql = [2, 0, 1, 31, 32, 33, 1, 63, 64, 0, 65, 1, 130, 3, 0]
    ctx = [q + int(rng.integers(0, 300)) for q in ql]
    nblk = sum((c + 15) // 16 for c in ctx)
    b = make_batch(rng, name="lengths", dtype="bf16", num_q_heads=hq, num_kv_heads=hkv,
                   head_dim=d, num_blocks=nblk + 16, context_lens=ctx, query_lens=ql,
                   stale="nan")
    _check(b, f"chunk lengths around the tile, hq={hq} hkv={hkv} d={d}")


def test_more_sequences_than_lookup_threads():
    rng = np.random.Generator(np.random.PCG64(73))
    n = 700
    ql = [1] * n
    for s, q in ((0, 40), (5, 70), (300, 2), (511, 64), (512, 129), (513, 33), (699, 65)):
        ql[s] = q
    ctx = [q + int(rng.integers(0, 60)) for q in ql]
    nblk = sum((c + 15) // 16 for c in ctx)
    b = make_batch(rng, name="many", dtype="bf16", num_q_heads=8, num_kv_heads=4,
                   head_dim=64, num_blocks=nblk + 16, context_lens=ctx, query_lens=ql,
                   stale="nan")
    _check(b, "700 sequences, 7 chunks among decode rows")


def test_split_tiles_of_several_chunks():
    rng = np.random.Generator(np.random.PCG64(74))
    ql = [20, 1, 64, 0, 5, 1]
    ctx = [3000, 2500, 4100, 100, 5000, 800]
    nblk = sum((c + 15) // 16 for c in ctx)
    b = make_batch(rng, name="splits", dtype="bf16", num_q_heads=16, num_kv_heads=8,
                   head_dim=128, num_blocks=nblk + 16, context_lens=ctx, query_lens=ql,
                   stale="nan")
    _check(b, "short chunks over long contexts, split and merged")

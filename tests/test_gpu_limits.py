"""GPU parity at the limits: item counts beyond one decode launch, broken lengths, and
chunking invariance.

The decode kernel scans its work items (sequences for bf16, query rows for fp32) in
LDS, at most 2,048 per launch; larger batches are cut into consecutive launches whose
items and partial slots must not interfere.  Both cases here exceed the limit and are
compared element by element with the fp64 oracle, through the plain and the fused
calls.
"""
import numpy as np
import pytest

import oracle.pagedkv_oracle as O
from tests.gpu_util import DeviceBatch, out_f64, to_raw, tolerance
from workloads import make_batch

pytestmark = pytest.mark.gpu


def _check(b, got, ref, what):
    tol = tolerance(b, ref)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert (err <= tol).all(), f"{what}: max err {err.max():.3g}"


def test_more_sequences_than_one_launch_holds_bf16():
    rng = np.random.Generator(np.random.PCG64(21))
    n = 2100
    ctx = [int(c) for c in rng.integers(1, 80, n, endpoint=True)]
    nb = sum((c + 15) // 16 for c in ctx) + 16
    print(f"[case] {n} bf16 decode sequences", flush=True)
    b = make_batch(rng, name="many_bf16", dtype="bf16", num_q_heads=8, num_kv_heads=2,
                   head_dim=64, num_blocks=nb, context_lens=ctx, query_lens=[1] * n,
                   stale="nan")
    kp, vp, ref = O.step(b)
    db = DeviceBatch(b)
    out = db.step()
    assert to_raw(db.k_pool).tobytes() == kp.tobytes(), "K pool after write"
    _check(b, out_f64(out), ref, "two calls")
    db2 = DeviceBatch(b)
    _check(b, out_f64(db2.step_fused()), ref, "fused call")


def test_more_rows_than_one_launch_holds_f32():
    rng = np.random.Generator(np.random.PCG64(22))
    print("[case] 2,101 fp32 query rows", flush=True)
    b = make_batch(rng, name="many_rows_f32", dtype="f32", num_q_heads=4, num_kv_heads=2,
                   head_dim=64, num_blocks=200, context_lens=[1600, 700, 50],
                   query_lens=[1500, 600, 1], stale="nan")
    kp, vp, ref = O.step(b)
    db = DeviceBatch(b)
    out = db.step()
    assert to_raw(db.v_pool).tobytes() == vp.tobytes(), "V pool after write"
    _check(b, out_f64(out), ref, "fp32 rows")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_broken_lengths_give_zero_rows(dtype, fused):
    """Sequences whose query count exceeds their context (a broken precondition; the
    host validator rejects them) produce zero rows, and the other rows of the batch
    are unaffected.  The batch is built valid, then two context lengths are lowered
    on the device: a decode row to 0 keys and a 70-row chunk to 50 keys."""
    import torch

    rng = np.random.Generator(np.random.PCG64(23))
    print(f"[case] broken lengths dtype={dtype} fused={fused}", flush=True)
    b = make_batch(rng, name="broken", dtype=dtype, num_q_heads=8, num_kv_heads=2,
                   head_dim=64, num_blocks=120, context_lens=[100, 40, 200, 230],
                   query_lens=[1, 1, 70, 30], stale="nan")
    kp, vp, ref = O.step(b)
    db = DeviceBatch(b)
    db.context_lens.copy_(torch.tensor([100, 0, 50, 230], dtype=torch.int32))
    out = db.step_fused() if fused else db.step()
    got = out_f64(out)
    qsl = b.query_start_loc
    broken = np.zeros(b.total_q, dtype=bool)
    broken[qsl[1]:qsl[2]] = True   # decode row with no keys
    broken[qsl[2]:qsl[3]] = True   # 70 rows over 50 keys
    assert (got[broken] == 0).all(), "rows of broken sequences must be zero"
    _check(b, got[~broken], ref[~broken], "valid rows")
    assert to_raw(db.k_pool).tobytes() == kp.tobytes(), "the slot write is unaffected"


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 16, 8, 128), ("bf16", 32, 8, 64),
                                            ("f32", 8, 2, 64)])
def test_chunk_and_decode_equal_rows_of_one_shot_prefill(dtype, hq, hkv, d):
    """Chunking invariance on the GPU: in one batch whose three sequences name the same
    blocks, the rows of a chunk [450, 700) over 700 keys equal rows 450..699 of a
    one-shot prefill of [0, 700), and a decode row at position 699 equals the last
    prefill row (same queries; only the first sequence writes the new K/V).  The three
    are computed by different tiles, splits and kernels, so they agree to the
    tolerance, and each matches the oracle."""
    import dataclasses

    rng = np.random.Generator(np.random.PCG64(24))
    print(f"[case] chunk invariance dtype={dtype} hq={hq} hkv={hkv} d={d}", flush=True)
    one = make_batch(rng, name="oneshot", dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                     head_dim=d, num_blocks=80, context_lens=[700], query_lens=[700],
                     stale="nan")
    a = 450
    rows = np.concatenate([np.arange(700), np.arange(a, 700), [699]])
    pad = lambda x: np.concatenate([x, np.zeros((len(rows) - 700,) + x.shape[1:], x.dtype)])  # noqa
    b = dataclasses.replace(
        one, name="chunk_invariance",
        block_tables=np.repeat(one.block_tables, 3, axis=0),
        context_lens=np.array([700, 700, 700], dtype=one.context_lens.dtype),
        query_start_loc=np.array([0, 700, 700 + 700 - a, len(rows)],
                                 dtype=one.query_start_loc.dtype),
        q=one.q[rows], k_new=pad(one.k_new), v_new=pad(one.v_new),
        slot_mapping=np.concatenate([one.slot_mapping,
                                     -np.ones(len(rows) - 700, one.slot_mapping.dtype)]))
    kp, vp, ref = O.step(b)
    got = out_f64(DeviceBatch(b).step())
    _check(b, got, ref, "against the oracle")
    tol = tolerance(b, ref[a:700])
    assert (np.abs(got[700:700 + 700 - a] - got[a:700]) <= tol).all(), "chunk rows"
    assert (np.abs(got[-1] - got[699]) <= tolerance(b, ref[699])).all(), "decode row"

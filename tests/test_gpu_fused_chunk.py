"""GPU parity for the fused call (paged_attention_varlen_with_write) on a batch of one
chunk sequence.  The chunk kernel then stores this step's new rows itself and reads
their keys and values from k_new / v_new, since the same launch is writing those pool
slots.  Cases: a chunk starting at position 0 (every key is new), one starting
mid-block, one starting on a block and key-step edge, a short chunk split over a long
context (split partials and merge), and the other head layouts (four and one query
heads per kv head, head_dim 64).  Before the call the pool slots of the new rows hold
NaN (a tile that read them back from the pool would come out NaN), and so does every
slot no row owns.  Checked: both pools bit-exact against the oracle's write, the output
against the oracle, and the same output bits as the two-call path (write, then plain
attention reading the pool)."""
import numpy as np
import pytest

import oracle.pagedkv_oracle as O
from tests.gpu_util import DeviceBatch, out_f64, to_raw, tolerance
from workloads import make_batch

pytestmark = pytest.mark.gpu

CASES = [
    # (q heads, kv heads, head_dim, context_len, query rows)
    (16, 8, 128, 300, 300),    # a fresh prompt: chunk at position 0
    (16, 8, 128, 1000, 257),   # chunk from position 743 (mid-block)
    (16, 8, 128, 1024, 512),   # chunk from position 512 (block and key-step edge)
    (16, 8, 128, 3000, 40),    # short chunk over a long context: split and merged
    (32, 8, 64, 700, 130),     # four query heads per kv head, head_dim 64
    (8, 8, 64, 200, 64),       # one query head per kv head
]


@pytest.mark.parametrize("hq,hkv,d,ctx,q", CASES)
def test_fused_chunk_reads_new_rows_from_k_new(hq, hkv, d, ctx, q):
    print(f"[case] fused chunk hq={hq} hkv={hkv} d={d} ctx={ctx} q={q}", flush=True)
    rng = np.random.Generator(np.random.PCG64(ctx * 7 + q))
    b = make_batch(rng, name="fused_chunk", dtype="bf16", num_q_heads=hq, num_kv_heads=hkv,
                   head_dim=d, num_blocks=(ctx + 15) // 16 + 24, context_lens=[ctx],
                   query_lens=[q], stale="nan")
    nan = np.uint16(0x7FC0)
    for slot in b.slot_mapping:
        b.k_pool[slot // 16, :, slot % 16, :] = nan
        b.v_pool[slot // 16, :, slot % 16, :] = nan
    kp_ref, vp_ref, ref = O.step(b)
    db = DeviceBatch(b)
    out = db.step_fused()
    assert to_raw(db.k_pool).tobytes() == kp_ref.tobytes(), "K pool after the fused call"
    assert to_raw(db.v_pool).tobytes() == vp_ref.tobytes(), "V pool after the fused call"
    got = out_f64(out)
    assert np.isfinite(got).all(), "non-finite output: a new row was read from the pool"
    tol = tolerance(b, ref)
    err = np.abs(got - ref)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{len(bad)} elements off, first {bad[0]}, max {err.max():.3g}"
    two = to_raw(DeviceBatch(b).step())
    assert two.tobytes() == to_raw(out).tobytes(), "fused and two-call outputs differ"

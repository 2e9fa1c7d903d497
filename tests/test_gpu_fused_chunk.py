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


def test_fused_chunk_graph_replays_follow_new_metadata():
    """A prefill loop captures one chunk step (the fused call on one sequence) and
    replays it with new values in the same buffers: the chunk at other positions of a
    prompt (from position 0, mid-block, at the largest context the host hint allows),
    new rows, slots and pool contents.  The launch stores the new rows and reads them
    from k_new / v_new inside the capture; every replay must equal the oracle, pools
    bit for bit, with the new rows' pool slots NaN before each replay."""
    import torch

    import paged_kv_cache_290_amd as pkv

    hq, hkv, d, q, max_ctx = 16, 8, 128, 200, 2000
    nb = (max_ctx + 15) // 16 + 24
    max_blocks = (max_ctx + 15) // 16

    def case(seed, ctx):
        rng = np.random.Generator(np.random.PCG64(seed))
        b = make_batch(rng, name=f"fused_replay{seed}", dtype="bf16", num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=d, num_blocks=nb, context_lens=[ctx],
                       query_lens=[q], max_blocks_per_seq=max_blocks, stale="nan")
        nan = np.uint16(0x7FC0)
        for slot in b.slot_mapping:
            b.k_pool[slot // 16, :, slot % 16, :] = nan
            b.v_pool[slot // 16, :, slot % 16, :] = nan
        return b

    print("[case] fused chunk graph over changing metadata", flush=True)
    b0 = case(300, 1000)
    db = DeviceBatch(b0)
    out = torch.empty_like(db.q)
    ws = torch.empty(pkv.workspace_size(1, q, hq, hkv, d, max_ctx, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def step():
        pkv.attention_with_write(db.q, db.k_new, db.v_new, db.k_pool, db.v_pool,
                                 db.slot_mapping, db.block_tables, db.context_lens,
                                 db.query_start_loc, scale=b0.scale, max_context_len=max_ctx,
                                 max_query_len=q, out=out, workspace=ws)

    step()  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)

    for seed, ctx in ((301, 200), (302, 743 + q), (303, max_ctx)):
        b = case(seed, ctx)
        src = DeviceBatch(b)
        for f in ("k_pool", "v_pool", "q", "k_new", "v_new", "block_tables", "context_lens",
                  "query_start_loc", "slot_mapping"):
            getattr(db, f).copy_(getattr(src, f))
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        kp_ref, vp_ref, ref = O.step(b)
        assert to_raw(db.k_pool).tobytes() == kp_ref.tobytes(), f"K pool, replay ctx={ctx}"
        assert to_raw(db.v_pool).tobytes() == vp_ref.tobytes(), f"V pool, replay ctx={ctx}"
        got = out_f64(out)
        assert np.isfinite(got).all(), f"replay ctx={ctx}: non-finite output"
        err = np.abs(got - ref)
        assert (err <= tolerance(b, ref)).all(), f"replay ctx={ctx}: max err {err.max():.3g}"

"""GPU parity at the edges of the decode plan's key-range rule.

A decode segment (row, kv-head group) is cut into key ranges, each a workgroup
leaving a partial result for a merge launch, when a wave would otherwise take more
than 16 blocks of the longest row, or when the segments leave at least half of the
256 compute units idle and the longest row gives each of a workgroup's 16 waves 4
blocks or more (then floor(256 / segments) ranges).  The batches below sit on both
sides of those edges; each output row is compared with the fp64 oracle, and the
pools bit for bit, through the two-call path and the fused call.
"""
import numpy as np
import pytest

import oracle.pagedkv_oracle as O
from tests.gpu_util import DeviceBatch, out_f64, to_raw, tolerance
from workloads import make_batch

pytestmark = pytest.mark.gpu

CASES = [
    # (rows, lowest and highest context, heads q/kv, head_dim): what the plan does
    (16, 1000, 1008, 16, 8, 128),   # 128 segments, longest row 63 blocks: no ranges
    (16, 1000, 1024, 16, 8, 128),   # 128 segments, 64 blocks: two ranges each
    (30, 512, 640, 16, 8, 128),     # 240 segments (chip nearly full): no ranges
    (17, 1900, 2048, 16, 8, 128),   # 136 segments: floor(256 / 136) = 1, no ranges
    (8, 1, 4096, 32, 8, 64),        # 64 segments of very unequal rows: four ranges
    (2, 5000, 8192, 8, 2, 64),      # 4 segments of long rows: 32 ranges each
]


@pytest.mark.parametrize("rows,lo,hi,hq,hkv,d", CASES)
@pytest.mark.parametrize("fused", [False, True])
def test_key_range_rule_edges_match_oracle(rows, lo, hi, hq, hkv, d, fused):
    print(f"[case] plan edge rows={rows} ctx={lo}-{hi} hq={hq} hkv={hkv} d={d} "
          f"fused={fused}", flush=True)
    rng = np.random.Generator(np.random.PCG64(rows * 10007 + hi))
    ctx = rng.integers(lo, hi, size=rows, endpoint=True)
    ctx[0] = hi  # the longest row sets the plan
    nb = int(sum((int(c) + 15) // 16 for c in ctx)) + 16
    b = make_batch(rng, name="plan_edges", dtype="bf16", num_q_heads=hq, num_kv_heads=hkv,
                   head_dim=d, num_blocks=nb, context_lens=ctx, query_lens=[1] * rows,
                   stale="nan")
    kp, vp, ref = O.step(b)
    db = DeviceBatch(b)
    out = db.step_fused() if fused else db.step()
    assert to_raw(db.k_pool).tobytes() == kp.tobytes()
    assert to_raw(db.v_pool).tobytes() == vp.tobytes()
    got = out_f64(out)
    assert np.isfinite(got).all(), "non-finite output"
    err = np.abs(got - ref)
    assert (err <= tolerance(b, ref)).all(), f"max err {err.max():.3g}"

"""GPU parity of bf16 decode rows at every position of the newest token inside its
16-token block (context lengths 16k + r, r = 1..16, including rows shorter than one
block), for the head layouts of the d=64 decode path (GQA groups 4, 2, 3 and 1), with
NaN in every pool slot no row owns, through both the fused call (the newest key and
value taken from k_new / v_new) and the two-call path, against the oracle."""
import numpy as np
import pytest

import oracle.pagedkv_oracle as O
from tests.gpu_util import DeviceBatch, out_f64, to_raw, tolerance
from workloads import make_batch

pytestmark = pytest.mark.gpu


def _assert_close(b, got, ref, what):
    tol = tolerance(b, ref)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{what}: {len(bad)} elements off, first {bad[0]}, max {err.max():.3g}"


@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 8), (12, 4), (8, 8)])
@pytest.mark.parametrize("neg_scale", [False, True])
def test_newest_token_at_every_block_position(hq, hkv, neg_scale):
    print(f"[case] decode positions hq={hq} hkv={hkv} neg_scale={neg_scale}", flush=True)
    rng = np.random.Generator(np.random.PCG64(1000 + hq * 10 + hkv + int(neg_scale)))
    ctx = [16 * int(k) + r for r in range(1, 17) for k in (0, rng.integers(1, 9))]
    nblk = sum((c + 15) // 16 for c in ctx)
    scale = -0.7 / np.sqrt(64) if neg_scale else None
    b = make_batch(rng, name="positions", dtype="bf16", num_q_heads=hq, num_kv_heads=hkv,
                   head_dim=64, num_blocks=nblk + 40, context_lens=ctx,
                   query_lens=[1] * len(ctx), stale="nan", scale=scale)
    kp, vp, ref = O.step(b)
    fused = DeviceBatch(b)
    out = fused.step_fused()
    assert to_raw(fused.k_pool).tobytes() == kp.tobytes(), "K pool after the fused call"
    assert to_raw(fused.v_pool).tobytes() == vp.tobytes(), "V pool after the fused call"
    _assert_close(b, out_f64(out), ref, "fused call")
    two = DeviceBatch(b)
    _assert_close(b, out_f64(two.step()), ref, "two calls")
